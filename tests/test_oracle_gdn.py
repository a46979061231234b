"""Pins of the fp64 log-linear gated DeltaNet oracle (matrix form).

Each pin is an independent computation: the textbook single-state gated
DeltaNet recurrence (lambda = 1 on every level), the one-state-per-level
Fenwick recurrence, the log-linear Mamba-2 oracle (itself pinned) when the
keys are orthonormal so that the delta-rule corrections between tokens
vanish, and hand-derived closed forms for T = 1, 2.  Planted mistakes in
the oracle are each caught.
"""
import inspect
import types

import numpy as np
import pytest

from oracle import fenwick, gdn_ref, loglin_ref

from .test_oracle_pins import rel_err


def gdn_problem(T, H=2, N=4, P=3, L=None, seed=0, Bt=1, decay=0.3):
    rng = np.random.default_rng(seed)
    L = L if L is not None else fenwick.max_level(T) + 1
    q = rng.standard_normal((Bt, T, H, N))
    k = rng.standard_normal((Bt, T, H, N))
    k /= np.linalg.norm(k, axis=3, keepdims=True)  # unit keys, as gated DeltaNet uses
    v = rng.standard_normal((Bt, T, H, P))
    log_alpha = -decay * rng.random((Bt, T, H))
    beta = rng.random((Bt, T, H))
    lam = rng.random((Bt, T, H, L)) + 0.2
    return q, k, v, log_alpha, beta, lam


@pytest.mark.parametrize("T,seed", [(1, 0), (2, 1), (7, 2), (16, 3), (37, 4)])
def test_lambda_one_is_gated_deltanet(T, seed):
    q, k, v, la, be, lam = gdn_problem(T, seed=seed)
    got = gdn_ref.gdn_forward(q, k, v, la, be, np.ones_like(lam))
    want = gdn_ref.gdn_recurrent_single(q, k, v, la, be)
    assert rel_err(got, want) < 1e-12


@pytest.mark.parametrize("T,seed", [(1, 5), (2, 6), (5, 7), (8, 8), (33, 9), (64, 10)])
def test_matrix_form_equals_level_recurrence(T, seed):
    args = gdn_problem(T, seed=seed, L=fenwick.max_level(T) + 2, Bt=2)
    assert rel_err(gdn_ref.gdn_forward(*args), gdn_ref.gdn_recurrent_levels(*args)) < 1e-12


def test_orthonormal_keys_reduce_to_loglinear_mamba2():
    """With k_t = e_t (T <= N) every H_r leaves k_s (s != r) unchanged, so
    G[t, s] = beta_s prod alpha q_t . k_s: log-linear Mamba-2 with C = q,
    B = beta k, X = v (one B/C group per head)."""
    T, N = 12, 12
    q, k, v, la, be, lam = gdn_problem(T, N=N, seed=11)
    k = np.zeros_like(k)
    for t in range(T):
        k[:, t, :, t] = 1.0
    got = gdn_ref.gdn_forward(q, k, v, la, be, lam)
    want = loglin_ref.loglin_forward(v, be[..., None] * k, q, la, lam)
    assert rel_err(got, want) < 1e-12


def test_closed_forms_T1_T2():
    q, k, v, la, be, lam = gdn_problem(2, H=1, seed=12)
    o = gdn_ref.gdn_forward(q, k, v, la, be, lam)[0, :, 0]
    q0, q1, k0, k1 = q[0, 0, 0], q[0, 1, 0], k[0, 0, 0], k[0, 1, 0]
    b0, b1 = be[0, 0, 0], be[0, 1, 0]
    a1 = np.exp(la[0, 1, 0])
    o0 = lam[0, 0, 0, 0] * b0 * (q0 @ k0) * v[0, 0, 0]
    h1k0 = k0 - b1 * k1 * (k1 @ k0)  # H_1 k_0
    o1 = lam[0, 1, 0, 0] * b1 * (q1 @ k1) * v[0, 1, 0] + lam[0, 1, 0, 1] * b0 * a1 * (q1 @ h1k0) * v[0, 0, 0]
    assert rel_err(o[0], o0) < 1e-13
    assert rel_err(o[1], o1) < 1e-13


MUTANTS = {
    # decay including alpha_s
    "decay_includes_s": ("np.exp(cum[t] - cum[s])", "np.exp(cum[t] - cum[s] + np.log(np.exp(cum[s] - (cum[s - 1] if s else 0))))"),
    # the H of the key position itself applied
    "h_before_use": ("            G[t, s] = bt[s] * np.exp(cum[t] - cum[s]) * (g @ kh[s])\n            g = g - bt[s] * kh[s] * (kh[s] @ g)",
                     "            g = g - bt[s] * kh[s] * (kh[s] @ g)\n            G[t, s] = bt[s] * np.exp(cum[t] - cum[s]) * (g @ kh[s])"),
    # beta of the query instead of the key
    "beta_of_query": ("G[t, s] = bt[s] *", "G[t, s] = bt[t] *"),
    # lambda read one level off
    "lambda_level_shift": ("np.take_along_axis(lamh, lev, axis=1)", "np.take_along_axis(lamh, np.minimum(lev + 1, lamh.shape[1] - 1), axis=1)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    src = inspect.getsource(gdn_ref)
    old, new = MUTANTS[name]
    assert src.count(old) == 1, name
    mod = types.ModuleType("oracle.gdn_ref_mutant")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), "<mutant>", "exec"), mod.__dict__)
    args = gdn_problem(13, seed=21)
    worst = max(rel_err(mod.gdn_forward(*args), gdn_ref.gdn_recurrent_levels(*args)),
                rel_err(mod.gdn_forward(args[0], args[1], args[2], args[3], args[4], np.ones_like(args[5])),
                        gdn_ref.gdn_recurrent_single(*args[:5])))
    assert worst > 1e-6, (name, worst)
