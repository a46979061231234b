"""Pins of the fp64 gradient oracle.

The gradient oracle is pinned to the forward oracle (itself pinned in
test_oracle_pins) by central finite differences of the scalar
<dO, O(X, B, C, log_a, lambda)> for every input element, so a mistake in
any gradient formula (a transposed product, a missing group sum, a decay
range off by one, the wrong level) shows as a mismatch.  Further pins:
dlambda at level l equals dO . O(lambda one-hot on l) (superposition over
levels, with no lambda in the formula being checked), dlog_a at r = 0 is
zero (log a_0 multiplies nothing), and planted mistakes in the gradient
oracle are each caught.
"""
import numpy as np
import pytest

from oracle import loglin_grad, loglin_ref

from .test_oracle_pins import rand_problem, rel_err

EPS = 1e-6


def loss(X, B, C, log_a, lam, dO):
    return float(np.sum(dO * loglin_ref.loglin_forward(X, B, C, log_a, lam)))


def finite_differences(args, dO, name):
    """Central differences of <dO, O> in every element of one input."""
    names = ("X", "B", "C", "log_a", "lam")
    idx = names.index(name)
    base = [np.array(a, dtype=np.float64, copy=True) for a in args]
    grad = np.zeros_like(base[idx])
    it = np.nditer(base[idx], flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        orig = base[idx][i]
        base[idx][i] = orig + EPS
        fp = loss(*base, dO)
        base[idx][i] = orig - EPS
        fm = loss(*base, dO)
        base[idx][i] = orig
        grad[i] = (fp - fm) / (2 * EPS)
    return grad


def fd_all(args, dO):
    return {"dX": finite_differences(args, dO, "X"),
            "dB": finite_differences(args, dO, "B"),
            "dC": finite_differences(args, dO, "C"),
            "dlog_a": finite_differences(args, dO, "log_a"),
            "dlam": finite_differences(args, dO, "lam")}


CASES = [  # (T, H, G, P, N, extra levels, Bt)
    (1, 1, 1, 2, 3, 0, 1),
    (2, 2, 1, 2, 2, 1, 1),
    (11, 2, 1, 3, 4, 1, 1),
    (16, 4, 2, 3, 2, 0, 1),
    (9, 2, 2, 2, 3, 2, 2),
]


@pytest.mark.parametrize("T,H,G,P,N,extra,Bt", CASES)
def test_gradients_match_finite_differences(T, H, G, P, N, extra, Bt):
    """Every gradient equals central differences of the pinned forward."""
    L = (max(T, 1) - 1).bit_length() + 1 + extra
    args = rand_problem(T, H=H, G=G, P=P, N=N, L=L, seed=T + 7 * H, Bt=Bt)
    dO = np.random.default_rng(99 + T).standard_normal(args[0].shape)
    got = loglin_grad.loglin_grad(*args, dO)
    want = fd_all(args, dO)
    for k, v in want.items():
        assert got[k].shape == v.shape, k
        assert rel_err(got[k], v) < 1e-7, (k, rel_err(got[k], v))


def test_dlambda_is_dO_dot_single_level_output():
    """dlambda[t, l] = dO_t . O_t computed with lambda one-hot on level l
    (the output is linear in lambda, level by level)."""
    X, B, C, log_a, lam = rand_problem(37, H=2, G=1, P=3, N=4, seed=5)
    dO = np.random.default_rng(1).standard_normal(X.shape)
    got = loglin_grad.loglin_grad(X, B, C, log_a, lam, dO)["dlam"]
    for lv in range(lam.shape[3]):
        onehot = np.zeros_like(lam)
        onehot[..., lv] = 1.0
        O = loglin_ref.loglin_forward(X, B, C, log_a, onehot)
        want = np.sum(dO * O, axis=3)
        assert rel_err(got[..., lv], want) < 1e-12 or np.max(np.abs(want)) == 0


def test_dlog_a_first_token_is_zero():
    """log a_0 enters no decay product (products run over r = s+1..t)."""
    X, B, C, log_a, lam = rand_problem(40, H=2, G=1, P=3, N=4, seed=8)
    dO = np.random.default_rng(2).standard_normal(X.shape)
    d = loglin_grad.loglin_grad(X, B, C, log_a, lam, dO)["dlog_a"]
    assert np.all(d[:, 0, :] == 0.0)
    assert np.max(np.abs(d[:, 1:, :])) > 0


def test_linear_in_upstream_gradient():
    X, B, C, log_a, lam = rand_problem(21, H=2, G=1, P=2, N=3, seed=3)
    rng = np.random.default_rng(4)
    d1, d2 = rng.standard_normal(X.shape), rng.standard_normal(X.shape)
    g1 = loglin_grad.loglin_grad(X, B, C, log_a, lam, d1)
    g2 = loglin_grad.loglin_grad(X, B, C, log_a, lam, d2)
    g = loglin_grad.loglin_grad(X, B, C, log_a, lam, d1 + 2 * d2)
    for k in g:
        assert rel_err(g[k], g1[k] + 2 * g2[k]) < 1e-12, k


def test_row_blocks_do_not_change_the_result():
    args = rand_problem(70, H=2, G=1, P=3, N=4, seed=6)
    dO = np.random.default_rng(5).standard_normal(args[0].shape)
    a = loglin_grad.loglin_grad(*args, dO, row_block=256)
    b = loglin_grad.loglin_grad(*args, dO, row_block=16)
    for k in a:
        assert rel_err(a[k], b[k]) < 1e-13, k


# ------------------------------------------------------- planted mistakes --

MUTANTS = {
    # dX through S^T instead of (S ⊙ M)^T: lambda and decay dropped
    "dX_no_mask": ("SM.T @ dOh[rows]", "(S * E).T @ dOh[rows]"),
    # dB summed with the wrong score (S instead of D)
    "dB_wrong_score": ("DM.T @ Cg[rows]", "SM.T @ Cg[rows]"),
    # dC with the key on the wrong side
    "dC_uses_C": ("DM @ Bg[:nc]", "DM @ Cg[:nc]"),
    # decay derivative over s <= r instead of s < r
    "dloga_inclusive": ("below[:, 1:] = pre[:, :-1]", "below[:, :] = pre"),
    # decay derivative over t > r instead of t >= r
    "dloga_strict_t": ("rows[:, None] >= r", "rows[:, None] > r"),
    # dlambda read one level off
    "dlam_shift": ("dlam[rows, lv] = np.sum(np.where(lev == lv, ESD",
                   "dlam[rows, lv] = np.sum(np.where(lev == lv + 1, ESD"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    """Each plausible slip in the gradient oracle fails the finite-difference pin."""
    import inspect
    import types
    src = inspect.getsource(loglin_grad)
    old, new = MUTANTS[name]
    assert src.count(old) == 1, name
    mod = types.ModuleType("oracle.loglin_grad_mutant")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), "<mutant>", "exec"), mod.__dict__)
    args = rand_problem(11, H=2, G=1, P=3, N=4, seed=17)
    dO = np.random.default_rng(3).standard_normal(args[0].shape)
    got = mod.loglin_grad(*args, dO)
    want = fd_all(args, dO)
    worst = max(rel_err(got[k], want[k]) for k in want)
    assert worst > 1e-3, (name, worst)


def test_sampled_entries_match_full_gradients():
    """The O(T)-per-entry helpers used at full size agree with the pinned
    full gradient oracle (every key column, query row and dlog_a entry)."""
    X, B, C, log_a, lam = rand_problem(45, H=4, G=2, P=3, N=4, seed=11)
    dO = np.random.default_rng(7).standard_normal(X.shape)
    for h in range(4):
        full = loglin_grad.loglin_grad_bh(X, B, C, log_a, lam, dO, 0, h)
        idx = np.arange(45)
        dX, dB = loglin_grad.grad_key_columns(X, B, C, log_a, lam, dO, 0, h, idx)
        dC, dlam = loglin_grad.grad_query_rows(X, B, C, log_a, lam, dO, 0, h, idx)
        assert rel_err(dX, full["dX"]) < 1e-12
        assert rel_err(dB, full["dB_h"]) < 1e-12
        assert rel_err(dC, full["dC_h"]) < 1e-12
        assert rel_err(dlam, full["dlam"]) < 1e-12
        dla = np.array([loglin_grad.grad_log_a_at(X, B, C, log_a, lam, dO, 0, h, r)
                        for r in range(45)])
        assert rel_err(dla, full["dlog_a"]) < 1e-12
