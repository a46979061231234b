"""Pins of the fp64 oracle against facts the pages and the mathematics fix.

Each test states what it pins.  None of them re-types the oracle's formula:
they use hand-derived values, the textbook Fenwick decomposition, the SSD
and linear-attention recurrences, a token-by-token Fenwick recurrence, or
per-bucket brute force in plain Python loops.
"""
import math
import os

import numpy as np
import pytest

from oracle import fenwick, loglin_ref, recurrent

RNG = np.random.default_rng


def rand_problem(T, H=2, G=1, P=3, N=4, L=None, seed=0, decay=0.3, Bt=1):
    rng = RNG(seed)
    L = L if L is not None else fenwick.max_level(T) + 1
    X = rng.standard_normal((Bt, T, H, P))
    B = rng.standard_normal((Bt, T, G, N))
    C = rng.standard_normal((Bt, T, G, N))
    log_a = -decay * rng.random((Bt, T, H))
    lam = rng.random((Bt, T, H, L)) + 0.2
    return X, B, C, log_a, lam


def rel_err(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ---------------------------------------------------------------- levels --

def read_level_table(path):
    rows = {}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        t, vals = line.split(":")
        rows[int(t)] = [int(v) for v in vals.split()]
    return rows


def test_level_table_T8_golden(golden_dir):
    """Hand-derived T = 8 level table (tree-partition section)."""
    table = read_level_table(os.path.join(golden_dir, "fenwick_levels_T8.txt"))
    assert sorted(table) == list(range(8))
    for t, row in table.items():
        got = fenwick.levels(t, np.arange(t + 1)).tolist()
        assert got == row, (t, got, row)


@pytest.mark.parametrize("T", [1, 2, 5, 64, 300, 1024])
def test_levels_equal_textbook_fenwick_buckets(T):
    """bit_length(t XOR s) equals the level of the Fenwick block holding s."""
    for t in range(T):
        seen = np.full(t + 1, -1)
        for lev, lo, hi in fenwick.fenwick_buckets(t):
            seen[lo:hi + 1] = lev
        assert (seen >= 0).all()
        np.testing.assert_array_equal(fenwick.levels(t, np.arange(t + 1)), seen)


@pytest.mark.parametrize("t", list(range(0, 130)) + [1023, 4095, 32767, 131071])
def test_bucket_invariants(t):
    """Buckets partition [0, t] into contiguous runs; level 0 is {t}; level
    l >= 1 holds 2**(l-1) positions iff bit l-1 of t is set; levels do not
    increase as s approaches t (most recent finest)."""
    bks = fenwick.fenwick_buckets(t)
    covered = sorted((lo, hi) for _, lo, hi in bks)
    pos = 0
    for lo, hi in covered:
        assert lo == pos and hi >= lo
        pos = hi + 1
    assert pos == t + 1
    sizes = {lev: hi - lo + 1 for lev, lo, hi in bks}
    assert sizes[0] == 1 and bks[0] == (0, t, t)
    for lev in range(1, t.bit_length() + 1):
        if (t >> (lev - 1)) & 1:
            assert sizes[lev] == 2 ** (lev - 1)
        else:
            assert lev not in sizes
    s = np.arange(t + 1)
    lv = fenwick.levels(t, s)
    assert (np.diff(lv) <= 0).all()


@pytest.mark.parametrize("k", range(1, 12))
def test_bucket_sizes_all_ones(k):
    """t = 2**k - 1 sees buckets of sizes 1, 1, 2, 4, ..., 2**(k-1)."""
    t = 2 ** k - 1
    sizes = [hi - lo + 1 for _, lo, hi in fenwick.fenwick_buckets(t)]
    assert sizes == [1, 1] + [2 ** i for i in range(1, k)]


@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 255, 256, 257, 2048, 32768, 131072])
def test_level_count(T):
    """Levels stay <= ceil(log2 T), so ceil(log2 T) + 1 weights suffice."""
    t = np.arange(T)
    top = int(fenwick.levels(t, 0).max())
    assert top == fenwick.max_level(T)
    assert top == (math.ceil(math.log2(T)) if T > 1 else 0)


# ---------------------------------------------------------- closed forms --

def read_worked(path):
    d = {}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, *vals = line.split()
        d[k] = [float(v) for v in vals]
    return d


def worked_inputs(d):
    T = len(d["X"])
    X = np.array(d["X"]).reshape(1, T, 1, 1)
    B = np.array(d["B"]).reshape(1, T, 1, 1)
    C = np.array(d["C"]).reshape(1, T, 1, 1)
    log_a = np.log(np.array(d["a"])).reshape(1, T, 1)
    L = fenwick.max_level(T) + 1
    lam = np.tile(d["lambda_base"][0] ** np.arange(L), (T, 1)).reshape(1, T, 1, L)
    return X, B, C, log_a, lam


def test_worked_example_T4(golden_dir):
    """Hand-worked T = 4 example: pins level placement, decay range and the
    C (query) / B (key) roles."""
    d = read_worked(os.path.join(golden_dir, "worked_T4.txt"))
    args = worked_inputs(d)
    y = loglin_ref.loglin_forward(*args)[0, :, 0, 0]
    np.testing.assert_allclose(y, d["y"], rtol=1e-12)


def test_closed_form_T1_T2():
    """T = 1: y0 = lam[0,0] (C0.B0) X0.  T = 2 adds
    y1 = lam[1,0] (C1.B1) X1 + lam[1,1] a1 (C1.B0) X0."""
    X, B, C, log_a, lam = rand_problem(2, H=1, G=1, P=3, N=5, seed=3)
    a = np.exp(log_a[0, :, 0])
    y = loglin_ref.loglin_forward(X, B, C, log_a, lam)[0, :, 0, :]
    c0b0 = C[0, 0, 0] @ B[0, 0, 0]
    c1b1 = C[0, 1, 0] @ B[0, 1, 0]
    c1b0 = C[0, 1, 0] @ B[0, 0, 0]
    y0 = lam[0, 0, 0, 0] * c0b0 * X[0, 0, 0]
    y1 = lam[0, 1, 0, 0] * c1b1 * X[0, 1, 0] + lam[0, 1, 0, 1] * a[1] * c1b0 * X[0, 0, 0]
    np.testing.assert_allclose(y[0], y0, rtol=1e-13)
    np.testing.assert_allclose(y[1], y1, rtol=1e-13)
    y_single = loglin_ref.loglin_forward(X[:, :1], B[:, :1], C[:, :1],
                                         log_a[:, :1], lam[:, :1, :, :1])
    np.testing.assert_allclose(y_single[0, 0, 0], y0, rtol=1e-13)


# ------------------------------------------------------------ reductions --

def ssd_recurrent(X, B, C, a, scale):
    """SSD / Mamba-2 scalar-decay recurrence: h_t = a_t h_{t-1} + B_t X_t^T,
    y_t = scale_t * h_t^T C_t (article on Transformers, RNNs and Mamba-2,
    sections on semiseparable matrices and state space duality)."""
    T, P = X.shape
    h = np.zeros((B.shape[1], P))
    y = np.zeros((T, P))
    for t in range(T):
        h = a[t] * h + np.outer(B[t], X[t])
        y[t] = scale[t] * (h.T @ C[t])
    return y


@pytest.mark.parametrize("T", [1, 7, 64, 100])
def test_reduces_to_ssd_when_lambda_constant(T):
    """All lambda equal (value c): O = c * SSD (write-up: equal weights give
    back the linear model)."""
    X, B, C, log_a, lam = rand_problem(T, H=2, G=1, P=3, N=4, seed=T)
    lam[:] = 1.7
    out = loglin_ref.loglin_forward(X, B, C, log_a, lam)
    for h in range(2):
        ref = ssd_recurrent(X[0, :, h], B[0, :, 0], C[0, :, 0],
                            np.exp(log_a[0, :, h]), np.full(T, 1.7))
        assert rel_err(out[0, :, h], ref) < 1e-12


def test_reduces_to_scaled_ssd_when_lambda_level_free():
    """lambda_t independent of the level: O = diag(lambda_t) SSD."""
    T = 77
    X, B, C, log_a, lam = rand_problem(T, H=1, G=1, P=2, N=3, seed=11)
    per_t = np.random.default_rng(1).random(T) + 0.5
    lam[:] = per_t[None, :, None, None]
    out = loglin_ref.loglin_forward(X, B, C, log_a, lam)
    ref = ssd_recurrent(X[0, :, 0], B[0, :, 0], C[0, :, 0],
                        np.exp(log_a[0, :, 0]), per_t)
    assert rel_err(out[0, :, 0], ref) < 1e-12


def test_reduces_to_causal_prefix_sum():
    """a = 1 and lambda = 1: y_t = C_t^T sum_{s<=t} B_s X_s^T, the causal 0/1
    mask of linear attention computed as a cumulative sum."""
    T = 90
    X, B, C, log_a, lam = rand_problem(T, H=1, G=1, P=4, N=3, seed=5)
    log_a[:] = 0.0
    lam[:] = 1.0
    out = loglin_ref.loglin_forward(X, B, C, log_a, lam)[0, :, 0]
    outer = np.einsum("tn,tp->tnp", B[0, :, 0], X[0, :, 0])
    state = np.cumsum(outer, axis=0)
    ref = np.einsum("tn,tnp->tp", C[0, :, 0], state)
    assert rel_err(out, ref) < 1e-12


# ------------------------------------------- recurrence and brute force --

@pytest.mark.parametrize("T,seed", [(1, 0), (2, 1), (3, 2), (7, 3), (8, 4),
                                    (33, 5), (64, 6), (64, 7)])
def test_dense_equals_fenwick_recurrence(T, seed):
    """Token-by-token Fenwick recurrence (decode form) equals the dense
    oracle, including heads sharing a B/C group."""
    X, B, C, log_a, lam = rand_problem(T, H=4, G=2, P=3, N=5, seed=seed)
    dense = loglin_ref.loglin_forward(X, B, C, log_a, lam, row_block=16)
    rec = recurrent.loglin_recurrent(X, B, C, log_a, lam)
    assert rel_err(dense, rec) < 1e-12


def brute_force_bucket(X, B, C, a, t, lo, hi):
    """Plain loops: sum over s in [lo, hi] of (C_t.B_s) prod_{r=s+1..t} a_r X_s."""
    P = X.shape[1]
    acc = np.zeros(P)
    for s in range(lo, hi + 1):
        d = 1.0
        for r in range(s + 1, t + 1):
            d *= a[r]
        acc += float(np.dot(C[t], B[s])) * d * X[s]
    return acc


@pytest.mark.parametrize("lev", range(0, 6))
def test_onehot_level_equals_bucket_brute_force(lev):
    """lambda one-hot on level l: output is attention restricted to the
    textbook Fenwick bucket of level l (superposition of per-level terms)."""
    T = 29
    X, B, C, log_a, lam = rand_problem(T, H=1, G=1, P=2, N=3, seed=lev)
    lam[:] = 0.0
    lam[..., lev] = 1.0
    out = loglin_ref.loglin_forward(X, B, C, log_a, lam)[0, :, 0]
    a = np.exp(log_a[0, :, 0])
    for t in range(T):
        ref = np.zeros(2)
        for bl, lo, hi in fenwick.fenwick_buckets(t):
            if bl == lev:
                ref = brute_force_bucket(X[0, :, 0], B[0, :, 0], C[0, :, 0], a, t, lo, hi)
        np.testing.assert_allclose(out[t], ref, rtol=1e-11, atol=1e-13)


def test_superposition_over_levels():
    """O(lambda) = sum_l O(lambda * e_l): the output is linear in lambda."""
    T = 50
    X, B, C, log_a, lam = rand_problem(T, H=2, G=2, P=2, N=3, seed=9)
    full = loglin_ref.loglin_forward(X, B, C, log_a, lam)
    acc = np.zeros_like(full)
    for lev in range(lam.shape[-1]):
        one = np.zeros_like(lam)
        one[..., lev] = lam[..., lev]
        acc += loglin_ref.loglin_forward(X, B, C, log_a, one)
    assert rel_err(acc, full) < 1e-12


def test_causality():
    """Changing inputs at positions > t leaves rows <= t unchanged."""
    T = 40
    X, B, C, log_a, lam = rand_problem(T, seed=2)
    base = loglin_ref.loglin_forward(X, B, C, log_a, lam)
    X2, B2, C2, la2 = X.copy(), B.copy(), C.copy(), log_a.copy()
    X2[:, 25:] += 1.0
    B2[:, 25:] -= 2.0
    C2[:, 25:] *= 3.0
    la2[:, 25:] -= 0.5
    pert = loglin_ref.loglin_forward(X2, B2, C2, la2, lam)
    np.testing.assert_array_equal(base[:, :25], pert[:, :25])


def test_rows_api_matches_full():
    T = 300
    X, B, C, log_a, lam = rand_problem(T, H=2, G=1, seed=4)
    full = loglin_ref.loglin_forward(X, B, C, log_a, lam)
    rows = np.array([0, 1, 63, 64, 128, 200, 299])
    part = loglin_ref.loglin_rows(X, B, C, log_a, lam, 0, 1, rows, row_block=3)
    np.testing.assert_allclose(part, full[0, rows, 1], rtol=1e-13, atol=1e-14)


def test_group_mapping_convention():
    """Parity unpinned (an interface convention): head h reads B/C group
    h // (H/G).  Expanding B/C per head gives the same result."""
    T = 20
    X, B, C, log_a, lam = rand_problem(T, H=6, G=3, seed=8)
    out = loglin_ref.loglin_forward(X, B, C, log_a, lam)
    idx = np.arange(6) // 2
    out2 = loglin_ref.loglin_forward(X, B[:, :, idx], C[:, :, idx], log_a, lam)
    np.testing.assert_allclose(out, out2, rtol=1e-14)


def test_rejects_short_lambda():
    X, B, C, log_a, lam = rand_problem(9, L=4)
    with pytest.raises(ValueError):
        loglin_ref.loglin_forward(X, B, C, log_a, lam)
