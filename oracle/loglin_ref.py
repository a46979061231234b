"""Plain fp64 CPU oracle of the log-linear Mamba-2 forward.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``.  The product path never imports,
calls or links anything here, and nothing here imports the product package.

What it computes is the plain definition, with no blocking beyond row blocks
and no reordering of the arithmetic:

    O = (C B^T  ⊙  M^H) X
    M^H[t, s] = (prod_{r=s+1..t} a_r) * lambda[t, level(t, s)]   for s <= t
              = 0                                                for s >  t

Sources:
  * log-linear attention write-up (yoousoft.com/industry/3746):
    - section "structured matrices unify attention variants" (结构矩阵，
      一统注意力变体): the masked form O = (A ⊙ M) V with a lower-triangular
      causal mask M and A = Q K^T for linear attention;
    - section "special structure: tree partition" (特殊结构：树划分): the
      matrix form with M^H filled by the Fenwick level of s relative to t, and
      per-level data-dependent scalar weights lambda;
    - section "log-linear generalisation of Mamba-2 and gated DeltaNet"
      (对Mamba-2和门控的对数线性推广): keep Mamba-2's transition and compose its
      mask with M^H.
  * Transformers / RNNs / Mamba-2 article (biyoush.com/article/202409/463109),
    section "state space duality" (狀態空間對偶性): with scalar A_t = a_t I the
    SSM is masked attention with C as the query, B as the key, u (here X) as
    the value and the mask entries given by products of a_r.

Readings where the pages are silent (formulas were lost in extraction):
  * decay covers a_{s+1} .. a_t (a_s excluded, a_t included), as in the SSD
    recurrence h_t = a_t h_{t-1} + B_t x_t^T;
  * lambda is indexed by the query position: lambda[b, t, h, level];
  * heads share B/C in consecutive groups: group(h) = h // (H / G);
  * no skip term, no dt scaling of X, no gate: exactly the formula above.

Arrays use the token-major layout of the library: X [Bt,T,H,P], B and C
[Bt,T,G,N], log_a [Bt,T,H], lam [Bt,T,H,L]; the result is [Bt,T,H,P] fp64.
"""
from __future__ import annotations

import numpy as np

from . import fenwick

F64 = np.float64


# -- the ingredients of the product, kept as separate functions so a test
#    can plant a mistake in one of them and check that a pin catches it ---

def _levels(t: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Fenwick level of s relative to t (tree-partition section)."""
    return fenwick.levels(t, s)


def _log_decay(cum: np.ndarray, t: np.ndarray, s: np.ndarray) -> np.ndarray:
    """log prod_{r=s+1..t} a_r from the inclusive prefix sum of log a."""
    return cum[t] - cum[s]


def _level_weight(lam_rows: np.ndarray, lev: np.ndarray) -> np.ndarray:
    """lambda of the query row at each entry's level: lam_rows [R, L] is
    indexed by the query position t, lev [R, S]."""
    return np.take_along_axis(lam_rows, lev, axis=1)


def _interaction(C_bg: np.ndarray, B_bg: np.ndarray, rows: np.ndarray,
                 ncols: int) -> np.ndarray:
    """Interaction block C_t . B_s for the given query rows and key columns
    [0, ncols): C plays the query, B the key (state space duality)."""
    Cq = np.asarray(C_bg[rows], dtype=F64)
    Bk = np.asarray(B_bg[:ncols], dtype=F64)
    return Cq @ Bk.T


def _group_of(h: int, nheads: int, ngroups: int) -> int:
    return h // (nheads // ngroups)


def _check(X, B, C, log_a, lam):
    Bt, T, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    if B.shape != (Bt, T, G, N) or C.shape != (Bt, T, G, N):
        raise ValueError("B/C shape mismatch")
    if log_a.shape != (Bt, T, H):
        raise ValueError("log_a shape mismatch")
    if lam.shape[:3] != (Bt, T, H):
        raise ValueError("lambda shape mismatch")
    if H % G:
        raise ValueError("nheads must be a multiple of ngroups")
    if lam.shape[3] < fenwick.max_level(T) + 1:
        raise ValueError("lambda has fewer levels than ceil(log2 T) + 1")
    return Bt, T, H, G, P, N


def mask_rows(log_a_bh: np.ndarray, lam_bh: np.ndarray, rows: np.ndarray,
              ncols: int) -> np.ndarray:
    """Rows of M^H for one (batch, head): shape [len(rows), ncols], fp64.

    ``log_a_bh`` is [T], ``lam_bh`` is [T, L].  Entries with s > t are zero;
    the exponent is masked before exp so no overflow can occur.
    """
    cum = np.cumsum(np.asarray(log_a_bh, dtype=F64))
    t = np.asarray(rows, dtype=np.int64)[:, None]
    s = np.arange(ncols, dtype=np.int64)[None, :]
    causal = s <= t
    lev = np.where(causal, _levels(t, s), 0)
    logd = np.where(causal, _log_decay(cum, t, np.minimum(s, t)), -np.inf)
    lam_rows = np.asarray(lam_bh, dtype=F64)[t[:, 0]]  # [R, L]
    weight = _level_weight(lam_rows, lev)
    return np.where(causal, np.exp(logd) * weight, 0.0)


def _rows_one_head(X, B, C, log_a, lam, b, h, rows):
    Bt, T, H, G, P, N = _check(X, B, C, log_a, lam)
    g = _group_of(h, H, G)
    rows = np.asarray(rows, dtype=np.int64)
    ncols = int(rows.max()) + 1
    M = mask_rows(log_a[b, :, h], lam[b, :, h, :], rows, ncols)
    A = _interaction(C[b, :, g, :], B[b, :, g, :], rows, ncols)  # [R, S]
    Xv = np.asarray(X[b, :ncols, h, :], dtype=F64)  # values [S, P]
    return (A * M) @ Xv  # [R, P]


def loglin_forward(X, B, C, log_a, lam, *, row_block: int = 256):
    """Full output O [Bt,T,H,P] in fp64, one (batch, head) at a time."""
    Bt, T, H, G, P, N = _check(X, B, C, log_a, lam)
    out = np.zeros((Bt, T, H, P), dtype=F64)
    for b in range(Bt):
        for h in range(H):
            out[b, :, h, :] = loglin_forward_bh(X, B, C, log_a, lam, b, h,
                                                row_block=row_block)
    return out


def loglin_forward_bh(X, B, C, log_a, lam, b, h, *, row_block: int = 256):
    """All rows of one (batch, head) slice, [T, P] fp64."""
    T = X.shape[1]
    res = np.empty((T, X.shape[3]), dtype=F64)
    for t0 in range(0, T, row_block):
        rows = np.arange(t0, min(T, t0 + row_block))
        res[rows] = _rows_one_head(X, B, C, log_a, lam, b, h, rows)
    return res


def loglin_rows(X, B, C, log_a, lam, b, h, rows, *, row_block: int = 64):
    """Selected output rows O[b, rows, h, :] in fp64, each from its full
    causal prefix.  Used where T is too long to form every row."""
    rows = np.asarray(rows, dtype=np.int64)
    res = np.empty((rows.size, X.shape[3]), dtype=F64)
    for i in range(0, rows.size, row_block):
        res[i:i + row_block] = _rows_one_head(X, B, C, log_a, lam, b, h,
                                              rows[i:i + row_block])
    return res
