"""Token-by-token Fenwick recurrence of log-linear Mamba-2 (fp64, CPU).

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` to pin the dense oracle in
``loglin_ref``; it is also the plain definition a one-token decode step
would be checked against.  The product path never imports it.

Source: log-linear attention write-up (yoousoft.com/industry/3746), section
"log-linear attention" (对数线性注意力) and "special structure: tree
partition" (特殊结构：树划分): decoding keeps O(log T) states, one per Fenwick
bucket, each summarising the segment that ends at a position, and the output
weights the bucket memories by per-level scalars.  The page's equations were
lost, so the recurrence below is derived from the bucket structure.

State S[l] (N x P) holds sum over the bucket of level l of
decay(s -> t) * B_s X_s^T.  Going from t-1 to t with z = number of trailing
zeros of t:
  * the buckets of levels 0..z at t-1 together form exactly level z+1 at t
    (that level is empty at t-1), and levels 1..z become empty;
  * every older bucket keeps its members and is decayed by a_t;
  * level 0 becomes {t} with weight 1.
Output y_t = sum_l lambda[t, l] * S[l]^T C_t.

No bit length, no prefix sums and no exp of differences: this uses a_t
directly, so it is independent of the dense oracle's arithmetic.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def _ctz(t: int) -> int:
    z = 0
    while t and not (t >> z) & 1:
        z += 1
    return z


def loglin_recurrent_bh(X_bh, B_bh, C_bh, a_bh, lam_bh):
    """One (batch, head) slice.  X_bh [T,P], B_bh/C_bh [T,N], a_bh [T] (the
    decay a_t itself, not its log), lam_bh [T,L].  Returns [T,P] fp64."""
    X = np.asarray(X_bh, F64)
    Bm = np.asarray(B_bh, F64)
    Cm = np.asarray(C_bh, F64)
    a = np.asarray(a_bh, F64)
    lam = np.asarray(lam_bh, F64)
    T, P = X.shape
    N = Bm.shape[1]
    L = lam.shape[1]
    S = np.zeros((L + 1, N, P), dtype=F64)
    y = np.zeros((T, P), dtype=F64)
    for t in range(T):
        if t > 0:
            z = _ctz(t)
            if np.any(S[z + 1] != 0):
                raise AssertionError("Fenwick invariant broken: level not empty")
            S[z + 1] = S[: z + 1].sum(axis=0)
            S[: z + 1] = 0.0
            S[1:] *= a[t]
        S[0] = np.outer(Bm[t], X[t])
        for lev in range(L):
            if lam[t, lev] != 0.0:
                y[t] += lam[t, lev] * (S[lev].T @ Cm[t])
        if np.any(S[L] != 0):
            raise AssertionError("more levels occupied than lambda provides")
    return y


def loglin_recurrent(X, B, C, log_a, lam):
    """Whole batch via the recurrence; same layout as ``loglin_ref``."""
    Bt, T, H, P = X.shape
    G = B.shape[2]
    out = np.zeros((Bt, T, H, P), dtype=F64)
    a = np.exp(np.asarray(log_a, dtype=F64))
    for b in range(Bt):
        for h in range(H):
            g = h // (H // G)
            out[b, :, h, :] = loglin_recurrent_bh(
                X[b, :, h, :], B[b, :, g, :], C[b, :, g, :], a[b, :, h],
                lam[b, :, h, :])
    return out
