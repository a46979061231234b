"""Plain fp64 CPU oracle of the gradients of the log-linear Mamba-2 forward.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``.  The product path never imports,
calls or links anything here, and nothing here imports the product package.

The forward is O = (S ⊙ M) X per (batch, head) with S[t, s] = C_t . B_s and
M[t, s] = E[t, s] * lambda[t, level(t, s)] for s <= t (zero above the
diagonal), E[t, s] = prod_{r=s+1..t} a_r.  For an upstream gradient dO the
gradients are written out from that definition, entry by entry of the
T x T matrices (in row blocks), with D[t, s] = dO_t . X_s:

    dX_s        = sum_t (S ⊙ M)[t, s] dO_t             ((S ⊙ M)^T dO)
    dB_s        = sum_t (D ⊙ M)[t, s] C_t  (summed over the heads of a group)
    dC_t        = sum_s (D ⊙ M)[t, s] B_s  (summed over the heads of a group)
    dlambda[t,l] = sum over s with level(t, s) = l of E S D [t, s]
    dlog_a_r    = sum over t >= r and s < r of (M ⊙ S ⊙ D)[t, s]

The last line is the derivative of E[t, s] = exp(sum_{r=s+1..t} log a_r):
log a_r enters exactly the entries with s < r <= t.  It is evaluated as that
double sum (prefix sums over s, then a masked sum over t), not through the
row-sum / column-sum identity the kernels use, so the two stay independent.

Sources: log-linear attention write-up (yoousoft.com/industry/3746),
sections "special structure: tree partition" (the masked form with M^H) and
"log-linear generalisation of Mamba-2 and gated DeltaNet" (Mamba-2's
transition composed with M^H); the write-up names the backward pass as the
harder half of a training kernel (section on the efficient training
algorithm and its benchmarks) but prints no formula for it, so the
gradients here are the plain calculus of the forward definition.

Pins (tests/test_oracle_grad.py): central finite differences of the pinned
forward oracle for every input; dlambda[t, l] equals dO_t . O_t of the
forward with lambda one-hot on level l; dlog_a at r = 0 is exactly zero;
gradients are linear in dO; planted mistakes are caught.  The O(T) sampled
helpers at the end are checked entry by entry against loglin_grad.
"""
from __future__ import annotations

import numpy as np

from . import fenwick
from .loglin_ref import _check, _group_of

F64 = np.float64


def _decay_rows(cum: np.ndarray, rows: np.ndarray, ncols: int):
    """E[t, s] for the given query rows and key columns [0, ncols); zero for
    s > t.  Also returns the level matrix and the causal mask."""
    t = np.asarray(rows, dtype=np.int64)[:, None]
    s = np.arange(ncols, dtype=np.int64)[None, :]
    causal = s <= t
    logd = np.where(causal, cum[t] - cum[np.minimum(s, t)], -np.inf)
    lev = np.where(causal, fenwick.levels(t, s), 0)
    return np.where(causal, np.exp(logd), 0.0), lev, causal


def loglin_grad_bh(X, B, C, log_a, lam, dO, b, h, *, row_block: int = 256):
    """Gradients of one (batch, head) slice, fp64.

    Returns a dict: dX [T,P], dB_h and dC_h [T,N] (this head's share of its
    group's dB and dC), dlam [T,L], dlog_a [T].
    """
    Bt, T, H, G, P, N = _check(X, B, C, log_a, lam)
    L = lam.shape[3]
    g = _group_of(h, H, G)
    cum = np.cumsum(np.asarray(log_a[b, :, h], dtype=F64))
    Xh = np.asarray(X[b, :, h, :], dtype=F64)
    Bg = np.asarray(B[b, :, g, :], dtype=F64)
    Cg = np.asarray(C[b, :, g, :], dtype=F64)
    dOh = np.asarray(dO[b, :, h, :], dtype=F64)
    lamh = np.asarray(lam[b, :, h, :], dtype=F64)

    dX = np.zeros((T, P), F64)
    dB = np.zeros((T, N), F64)
    dC = np.zeros((T, N), F64)
    dlam = np.zeros((T, L), F64)
    dla = np.zeros(T, F64)
    for t0 in range(0, T, row_block):
        rows = np.arange(t0, min(T, t0 + row_block))
        nc = int(rows[-1]) + 1
        E, lev, causal = _decay_rows(cum, rows, nc)
        M = E * np.take_along_axis(lamh[rows], lev, axis=1)  # lambda of the query row
        S = Cg[rows] @ Bg[:nc].T  # C_t . B_s
        D = dOh[rows] @ Xh[:nc].T  # dO_t . X_s
        SM = S * M
        DM = D * M
        dX[:nc] += SM.T @ dOh[rows]
        dB[:nc] += DM.T @ Cg[rows]
        dC[rows] = DM @ Bg[:nc]
        ESD = np.where(causal, E * S * D, 0.0)
        for lv in range(L):
            dlam[rows, lv] = np.sum(np.where(lev == lv, ESD, 0.0), axis=1)
        # dlog_a_r += sum_{t in rows, t >= r} sum_{s < r} G[t, s]
        Gm = np.where(causal, SM * D, 0.0)
        pre = np.cumsum(Gm, axis=1)  # pre[t, m] = sum_{s <= m} G[t, s]
        below = np.zeros_like(pre)
        below[:, 1:] = pre[:, :-1]  # below[t, r] = sum_{s < r} G[t, s]
        r = np.arange(nc)[None, :]
        dla[:nc] += np.sum(np.where(rows[:, None] >= r, below, 0.0), axis=0)
    return dict(dX=dX, dB_h=dB, dC_h=dC, dlam=dlam, dlog_a=dla)


def loglin_grad(X, B, C, log_a, lam, dO, *, row_block: int = 256):
    """All gradients in fp64: dX [Bt,T,H,P], dB and dC [Bt,T,G,N] (heads of
    a group summed in head order), dlam [Bt,T,H,L], dlog_a [Bt,T,H]."""
    Bt, T, H, G, P, N = _check(X, B, C, log_a, lam)
    if dO.shape != X.shape:
        raise ValueError("dO shape mismatch")
    L = lam.shape[3]
    out = dict(dX=np.zeros((Bt, T, H, P), F64), dB=np.zeros((Bt, T, G, N), F64),
               dC=np.zeros((Bt, T, G, N), F64), dlam=np.zeros((Bt, T, H, L), F64),
               dlog_a=np.zeros((Bt, T, H), F64))
    for b in range(Bt):
        for h in range(H):
            r = loglin_grad_bh(X, B, C, log_a, lam, dO, b, h, row_block=row_block)
            g = _group_of(h, H, G)
            out["dX"][b, :, h] = r["dX"]
            out["dB"][b, :, g] += r["dB_h"]
            out["dC"][b, :, g] += r["dC_h"]
            out["dlam"][b, :, h] = r["dlam"]
            out["dlog_a"][b, :, h] = r["dlog_a"]
    return out


# --------------------------------------------------- sampled entries, O(T) each
#
# For sequences too long to form every row, single gradient entries follow
# from one row or one column of the T x T matrices.  Same definitions as
# above; tests pin these against loglin_grad on small sizes.

def _bh_arrays(X, B, C, log_a, lam, dO, b, h):
    Bt, T, H, G, P, N = _check(X, B, C, log_a, lam)
    g = _group_of(h, H, G)
    return (np.cumsum(np.asarray(log_a[b, :, h], dtype=F64)),
            np.asarray(X[b, :, h, :], dtype=F64), np.asarray(B[b, :, g, :], dtype=F64),
            np.asarray(C[b, :, g, :], dtype=F64), np.asarray(dO[b, :, h, :], dtype=F64),
            np.asarray(lam[b, :, h, :], dtype=F64))


def grad_key_columns(X, B, C, log_a, lam, dO, b, h, cols):
    """dX[s] and this head's share of dB[s] for the key positions `cols`:
    column s of S ⊙ M and of D ⊙ M over the queries t >= s."""
    cum, Xh, Bg, Cg, dOh, lamh = _bh_arrays(X, B, C, log_a, lam, dO, b, h)
    T = cum.shape[0]
    dX = np.zeros((len(cols), Xh.shape[1]), F64)
    dB = np.zeros((len(cols), Bg.shape[1]), F64)
    for i, s in enumerate(np.asarray(cols, dtype=np.int64)):
        t = np.arange(s, T, dtype=np.int64)
        lev = fenwick.levels(t, np.full_like(t, s))
        m = np.exp(cum[t] - cum[s]) * lamh[t, lev]  # M[t, s]
        S = Cg[t] @ Bg[s]
        D = dOh[t] @ Xh[s]
        dX[i] = (m * S) @ dOh[t]
        dB[i] = (m * D) @ Cg[t]
    return dX, dB


def grad_query_rows(X, B, C, log_a, lam, dO, b, h, rows):
    """This head's share of dC[t] and dlambda[t, :] for the query positions
    `rows`: row t of D ⊙ M and of E ⊙ S ⊙ D over the keys s <= t."""
    cum, Xh, Bg, Cg, dOh, lamh = _bh_arrays(X, B, C, log_a, lam, dO, b, h)
    L = lamh.shape[1]
    dC = np.zeros((len(rows), Bg.shape[1]), F64)
    dlam = np.zeros((len(rows), L), F64)
    for i, t in enumerate(np.asarray(rows, dtype=np.int64)):
        s = np.arange(0, t + 1, dtype=np.int64)
        lev = fenwick.levels(np.full_like(s, t), s)
        e = np.exp(cum[t] - cum[s])
        S = Bg[s] @ Cg[t]
        D = Xh[s] @ dOh[t]
        dC[i] = (e * lamh[t, lev] * D) @ Bg[s]
        dlam[i] = np.bincount(lev, weights=e * S * D, minlength=L)[:L]
    return dC, dlam


def grad_log_a_at(X, B, C, log_a, lam, dO, b, h, r):
    """dlog_a[r] = sum over t >= r, s < r of (M ⊙ S ⊙ D)[t, s]; costs
    (T - r) * r entries, so it is meant for r near either end."""
    cum, Xh, Bg, Cg, dOh, lamh = _bh_arrays(X, B, C, log_a, lam, dO, b, h)
    T = cum.shape[0]
    if r == 0:
        return 0.0
    t = np.arange(r, T, dtype=np.int64)[:, None]
    s = np.arange(0, r, dtype=np.int64)[None, :]
    lev = fenwick.levels(t, s)
    m = np.exp(cum[t] - cum[s]) * np.take_along_axis(lamh[t[:, 0]], lev, axis=1)
    S = Cg[t[:, 0]] @ Bg[:r].T
    D = dOh[t[:, 0]] @ Xh[:r].T
    return float(np.sum(m * S * D))
