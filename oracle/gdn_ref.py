"""Plain fp64 CPU oracle of the log-linear Gated DeltaNet forward.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``.  The product path never imports,
calls or links anything here, and nothing here imports the product package.

Source: log-linear attention write-up (yoousoft.com/industry/3746), section
"log-linear generalisation of Mamba-2 and gated DeltaNet": the two models
differ in how the transition A is parameterised; each keeps its own A and
its attention mask is composed with the log-linear (Fenwick, per-level
lambda) mask M^H.  The page prints no formula beyond that.  Reading (the
plainest one the rest of the page supports): gated DeltaNet's transition
A_t = alpha_t (I - beta_t k_t k_t^T) acts on every Fenwick level state, the
new token enters level 0 as beta_t k_t v_t^T, and the output weights the
level states by lambda[t, level]:

    S_t^(l) as in the Fenwick recurrence of the Mamba-2 case, with A_t in
    place of the scalar a_t;   o_t = sum_l lambda[t, l] S_t^(l)^T q_t.

Because every level state sees the same transitions, this equals the gated
DeltaNet attention matrix with each entry reweighted by its level:

    O = (G ⊙ M^H) V,
    G[t, s] = beta_s (gamma_t / gamma_s) q_t^T H_t H_{t-1} ... H_{s+1} k_s,
    H_r = I - beta_r k_r k_r^T,  gamma_t / gamma_s = prod_{r=s+1..t} alpha_r,
    M^H[t, s] = lambda[t, level(t, s)]  (s <= t).

``gdn_forward`` evaluates that matrix form, entry by entry; the two
recurrences below (single state, and one state per Fenwick level) are
independent computations used as pins.

Layouts (token-major, like the Mamba-2 path): q, k [Bt,T,H,N] (one key and
query per head), v [Bt,T,H,P], log_alpha [Bt,T,H] (alpha = exp), beta
[Bt,T,H], lam [Bt,T,H,L]; output [Bt,T,H,P] fp64.
"""
from __future__ import annotations

import numpy as np

from . import fenwick

F64 = np.float64


def _check(q, k, v, log_alpha, beta, lam):
    Bt, T, H, N = q.shape
    P = v.shape[3]
    if k.shape != q.shape or v.shape[:3] != (Bt, T, H):
        raise ValueError("q/k/v shape mismatch")
    if log_alpha.shape != (Bt, T, H) or beta.shape != (Bt, T, H):
        raise ValueError("log_alpha/beta shape mismatch")
    if lam.shape[:3] != (Bt, T, H) or lam.shape[3] < fenwick.max_level(T) + 1:
        raise ValueError("lambda shape mismatch or too few levels")
    return Bt, T, H, N, P


def gdn_scores_bh(q, k, log_alpha, beta, b, h):
    """The gated DeltaNet attention matrix G [T, T] (zero above the diagonal)
    of one (batch, head): row t walks s = t, t-1, ..., 0 carrying
    g = H_{s+1} ... H_t q_t (the H_r are symmetric)."""
    qh = np.asarray(q[b, :, h, :], F64)
    kh = np.asarray(k[b, :, h, :], F64)
    bt = np.asarray(beta[b, :, h], F64)
    cum = np.cumsum(np.asarray(log_alpha[b, :, h], F64))
    T = qh.shape[0]
    G = np.zeros((T, T), F64)
    for t in range(T):
        g = qh[t].copy()
        for s in range(t, -1, -1):
            G[t, s] = bt[s] * np.exp(cum[t] - cum[s]) * (g @ kh[s])
            g = g - bt[s] * kh[s] * (kh[s] @ g)  # g <- H_s g, for the next s
    return G


def gdn_forward(q, k, v, log_alpha, beta, lam):
    """O = (G ⊙ M^H) V for every (batch, head), fp64 [Bt,T,H,P]."""
    Bt, T, H, N, P = _check(q, k, v, log_alpha, beta, lam)
    out = np.zeros((Bt, T, H, P), F64)
    t = np.arange(T)[:, None]
    s = np.arange(T)[None, :]
    lev = np.where(s <= t, fenwick.levels(t, np.minimum(s, t)), 0)
    for b in range(Bt):
        for h in range(H):
            G = gdn_scores_bh(q, k, log_alpha, beta, b, h)
            lamh = np.asarray(lam[b, :, h, :], F64)
            Mh = np.where(s <= t, np.take_along_axis(lamh, lev, axis=1), 0.0)
            out[b, :, h, :] = (G * Mh) @ np.asarray(v[b, :, h, :], F64)
    return out


# ------------------------------------------------------------- pins ----

def gdn_recurrent_single(q, k, v, log_alpha, beta):
    """Textbook gated DeltaNet: S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1}
    + beta_t k_t v_t^T, o_t = S_t^T q_t (no levels)."""
    Bt, T, H, N = q.shape
    P = v.shape[3]
    out = np.zeros((Bt, T, H, P), F64)
    for b in range(Bt):
        for h in range(H):
            S = np.zeros((N, P), F64)
            for t in range(T):
                kt = np.asarray(k[b, t, h], F64)
                a = np.exp(float(log_alpha[b, t, h]))
                bt = float(beta[b, t, h])
                S = a * (S - bt * np.outer(kt, kt @ S)) + bt * np.outer(kt, np.asarray(v[b, t, h], F64))
                out[b, t, h] = S.T @ np.asarray(q[b, t, h], F64)
    return out


def gdn_recurrent_levels(q, k, v, log_alpha, beta, lam):
    """One state per Fenwick level.  For t > 0 with z = trailing zeros of t:
    levels 0..z merge into level z+1 (they cover the block of 2^z tokens that
    ends at t-1), levels 1..z empty; every level state then takes the
    transition A_t; level 0 starts as beta_t k_t v_t^T; o_t = sum_l
    lambda[t, l] S^(l)^T q_t."""
    Bt, T, H, N, P = _check(q, k, v, log_alpha, beta, lam)
    L = lam.shape[3]
    out = np.zeros((Bt, T, H, P), F64)
    for b in range(Bt):
        for h in range(H):
            S = np.zeros((L, N, P), F64)
            for t in range(T):
                if t > 0:
                    z = (t & -t).bit_length() - 1
                    assert not S[z + 1].any()
                    S[z + 1] = S[: z + 1].sum(axis=0)
                    S[: z + 1] = 0.0
                kt = np.asarray(k[b, t, h], F64)
                a = np.exp(float(log_alpha[b, t, h]))
                bt = float(beta[b, t, h])
                ks = np.einsum("n,lnp->lp", kt, S)  # k_t^T S^(l) for every level
                S = a * (S - bt * kt[None, :, None] * ks[:, None, :])
                S[0] = bt * np.outer(kt, np.asarray(v[b, t, h], F64))
                qt = np.asarray(q[b, t, h], F64)
                lt = np.asarray(lam[b, t, h], F64)
                out[b, t, h] = np.einsum("l,lnp,n->p", lt, S, qt)
    return out
