"""Seeded synthetic inputs for the log-linear Mamba-2 forward.

This module only draws random numbers and rounds them to the storage type.
It holds none of the method's arithmetic, so both the fp64 oracle (through
the tests) and the HIP path consume exactly the same values.

Workload shapes follow the benchmark setup of the log-linear attention
write-up (yoousoft.com, section on the Mamba-2 / gated generalisation and
the H100 setup paragraph): group size 2, 48 heads, head dim 64, state 128,
chunk 64, at sequence lengths 8K, 32K and 131K.  Decay follows Mamba-2's
per-head scalar parameterisation, log a_t = -dt_t * exp(A_log[h]).

Every tensor is drawn in float32 from numpy PCG64 streams, in flat blocks
of BLOCK elements; block i of tensor k uses its own stream seeded with
SeedSequence([seed, k, i]) (k: 0 X, 1 B, 2 C, 3 dt noise, 4 lambda, 5 A_log,
6 the output gradient dO of the backward pass; 7..13 the gated DeltaNet
inputs q, k, v, dt noise, beta noise, lambda, A_log).
The values therefore do not depend on how many threads fill the blocks.
bf16 inputs are rounded to nearest-even from those float32 draws.
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import math
import os

import numpy as np

__all__ = [
    "Config",
    "CONFIGS",
    "make_inputs",
    "bf16_round",
    "num_levels",
    "make_grad_output",
    "make_gdn_inputs",
]


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    batch: int
    seqlen: int
    nheads: int
    ngroups: int
    headdim: int  # P, value dim
    dstate: int  # N, state dim
    chunk: int
    nlevels: int  # L = ceil(log2 T) + 1
    dtype: str  # "fp32" or "bf16"
    decay: str  # "softplus" (configs 1-2) or "mamba2" (configs 3-5)

    def shapes(self):
        Bt, T, H, G, P, N, L = (self.batch, self.seqlen, self.nheads,
                                self.ngroups, self.headdim, self.dstate,
                                self.nlevels)
        return dict(X=(Bt, T, H, P), B=(Bt, T, G, N), C=(Bt, T, G, N),
                    log_a=(Bt, T, H), lam=(Bt, T, H, L), out=(Bt, T, H, P))

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


def num_levels(seqlen: int) -> int:
    """Number of Fenwick levels needed for a sequence: ceil(log2 T) + 1."""
    return (max(seqlen, 1) - 1).bit_length() + 1


CONFIGS = {
    "tiny_fp32": Config("tiny_fp32", 1, 256, 1, 1, 16, 16, 16, 9, "fp32",
                        "softplus"),
    "t2k_bf16": Config("t2k_bf16", 2, 2048, 8, 8, 64, 64, 64, 12, "bf16",
                       "softplus"),
    "t8k_bf16": Config("t8k_bf16", 1, 8192, 48, 24, 64, 128, 64, 14, "bf16",
                       "mamba2"),
    "t32k_bf16": Config("t32k_bf16", 1, 32768, 48, 24, 64, 128, 64, 16,
                        "bf16", "mamba2"),
    "t131k_bf16": Config("t131k_bf16", 1, 131072, 48, 24, 64, 128, 64, 18,
                         "bf16", "mamba2"),
}


def _bf16_round_flat(x, bits, vals):
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    bits[:] = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    vals.view(np.uint32)[:] = bits.astype(np.uint32) << np.uint32(16)


def bf16_round(x: np.ndarray):
    """Round float32 values to bfloat16, nearest-even.

    Returns ``(bits, values)``: the raw uint16 bf16 bit patterns and the same
    numbers widened back to float32 (exactly representable).  Inputs are
    finite; no NaN handling is needed for these draws.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    bits = np.empty(flat.size, dtype=np.uint16)
    vals = np.empty(flat.size, dtype=np.float32)
    nblk = (flat.size + BLOCK - 1) // BLOCK

    def run(i):
        sl = slice(i * BLOCK, min(flat.size, (i + 1) * BLOCK))
        _bf16_round_flat(flat[sl], bits[sl], vals[sl])

    if nblk <= 1:
        for i in range(nblk):
            run(i)
    else:
        with cf.ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(run, range(nblk)))
    return bits.reshape(x.shape), vals.reshape(x.shape)


BLOCK = 1 << 22
_THREADS = min(16, os.cpu_count() or 1)


def _normal(seed: int, tensor_id: int, shape) -> np.ndarray:
    """Standard normal float32 draws, filled block by block in threads."""
    out = np.empty(int(np.prod(shape)), dtype=np.float32)

    def fill(i):
        lo = i * BLOCK
        hi = min(out.size, lo + BLOCK)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_id, i])))
        rng.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])

    nblk = (out.size + BLOCK - 1) // BLOCK
    if nblk <= 1:
        for i in range(nblk):
            fill(i)
    else:
        with cf.ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(fill, range(nblk)))
    return out.reshape(shape)


def _softplus(x: np.ndarray) -> np.ndarray:
    # numerically safe softplus in float32 (a distribution shape, not the method)
    return (np.maximum(x, 0) + np.log1p(np.exp(-np.abs(x)))).astype(np.float32)


def make_inputs(cfg: Config, seed: int = 0, *, variant: str | None = None):
    """Draw the inputs of one configuration.

    Returns a dict with float32 arrays ``X, B, C, log_a, lam`` holding the
    exact values the kernels see (bf16-rounded for bf16 configs; log_a is
    always float32), plus ``bits`` (uint16 arrays for the bf16 tensors, or
    None for fp32 configs).

    ``variant`` modifies the draw after the fact (the draw itself is
    unchanged), to exercise parts of the method the default draws barely
    reach:
      - "slow_decay": log_a scaled by 1e-3
      - "no_decay":   log_a = 0 (a = 1)
      - "lam_onehot_<l>": lambda = 1 on level l, 0 elsewhere
      - "lam_intra": lambda zero on every level above log2(chunk)
      - "lam_inter": lambda zero on levels 0..log2(chunk)
      - "lam_ones":  lambda = 1 everywhere
    Several modifications join with "+", applied left to right (for
    instance "slow_decay+lam_onehot_14").
    """
    sh = cfg.shapes()
    f32 = np.float32
    X = _normal(seed, 0, sh["X"])
    inv_sqrt_n = f32(1.0 / math.sqrt(cfg.dstate))
    B = _normal(seed, 1, sh["B"])
    B *= inv_sqrt_n
    C = _normal(seed, 2, sh["C"])
    C *= inv_sqrt_n
    if cfg.decay == "softplus":
        log_a = -f32(0.5) * _softplus(_normal(seed, 3, sh["log_a"]))
    elif cfg.decay == "mamba2":
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 5, 0])))
        A_log = rng.uniform(0.0, math.log(16.0), size=(cfg.nheads,)).astype(f32)
        dt = _softplus(_normal(seed, 3, sh["log_a"]) - f32(2.0))
        log_a = -(dt * np.exp(A_log)[None, None, :]).astype(f32)
    else:
        raise ValueError(cfg.decay)
    lam = _softplus(_normal(seed, 4, sh["lam"]))

    for mod in ([] if variant is None else variant.split("+")):
        c = cfg.chunk.bit_length() - 1
        if mod == "slow_decay":
            log_a = (log_a * f32(1e-3)).astype(f32)
        elif mod == "no_decay":
            log_a = np.zeros_like(log_a)
        elif mod.startswith("lam_onehot_"):
            lev = int(mod.rsplit("_", 1)[1])
            lam = np.zeros_like(lam)
            lam[..., lev] = 1.0
        elif mod == "lam_intra":
            lam = lam.copy()
            lam[..., c + 1:] = 0.0
        elif mod == "lam_inter":
            lam = lam.copy()
            lam[..., :c + 1] = 0.0
        elif mod == "lam_ones":
            lam = np.ones_like(lam)
        else:
            raise ValueError(f"unknown variant {mod!r}")

    out = dict(log_a=np.ascontiguousarray(log_a, dtype=f32))
    if cfg.dtype == "bf16":
        bits = {}
        for k, v in (("X", X), ("B", B), ("C", C), ("lam", lam)):
            bits[k], out[k] = bf16_round(v)
        out["bits"] = bits
    elif cfg.dtype == "fp32":
        for k, v in (("X", X), ("B", B), ("C", C), ("lam", lam)):
            out[k] = np.ascontiguousarray(v, dtype=f32)
        out["bits"] = None
    else:
        raise ValueError(cfg.dtype)
    return out


def make_grad_output(cfg: Config, seed: int = 0):
    """Seeded upstream gradient dO [Bt,T,H,P] ~ N(0, 1) for the backward
    pass, in the configuration's storage type (its own stream, so the
    forward inputs of the same seed are unchanged).

    Returns ``(values, bits)``: float32 values exactly as the kernels see
    them, and the uint16 bf16 bit patterns (None for fp32 configs).
    """
    dO = _normal(seed, 6, cfg.shapes()["out"])
    if cfg.dtype == "bf16":
        bits, vals = bf16_round(dO)
        return vals, bits
    if cfg.dtype == "fp32":
        return np.ascontiguousarray(dO, dtype=np.float32), None
    raise ValueError(cfg.dtype)


def make_gdn_inputs(cfg: Config, seed: int = 0):
    """Seeded inputs of the log-linear gated DeltaNet forward for the shapes
    of `cfg` (one query and key per head: q, k [Bt,T,H,N], v [Bt,T,H,P]).

    Distributions follow gated DeltaNet practice: q and k L2-normalised per
    token (so each I - beta k k^T is a contraction), v ~ N(0, 1), beta =
    sigmoid(N(0, 1)), the Mamba-2 style decay of `cfg` for log alpha, and
    lambda = softplus(N(0, 1)).  beta and log_alpha stay float32; q, k, v
    and lambda are rounded to the configuration's storage type.  Returns a
    dict of float32 arrays holding exactly the values the kernels see, plus
    ``bits`` (uint16 patterns for bf16 configs, else None).
    """
    Bt, T, H, N, P, L = cfg.batch, cfg.seqlen, cfg.nheads, cfg.dstate, cfg.headdim, cfg.nlevels
    f32 = np.float32

    def unit(x):
        return (x / np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))).astype(f32)

    q = unit(_normal(seed, 7, (Bt, T, H, N)))
    k = unit(_normal(seed, 8, (Bt, T, H, N)))
    v = _normal(seed, 9, (Bt, T, H, P))
    if cfg.decay == "mamba2":
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 13, 0])))
        A_log = rng.uniform(0.0, math.log(16.0), size=(H,)).astype(f32)
        dt = _softplus(_normal(seed, 10, (Bt, T, H)) - f32(2.0))
        log_alpha = -(dt * np.exp(A_log)[None, None, :]).astype(f32)
    else:
        log_alpha = -f32(0.5) * _softplus(_normal(seed, 10, (Bt, T, H)))
    beta = (1.0 / (1.0 + np.exp(-_normal(seed, 11, (Bt, T, H)).astype(np.float64)))).astype(f32)
    lam = _softplus(_normal(seed, 12, (Bt, T, H, L)))
    out = dict(log_alpha=np.ascontiguousarray(log_alpha, f32), beta=np.ascontiguousarray(beta, f32))
    if cfg.dtype == "bf16":
        bits = {}
        for name, x in (("q", q), ("k", k), ("v", v), ("lam", lam)):
            bits[name], out[name] = bf16_round(x)
        out["bits"] = bits
    elif cfg.dtype == "fp32":
        for name, x in (("q", q), ("k", k), ("v", v), ("lam", lam)):
            out[name] = np.ascontiguousarray(x, f32)
        out["bits"] = None
    else:
        raise ValueError(cfg.dtype)
    return out
