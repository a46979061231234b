"""Shared helpers of the GPU parity tests: move seeded inputs to the device,
run the HIP path through the C ABI binding, compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

from ssm_scan_amd import inputs
from ssm_scan_amd import loglin as L

BF16_TOL = 2e-2  # max relative error, bf16 inputs with fp32 accumulation
FP32_TOL = 1e-4  # max relative error, fp32 inputs


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(d, cfg, dev="cuda"):
    """Device tensors holding exactly the generator's values."""
    t = {}
    if cfg.dtype == "bf16":
        for k in ("X", "B", "C", "lam"):
            bits = np.ascontiguousarray(d["bits"][k]).view(np.int16)
            t[k] = torch.from_numpy(bits).to(dev).view(torch.bfloat16)
    else:
        for k in ("X", "B", "C", "lam"):
            t[k] = torch.from_numpy(np.ascontiguousarray(d[k])).to(dev)
    t["log_a"] = torch.from_numpy(d["log_a"]).to(dev)
    return t


def run_gpu(cfg, t, chunk=None, seg_log2=None, out=None, stream=None, heads_per_block=None):
    chunk = chunk or cfg.chunk
    if out is None:
        out = torch.empty_like(t["X"])
    L.loglin_fwd(t["X"], t["B"], t["C"], t["log_a"], t["lam"], chunk, out,
                 seg_log2=seg_log2, stream=stream, heads_per_block=heads_per_block)
    return out


def max_rel_err(out, ref):
    """max over (batch, head) slices of max|out - ref| / max|ref|; arrays
    [Bt, T, H, P] (or any [Bt, R, H, P] sample of rows)."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(out - ref).max(axis=(1, 3))
    scale = np.abs(ref).max(axis=(1, 3))
    return float((err / np.maximum(scale, 1e-30)).max())


def tol_of(cfg):
    return BF16_TOL if cfg.dtype == "bf16" else FP32_TOL


def small_cfg(dtype="bf16", T=320, H=4, G=2, P=64, N=128, C=64, Bt=1,
              decay="mamba2"):
    return inputs.Config(f"test_{dtype}_T{T}_H{H}_G{G}_P{P}_N{N}_C{C}_B{Bt}", Bt, T, H, G,
                         P, N, C, inputs.num_levels(T), dtype, decay)
