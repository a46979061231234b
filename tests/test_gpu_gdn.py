"""HIP log-linear gated DeltaNet forward (loglin_gdn_fwd) vs the fp64 oracle,
element by element, through the C ABI.

Short sequences use the oracle's matrix form; longer ones its one-state-
per-level Fenwick recurrence (the two are pinned to each other and to the
textbook gated DeltaNet in test_oracle_gdn).  Bar: max over batch-head
slices of max |out - ref| / max |ref| <= 2e-2 for bf16, <= 1e-4 for fp32.
"""
import numpy as np
import pytest
import torch

from oracle import gdn_ref
from ssm_scan_amd import inputs
from ssm_scan_amd import loglin as L

from .gpu_helpers import max_rel_err, say, tol_of

pytestmark = pytest.mark.gpu


def gdn_cfg(dtype="bf16", T=256, H=2, N=128, P=64, Bt=1, decay="mamba2", extra=0):
    return inputs.Config(f"gdn_{dtype}_T{T}_H{H}_N{N}_P{P}_B{Bt}", Bt, T, H, H, P, N, 32,
                         inputs.num_levels(T) + extra, dtype, decay)


def to_dev(d, cfg):
    t = {}
    for name in ("q", "k", "v", "lam"):
        if cfg.dtype == "bf16":
            t[name] = torch.from_numpy(np.ascontiguousarray(d["bits"][name]).view(np.int16)).cuda().view(
                torch.bfloat16)
        else:
            t[name] = torch.from_numpy(d[name]).cuda()
    t["log_alpha"] = torch.from_numpy(d["log_alpha"]).cuda()
    t["beta"] = torch.from_numpy(d["beta"]).cuda()
    return t


def run(t):
    out = torch.empty_like(t["v"])
    L.loglin_gdn_fwd(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], t["lam"], out)
    return out


def check(cfg, seed=0, lam=None, log_alpha_scale=None):
    say(f"[gdn] {cfg.name} L={cfg.nlevels} seed={seed} lam={lam} la_scale={log_alpha_scale}")
    d = inputs.make_gdn_inputs(cfg, seed)
    if log_alpha_scale is not None:
        d["log_alpha"] = (d["log_alpha"] * np.float32(log_alpha_scale)).astype(np.float32)
    if lam is not None:
        d["lam"] = lam(d["lam"]).astype(np.float32)
        if cfg.dtype == "bf16":
            d["bits"]["lam"], d["lam"] = inputs.bf16_round(d["lam"])
    t = to_dev(d, cfg)
    out = run(t)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    args = (d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["lam"])
    ref = gdn_ref.gdn_forward(*args) if cfg.seqlen <= 256 else gdn_ref.gdn_recurrent_levels(*args)
    err = max_rel_err(got, ref)
    say(f"       max_rel_err={err:.3e} (tol {tol_of(cfg):.0e})")
    assert np.isfinite(got).all()
    assert err <= tol_of(cfg), err
    return got


@pytest.mark.parametrize("T", [32, 96, 256, 1024, 2048])
def test_bf16_lengths(T):
    """One chunk, a ragged chunk count (3), and longer sequences (every
    chunk level up to 6), key dim 128, value dim 64."""
    check(gdn_cfg(T=T))


@pytest.mark.parametrize("N,P", [(64, 32), (32, 16), (16, 64), (128, 16)])
def test_bf16_shapes(N, P):
    check(gdn_cfg(T=320, N=N, P=P))


@pytest.mark.parametrize("T,N,P", [(96, 16, 16), (640, 64, 32), (256, 128, 64)])
def test_fp32(T, N, P):
    check(gdn_cfg(dtype="fp32", T=T, N=N, P=P, decay="softplus"))


def test_batch_and_heads():
    check(gdn_cfg(T=192, H=3, Bt=2))


@pytest.mark.parametrize("lev", [0, 3, 5, 6, 9])
def test_lambda_one_hot(lev):
    """lambda one-hot on one level: the intra-chunk levels (0..5) and the
    chunk levels (6 and up) in isolation."""
    def f(lam):
        out = np.zeros_like(lam)
        out[..., lev] = 1.0
        return out
    check(gdn_cfg(T=1024), lam=f)


def test_lambda_ones_is_gated_deltanet():
    cfg = gdn_cfg(T=512)
    got = check(cfg, lam=np.ones_like)
    d = inputs.make_gdn_inputs(cfg, 0)
    ref = gdn_ref.gdn_recurrent_single(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"])
    assert max_rel_err(got, ref) <= tol_of(cfg)


@pytest.mark.parametrize("scale", [1e-3, 0.0])
def test_slow_and_no_decay(scale):
    """Slow or no decay: long-range levels carry weight."""
    check(gdn_cfg(T=1024), log_alpha_scale=scale)


def test_extra_levels_and_seeds():
    check(gdn_cfg(T=320, extra=3), seed=1)
    check(gdn_cfg(T=320), seed=2)


def test_repeatable_bitwise():
    cfg = gdn_cfg(T=256)
    t = to_dev(inputs.make_gdn_inputs(cfg, 3), cfg)
    a, b = run(t), run(t)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
