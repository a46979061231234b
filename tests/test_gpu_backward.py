"""HIP backward pass vs the fp64 gradient oracle, element by element, through
the C ABI (loglin_bwd).

Sizes are ones the oracle finishes in seconds while spanning several chunks,
ragged chunk counts and every level.  Bar, per gradient: max over slices
(batch-head, or batch-group for dB and dC) of max |got - ref| / max |ref|,
<= 2e-2 for bf16 inputs and <= 1e-4 for fp32 (the forward's bar).
"""
import numpy as np
import pytest
import torch

from oracle import loglin_grad
from ssm_scan_amd import inputs
from ssm_scan_amd import loglin as L

from .gpu_helpers import say, small_cfg, to_device, tol_of

pytestmark = pytest.mark.gpu

GRADS = ("dX", "dB", "dC", "dlog_a", "dlam")


def slice_rel_err(got, ref):
    """max over the (dim 0, dim 2) slices of max|got - ref| / max|ref|."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if got.ndim == 3:
        got, ref = got[..., None], ref[..., None]
    err = np.abs(got - ref).max(axis=(1, 3))
    scale = np.abs(ref).max(axis=(1, 3))
    return float((err / np.maximum(scale, 1e-30)).max())


def grad_output(cfg, seed, dev="cuda"):
    vals, bits = inputs.make_grad_output(cfg, seed)
    if bits is not None:
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        t = torch.from_numpy(vals).to(dev)
    return vals, t


def run_bwd(t, dO, chunk, workspace=None):
    g = dict(dX=torch.empty_like(t["X"]), dB=torch.empty_like(t["B"]),
             dC=torch.empty_like(t["C"]), dlog_a=torch.empty_like(t["log_a"]),
             dlam=torch.empty_like(t["lam"]))
    L.loglin_bwd(t["X"], t["B"], t["C"], t["log_a"], t["lam"], dO, chunk, g["dX"], g["dB"],
                 g["dC"], g["dlog_a"], g["dlam"], workspace=workspace)
    return g


def check(cfg, seed=0, variant=None, chunk=None, extra_levels=0):
    chunk = chunk or cfg.chunk
    if extra_levels:
        cfg = cfg.replace(nlevels=cfg.nlevels + extra_levels)
    say(f"[backward] {cfg.name} L={cfg.nlevels} seed={seed} variant={variant} chunk={chunk}")
    d = inputs.make_inputs(cfg, seed, variant=variant)
    t = to_device(d, cfg)
    dOv, dO = grad_output(cfg, seed)
    g = run_bwd(t, dO, chunk)
    torch.cuda.synchronize()
    got = {k: v.float().cpu().numpy() for k, v in g.items()}
    ref = loglin_grad.loglin_grad(d["X"], d["B"], d["C"], d["log_a"], d["lam"], dOv)
    tol = tol_of(cfg)
    errs = {k: slice_rel_err(got[k], ref[k]) for k in GRADS}
    say("           " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()) + f" (tol {tol:.0e})")
    for k in GRADS:
        assert np.isfinite(got[k]).all(), k
        assert errs[k] <= tol, (k, errs[k])
    ll = inputs.num_levels(cfg.seqlen)
    assert np.all(got["dlam"][..., ll:] == 0.0)  # levels the sequence never reaches
    return got, ref


def test_tiny_fp32_config():
    """256 tokens, 1 head, P = N = 16, chunk 16 (16 chunks, 4 chunk levels)."""
    check(inputs.CONFIGS["tiny_fp32"])


@pytest.mark.parametrize("T,P,N,C", [(192, 32, 64, 16), (448, 64, 32, 32), (320, 16, 128, 64),
                                     (64, 32, 16, 64)])
def test_fp32_shapes(T, P, N, C):
    """fp32 shapes and chunks; 12, 14 and 5 chunks are ragged counts, and
    T = 64 at chunk 64 is a single chunk (no chunk levels)."""
    check(small_cfg(dtype="fp32", T=T, H=2, G=1, P=P, N=N, C=C, decay="softplus"))


@pytest.mark.parametrize("T", [64, 128, 320, 1344, 2048])
def test_headline_shape_lengths(T):
    """P = 64, N = 128, groups of 2, chunk 64, Mamba-2 decay; T = 64 is one
    chunk, 320 and 1344 are ragged chunk counts (5, 21)."""
    check(small_cfg(T=T))


@pytest.mark.parametrize("P,N,C", [(32, 64, 32), (64, 32, 64), (32, 128, 64), (64, 64, 32), (64, 64, 64)])
def test_bf16_shapes(P, N, C):
    check(small_cfg(T=704, H=4, G=1, P=P, N=N, C=C))


def test_t2k_bf16_config():
    """2 x 2048 tokens, 8 heads (one per group), P = N = 64, chunk 64."""
    check(inputs.CONFIGS["t2k_bf16"])


@pytest.mark.parametrize("seed", [1, 2])
def test_other_seeds(seed):
    check(small_cfg(T=1024, H=4, G=2), seed=seed)


@pytest.mark.parametrize("variant", ["slow_decay", "no_decay", "lam_intra", "lam_inter",
                                     "lam_ones", "lam_onehot_0", "lam_onehot_3",
                                     "lam_onehot_6", "lam_onehot_7", "lam_onehot_10"])
def test_variants(variant):
    """Decay and lambda variants that isolate the intra block, the chunk
    levels, single levels and the long-range terms."""
    check(small_cfg(T=1344, H=2, G=1), variant=variant)


def test_group_of_four_heads_and_batch():
    check(small_cfg(T=512, H=8, G=2, Bt=2))


def test_batch_long_levels():
    """Two sequences of 40 chunks: chunk levels 1-6, the upper ones in
    several pieces (the reduce) and above the groups of 8 (the group walk)."""
    check(small_cfg(T=64 * 40, H=4, G=2, Bt=2), variant="slow_decay")


def test_extra_levels_are_zero():
    check(small_cfg(T=320, H=2, G=1), extra_levels=3)


def test_chunk_choices_agree():
    """The gradients do not depend on the chunk (32 or 64)."""
    cfg = small_cfg(T=1024, H=2, G=1)
    a, ref = check(cfg, chunk=32)
    b, _ = check(cfg, chunk=64)
    for k in GRADS:
        assert slice_rel_err(a[k], b[k]) <= 2 * tol_of(cfg), k


def test_repeatable_bitwise():
    """No atomics: two calls give identical bits."""
    cfg = small_cfg(T=640, H=4, G=2)
    d = inputs.make_inputs(cfg, 3)
    t = to_device(d, cfg)
    _, dO = grad_output(cfg, 3)
    g1 = run_bwd(t, dO, 64)
    g2 = run_bwd(t, dO, 64)
    torch.cuda.synchronize()
    for k in GRADS:
        assert torch.equal(g1[k], g2[k]), k


def test_workspace_reuse_with_stale_contents():
    """A workspace holding another call's data gives the same result."""
    cfg = small_cfg(T=512, H=2, G=1)
    dims = L.dims_of(*(torch.empty(s, dtype=torch.bfloat16, device="cuda") for s in
                       ((1, 512, 2, 64), (1, 512, 1, 128), (1, 512, 2, cfg.nlevels))))
    ws = torch.full((L.loglin_bwd_workspace_bytes(dims, 64),), 0x7F, dtype=torch.uint8,
                    device="cuda")
    outs = []
    for seed in (4, 5, 4):
        d = inputs.make_inputs(cfg, seed)
        t = to_device(d, cfg)
        _, dO = grad_output(cfg, seed)
        outs.append(run_bwd(t, dO, 64, workspace=ws))
    torch.cuda.synchronize()
    for k in GRADS:
        assert torch.equal(outs[0][k], outs[2][k]), k
