"""HIP path vs the fp64 oracle, element by element, through the C ABI.

Sizes here are ones the oracle finishes in seconds while spanning several
chunks, a ragged number of chunks and every level.  Full-size workloads are
in test_gpu_full.py.  Bar: max relative error (per batch-head slice, max
|out - ref| / max |ref|) <= 2e-2 for bf16 inputs, <= 1e-4 for fp32.
"""
import numpy as np
import pytest
import torch

from oracle import loglin_ref
from ssm_scan_amd import inputs
from ssm_scan_amd import loglin as L

from .gpu_helpers import (max_rel_err, run_gpu, say, small_cfg, to_device, tol_of)

pytestmark = pytest.mark.gpu


def check(cfg, seed=0, variant=None, chunk=None, seg_log2=None, heads_per_block=None):
    say(f"[parity] {cfg.name} seed={seed} variant={variant} chunk={chunk} seg={seg_log2} "
        f"hp={heads_per_block}")
    d = inputs.make_inputs(cfg, seed, variant=variant)
    t = to_device(d, cfg)
    out = run_gpu(cfg, t, chunk=chunk, seg_log2=seg_log2, heads_per_block=heads_per_block)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    ref = loglin_ref.loglin_forward(d["X"], d["B"], d["C"], d["log_a"], d["lam"])
    err = max_rel_err(got, ref)
    say(f"         max_rel_err={err:.3e} (tol {tol_of(cfg):.0e})")
    assert np.isfinite(got).all()
    assert err <= tol_of(cfg), err
    return got, ref


def test_tiny_fp32_config():
    """256 tokens, 1 head, P=N=16, chunk 16, fp32 (1e-4 bar)."""
    check(inputs.CONFIGS["tiny_fp32"])


def test_t2k_bf16_config():
    """2 x 2048 tokens, 8 heads, P=N=64, chunk 64, bf16."""
    check(inputs.CONFIGS["t2k_bf16"])


@pytest.mark.parametrize("seed", [1, 2])
def test_t2k_bf16_other_seeds(seed):
    cfg = inputs.CONFIGS["t2k_bf16"].replace(batch=1, nheads=4, ngroups=4)
    check(cfg, seed=seed)


@pytest.mark.parametrize("T", [64, 128, 320, 1344, 2048])
def test_headline_shape_lengths(T):
    """Headline head shape (P=64, N=128, groups of 2), Mamba-2 decay; T=64 is
    one chunk (no inter levels, no workspace); 320 and 1344 are ragged chunk
    counts (5, 21)."""
    check(small_cfg(T=T))


@pytest.mark.parametrize("dtype,P,N,C", [
    ("bf16", 16, 32, 16), ("bf16", 32, 64, 32), ("bf16", 64, 32, 64),
    ("bf16", 16, 128, 32), ("bf16", 64, 64, 64), ("fp32", 16, 16, 16), ("fp32", 64, 128, 64),
    ("fp32", 32, 64, 32), ("fp32", 64, 16, 16),
])
def test_shapes_and_chunks(dtype, P, N, C):
    check(small_cfg(dtype=dtype, T=C * 11, H=2, G=1, P=P, N=N, C=C, decay="softplus"))


def test_batch_gt_one():
    check(small_cfg(T=512, H=4, G=2, Bt=3))


@pytest.mark.parametrize("seg", [None, 0])
def test_batch_segments(seg):
    """Two sequences long enough for the state pass and the level scan
    (5 segments of 8 chunks, or 40 one-chunk segments in three ranges)."""
    check(small_cfg(T=64 * 40, H=4, G=2, Bt=2), seg_log2=seg, variant="slow_decay")


@pytest.mark.parametrize("variant", ["slow_decay", "no_decay", "lam_intra", "lam_inter",
                                     "lam_ones"])
def test_variants(variant):
    """Slow / no decay reach the deep levels; lambda zeroed on inter (or
    intra) levels isolates the intra-chunk kernel (or the inter path)."""
    check(small_cfg(T=1024, H=2, G=1), variant=variant)


@pytest.mark.parametrize("level", range(0, 12))
def test_onehot_levels(level):
    """lambda one-hot on each level: every Fenwick level in isolation
    (levels 0..6 intra-chunk, 7..11 inter-chunk at chunk 64, T = 2048)."""
    check(small_cfg(T=2048, H=2, G=1), variant=f"lam_onehot_{level}")


@pytest.mark.parametrize("seg", [0, 1, 2, 3])
@pytest.mark.parametrize("T", [1344, 2048])
def test_segment_depths(seg, T):
    """Chunks per segment 1..8: levels move between the on-chip Fenwick
    stack of the output pass and the slots of the level scan."""
    check(small_cfg(T=T, H=2, G=1), seg_log2=seg, variant="slow_decay")


@pytest.mark.parametrize("nseg,C", [(100, 64), (128, 64), (130, 64), (256, 32), (257, 32)])
def test_segment_ranges(nseg, C):
    """One-chunk segments, 100 to 256 of them (the level scan in ranges of
    16 segments: blocks of 2 to 8 ranges, a short last range, gaps of levels
    above a range; 32-token chunks keep the oracle's sequence short) and 257
    (the single sweep)."""
    check(small_cfg(T=C * nseg, H=2, G=1, C=C), seg_log2=0, variant="slow_decay")


@pytest.mark.parametrize("seg", [0, 1, 2, 3])
def test_segment_depths_fp32(seg):
    cfg = small_cfg(dtype="fp32", T=16 * 37, H=2, G=1, P=16, N=32, C=16, decay="softplus")
    check(cfg, seg_log2=seg)


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_chunk_invariance(chunk):
    """The result does not depend on the chunk size (up to rounding)."""
    check(small_cfg(T=1024, H=2, G=1), chunk=chunk, variant="slow_decay")


def test_fp32_chunk_invariance_tight():
    cfg = small_cfg(dtype="fp32", T=512, H=2, G=1, P=32, N=32, C=16, decay="softplus")
    d = inputs.make_inputs(cfg, 3, variant="slow_decay")
    t = to_device(d, cfg)
    outs = [run_gpu(cfg, t, chunk=c).cpu().numpy() for c in (16, 32, 64)]
    ref = loglin_ref.loglin_forward(d["X"], d["B"], d["C"], d["log_a"], d["lam"])
    for o in outs:
        assert max_rel_err(o, ref) <= 1e-4


def test_determinism():
    """Two runs on the same inputs are bit-identical (no atomics)."""
    cfg = small_cfg(T=2048, H=4, G=2)
    d = inputs.make_inputs(cfg, 0)
    t = to_device(d, cfg)
    a = run_gpu(cfg, t).clone()
    b = run_gpu(cfg, t).clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_causality():
    """Perturbing tokens >= t0 leaves every output row < t0 bit-identical."""
    cfg = small_cfg(T=1024, H=2, G=1)
    d = inputs.make_inputs(cfg, 0)
    t = to_device(d, cfg)
    a = run_gpu(cfg, t).clone()
    t0 = 700
    for k in ("X", "B", "C", "lam"):
        t[k][:, t0:] = t[k][:, t0:] * 2 + 1
    t["log_a"][:, t0:] -= 0.3
    b = run_gpu(cfg, t)
    torch.cuda.synchronize()
    assert torch.equal(a[:, :t0], b[:, :t0])
    assert not torch.equal(a[:, t0:], b[:, t0:])


def test_extra_levels_ignored():
    """lambda with more levels than ceil(log2 T) + 1: extra ones unused."""
    cfg = small_cfg(T=512, H=2, G=1)
    d = inputs.make_inputs(cfg, 0)
    t = to_device(d, cfg)
    a = run_gpu(cfg, t).clone()
    lam2 = torch.cat([t["lam"], torch.full_like(t["lam"][..., :3], 7.0)], dim=-1).contiguous()
    t2 = dict(t, lam=lam2)
    b = run_gpu(cfg, t2)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("H,G", [(2, 2), (3, 1), (4, 1), (6, 3)])
def test_head_grouping(H, G):
    """Heads per group 1, 3, 4 and 2 with one head per work-group."""
    check(small_cfg(T=1344, H=H, G=G), variant="slow_decay")


@pytest.mark.parametrize("T,seg", [(1344, None), (64 * 33, None), (64 * 64, None), (2048, 1),
                                   (2048, 0), (64, None), (320, None)])
def test_head_pairs(T, seg):
    """Two heads of a group per work-group (shared B, C and scores, lowest
    level slot above the segment in LDS): 2 and 4 heads per group, chunk
    counts whose segments reach 1..3 levels above them, segment depths 0..3
    and one chunk."""
    check(small_cfg(T=T, H=4, G=1), variant="slow_decay", seg_log2=seg, heads_per_block=2)
    check(small_cfg(T=T, H=4, G=2), seg_log2=seg, heads_per_block=2)


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_head_pairs_chunks(chunk):
    check(small_cfg(T=1024, H=2, G=1), chunk=chunk, variant="slow_decay", heads_per_block=2)


@pytest.mark.parametrize("level", [0, 5, 6, 7, 9, 11])
def test_head_pairs_onehot_levels(level):
    check(small_cfg(T=2048, H=2, G=1), variant=f"lam_onehot_{level}", heads_per_block=2)


def test_head_pairs_odd_levels():
    """An odd level count: bf16 rows of the second head start mid-word."""
    cfg = small_cfg(T=512, H=2, G=1)
    d = inputs.make_inputs(cfg, 0)
    t = to_device(d, cfg)
    lam2 = torch.cat([t["lam"], torch.full_like(t["lam"][..., :3], 7.0)], dim=-1).contiguous()
    t2 = dict(t, lam=lam2)
    a = run_gpu(cfg, t2, heads_per_block=1).clone()
    b2 = run_gpu(cfg, t2, heads_per_block=2)
    torch.cuda.synchronize()
    ref = loglin_ref.loglin_forward(d["X"], d["B"], d["C"], d["log_a"], d["lam"])
    assert max_rel_err(b2.float().cpu().numpy(), ref) <= 2e-2
    assert max_rel_err(a.float().cpu().numpy(), ref) <= 2e-2


@pytest.mark.parametrize("T,seg", [(1344, None), (2048, 0), (64 * 64, None)])
def test_one_head_per_block(T, seg):
    """One head per output work-group forced where pairs are the default."""
    check(small_cfg(T=T, H=4, G=2), variant="slow_decay", seg_log2=seg, heads_per_block=1)


def run_masked(cfg, t, mask, **kw):
    out = torch.empty_like(t["X"])
    L.loglin_fwd(t["X"], t["B"], t["C"], t["log_a"], t["lam"], cfg.chunk, out, level_mask=mask,
                 **kw)
    return out


@pytest.mark.parametrize("name", ["one", "intra", "inter", "mixed"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_level_mask(name, dtype):
    """Only the masked levels enter the output: against the oracle with the
    other levels' weights set to zero."""
    cfg = small_cfg(dtype=dtype, T=2048, H=2, G=1, P=64, N=128 if dtype == "bf16" else 64,
                    C=64 if dtype == "bf16" else 32)
    LL = inputs.num_levels(cfg.seqlen)
    c = cfg.chunk.bit_length() - 1
    masks = {"one": 1 << (c + 2), "intra": (2 << c) - 1, "inter": ((1 << LL) - 1) & ~((2 << c) - 1),
             "mixed": 0b101001 | (1 << (LL - 1))}
    mask = masks[name]
    say(f"[mask] {cfg.name} mask={mask:#x}")
    d = inputs.make_inputs(cfg, 0, variant="slow_decay")
    t = to_device(d, cfg)
    got = run_masked(cfg, t, mask)
    torch.cuda.synchronize()
    keep = np.array([(mask >> l) & 1 for l in range(d["lam"].shape[-1])], dtype=np.float32)
    ref = loglin_ref.loglin_forward(d["X"], d["B"], d["C"], d["log_a"], d["lam"] * keep)
    err = max_rel_err(got.float().cpu().numpy(), ref)
    say(f"         max_rel_err={err:.3e}")
    assert err <= tol_of(cfg), err


def test_per_level_passes_sum_to_fused():
    """One pass per level (the unfused variant), summed in fp32, equals the
    fused output."""
    cfg = small_cfg(T=4096, H=4, G=2)
    d = inputs.make_inputs(cfg, 0, variant="slow_decay")
    t = to_device(d, cfg)
    LL = inputs.num_levels(cfg.seqlen)
    total = sum(run_masked(cfg, t, 1 << l).float() for l in range(LL))
    fused = run_gpu(cfg, t).float()
    torch.cuda.synchronize()
    ref = loglin_ref.loglin_forward(d["X"], d["B"], d["C"], d["log_a"], d["lam"])
    assert max_rel_err(total.cpu().numpy(), ref) <= tol_of(cfg)
    assert max_rel_err(total.cpu().numpy(), fused.cpu().numpy()) <= tol_of(cfg)
