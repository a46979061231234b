"""Full-size workloads (8K, 32K, 131K tokens; 48 heads in groups of 2;
P=64, N=128, chunk 64, bf16) in the launch configuration the benchmark
times (default segment depth, one head per output work-group).

At 8K the oracle forms every output of every head.  Longer sequences are
checked on rows the oracle computes one by one from their full causal
prefix: whole chunks at the chunk indices where Fenwick levels switch
(0, 1, 2^k - 1, 2^k, the last one), the rows 2^k - 1, 2^k, 2^k + 1, and
seeded random rows, for heads spread over every XCD's share of the output
pass's tiles (each XCD serves a contiguous run of six heads at this size).

Under the workloads' Mamba-2 decay a key 3000 tokens back weighs about
e^-500, so the levels far above a segment and the deep entries of the
level scan's stack would pass any test unchecked.  The slow-decay variants
(log a scaled by 1e-3) and the one-hot lambda on the deepest levels give
them full weight; those runs include every row of chunks in segments
whose index has four or more set bits (levels beyond the three slots the
output pass keeps in registers are streamed from memory there).

Levels switch where the write-up's tree partition puts them (section
"special structure: tree partition": levels up to ceil(log2 T)); the
levels above a chunk are the inter-chunk phase of the chunked algorithm
(section "efficient training algorithm").
"""
import concurrent.futures as cf
import os

import numpy as np
import pytest
import torch
from threadpoolctl import threadpool_limits

from oracle import loglin_ref
from ssm_scan_amd import inputs
from ssm_scan_amd import loglin as L

from .gpu_helpers import BF16_TOL, max_rel_err, run_gpu, say, to_device

pytestmark = pytest.mark.gpu

# the GPU machine gives one GPU a 16-core share, whatever os.cpu_count() says
ORACLE_THREADS = max(1, min(16, os.cpu_count() or 1))
# heads h with h // 6 = 0..7: one per XCD share of the output pass at 48
# heads (tile order: heads of a group, then segments, then groups)
XCD_HEADS = (0, 7, 13, 19, 26, 32, 39, 45)


def chunk_rows(chunks, C, T):
    rows = set()
    for j in chunks:
        if 0 <= j * C < T:
            rows.update(range(j * C, min(T, (j + 1) * C)))
    return rows


def boundary_rows(T, C, n_random, seed):
    rows = {0, 1, C - 1, C, C + 1, T - 1, T - C, T // 2, T // 2 - 1}
    k = 1
    while (1 << k) <= T:
        rows.update({(1 << k) - 1, 1 << k, (1 << k) + 1})
        k += 1
    rng = np.random.default_rng(seed)
    rows.update(rng.integers(0, T, size=n_random).tolist())
    return {r for r in rows if 0 <= r < T}


def level_switch_chunks(nc):
    """Chunk indices 0, 1, 2^k - 1, 2^k and the last chunk."""
    js = {0, 1, nc - 1}
    k = 0
    while (1 << k) < nc:
        js.update({(1 << k) - 1, 1 << k})
        k += 1
    return sorted(j for j in js if j < nc)


def streamed_segment_chunks(nc, m):
    """One chunk (first, middle or last in turn) of each segment of 2^m
    chunks whose index has four or more set bits, and every chunk of the
    last such segment."""
    seg = 1 << m
    ns = (nc + seg - 1) // seg
    qs = [q for q in range(ns) if bin(q).count("1") >= 4]
    js = set()
    for i, q in enumerate(qs):
        js.add(q * seg + (0, seg // 2, seg - 1)[i % 3])
    if qs:
        js.update(range(qs[-1] * seg, min(nc, (qs[-1] + 1) * seg)))
    return sorted(j for j in js if j < nc)


def oracle_rows(d, heads, rows):
    """O[0, rows, h, :] of the fp64 oracle for each head, in threads (numpy
    releases the GIL in the heavy operations)."""
    rows = np.array(sorted(rows))
    pieces = [rows[i:i + 96] for i in range(0, rows.size, 96)]
    jobs = [(h, p) for h in heads for p in pieces]

    def run(job):
        h, p = job
        return loglin_ref.loglin_rows(d["X"], d["B"], d["C"], d["log_a"], d["lam"], 0, h, p)

    with threadpool_limits(1), cf.ThreadPoolExecutor(ORACLE_THREADS) as ex:
        res = list(ex.map(run, jobs))
    out = {}
    for (h, _), r in zip(jobs, res):
        out.setdefault(h, []).append(r)
    return rows, {h: np.concatenate(v, axis=0) for h, v in out.items()}


def compare_rows(tag, out, rows, refs):
    """Max relative error per head (max |out - ref| / max |ref| over the
    sampled rows) and the element-wise relative error with a floor of
    1e-3 max |ref|; returns the worst of the former."""
    idx = torch.from_numpy(rows).to(out.device)
    worst = 0.0
    for h, ref in refs.items():
        got = out[0, idx, h, :].float().cpu().numpy().astype(np.float64)
        assert np.isfinite(got).all(), (tag, h)
        scale = np.abs(ref).max()
        err = float(np.abs(got - ref).max() / scale)
        elem = float((np.abs(got - ref) / np.maximum(np.abs(ref), 1e-3 * scale)).max())
        say(f"[full] {tag} head {h}: {len(rows)} rows, max_rel_err={err:.3e} "
            f"elementwise(floor 1e-3)={elem:.3e}")
        worst = max(worst, err)
    return worst


def run_case(name, variant, heads, rows_fn, **kw):
    cfg = inputs.CONFIGS[name]
    say(f"[full] {name} variant={variant}: generating inputs")
    d = inputs.make_inputs(cfg, 0, variant=variant)
    t = to_device(d, cfg)
    say(f"[full] {name} variant={variant}: running loglin_fwd "
        f"(seg_log2={L.loglin_plan_seg_log2(L.dims_of(t['X'], t['B'], t['lam']), cfg.chunk)})")
    out = run_gpu(cfg, t, **kw)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    rows = rows_fn(cfg)
    say(f"[full] {name} variant={variant}: oracle on {len(rows)} rows x {len(heads)} heads")
    rows, refs = oracle_rows(d, heads, rows)
    worst = compare_rows(f"{name}/{variant}", out, rows, refs)
    say(f"[full] {name} variant={variant}: worst max_rel_err={worst:.3e} (tol {BF16_TOL:g})")
    return worst


def stratified_rows(cfg, n_random=16, seed=1):
    T, C = cfg.seqlen, cfg.chunk
    return boundary_rows(T, C, n_random, seed) | chunk_rows(level_switch_chunks(T // C), C, T)


def deep_rows(cfg, n_random=16, seed=2):
    T, C = cfg.seqlen, cfg.chunk
    m = 3  # the library's segment depth at these sizes (checked below)
    return boundary_rows(T, C, n_random, seed) | chunk_rows(streamed_segment_chunks(T // C, m), C, T)


def test_t8k_every_output_all_heads():
    """8K workload: every output of all 48 heads against the full oracle."""
    cfg = inputs.CONFIGS["t8k_bf16"]
    say("[full] t8k_bf16 all heads: generating inputs")
    d = inputs.make_inputs(cfg, 0)
    t = to_device(d, cfg)
    out = run_gpu(cfg, t)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    say(f"[full] t8k_bf16 all heads: full oracle, {cfg.nheads} heads on {ORACLE_THREADS} threads")

    def one(h):
        return loglin_ref.loglin_forward_bh(d["X"], d["B"], d["C"], d["log_a"], d["lam"], 0, h)

    with threadpool_limits(1), cf.ThreadPoolExecutor(ORACLE_THREADS) as ex:
        ref = np.stack(list(ex.map(one, range(cfg.nheads))), axis=1)[None]
    err = max_rel_err(got, ref)
    per_head = np.abs(got - ref).max(axis=(1, 3))[0] / np.abs(ref).max(axis=(1, 3))[0]
    say(f"[full] t8k_bf16 all heads: max_rel_err={err:.3e} (worst head {int(per_head.argmax())}), "
        f"median head {float(np.median(per_head)):.3e}")
    assert np.isfinite(got).all()
    assert err <= BF16_TOL


@pytest.mark.parametrize("name,heads,n_random", [
    ("t32k_bf16", XCD_HEADS, 16),
    ("t131k_bf16", (0, 26, 47), 8),
])
def test_full_size_stratified_rows(name, heads, n_random):
    """Default decay: whole chunks where levels switch, boundary and random
    rows."""
    worst = run_case(name, None, heads, lambda cfg: stratified_rows(cfg, n_random=n_random))
    assert worst <= BF16_TOL


@pytest.mark.parametrize("name,heads", [
    ("t8k_bf16", XCD_HEADS),
    ("t32k_bf16", XCD_HEADS),
])
def test_full_size_slow_decay(name, heads):
    """log a x 1e-3: every level carries weight, including the streamed
    slots (segments with four or more set bits) and the level scan's
    deepest stack entries."""
    cfg = inputs.CONFIGS[name]
    dims = L.make_dims(cfg.batch, cfg.seqlen, cfg.nheads, cfg.ngroups, cfg.headdim, cfg.dstate,
                       cfg.nlevels, L.LOGLIN_BF16)
    assert L.loglin_plan_seg_log2(dims, cfg.chunk) == 3
    worst = run_case(name, "slow_decay", heads, deep_rows)
    assert worst <= BF16_TOL


@pytest.mark.parametrize("level", [12, 13, 14, 15])
def test_t32k_onehot_deep_levels(level):
    """lambda one-hot on each of the four deepest levels at 32K (slow decay,
    so the keys half a sequence back count): each isolates one level above
    the segment, resident or streamed."""
    worst = run_case("t32k_bf16", f"slow_decay+lam_onehot_{level}", XCD_HEADS[::2],
                     lambda cfg: deep_rows(cfg, n_random=8, seed=level))
    say(f"[full] t32k_bf16 one-hot level {level}: max_rel_err={worst:.3e}")
    assert worst <= BF16_TOL


def test_t131k_slow_decay():
    """131K tokens, slow decay: 256 segments, the level scan's stack eight
    deep, levels up to 17."""
    worst = run_case("t131k_bf16", "slow_decay", (0, 47),
                     lambda cfg: boundary_rows(cfg.seqlen, cfg.chunk, 8, 4)
                     | chunk_rows([cfg.seqlen // cfg.chunk - 1], cfg.chunk, cfg.seqlen))
    assert worst <= BF16_TOL


@pytest.mark.parametrize("chunk", [64, 32])
def test_many_segments(chunk):
    """One chunk per segment at 65536 tokens: 1024 (chunk 64) or 2048
    (chunk 32) segments take the level scan's deepest stack instantiation,
    and 2048 also refills its staged segment log-decays past the first
    1024.  Slow decay keeps every level weighted."""
    T = 65536
    cfg = inputs.Config(f"t64k_seg0_c{chunk}", 1, T, 2, 1, 64, 128, chunk, inputs.num_levels(T),
                        "bf16", "mamba2")
    say(f"[full] {cfg.name}: generating inputs")
    d = inputs.make_inputs(cfg, 5, variant="slow_decay")
    t = to_device(d, cfg)
    dims = L.dims_of(t["X"], t["B"], t["lam"])
    assert L.loglin_plan_seg_log2(dims, chunk, seg_log2=0) == 0
    out = run_gpu(cfg, t, seg_log2=0)
    torch.cuda.synchronize()
    rows = boundary_rows(T, chunk, 12, 5) | chunk_rows([T // chunk - 1, 1023, 1024], chunk, T)
    rows, refs = oracle_rows(d, (0, 1), rows)
    worst = compare_rows(cfg.name, out, rows, refs)
    assert worst <= BF16_TOL
