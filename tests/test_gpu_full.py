"""Full-size workloads (8K, 32K, 131K tokens; 48 heads in groups of 2;
P=64, N=128, chunk 64, bf16) in the launch configuration the benchmark
times.  The oracle computes a stratified sample of output rows one by one
from their full causal prefix: rows at chunk and power-of-two boundaries
(every Fenwick level switches there), the last row, and seeded random rows,
for heads covering several B/C groups."""
import numpy as np
import pytest
import torch

from oracle import loglin_ref
from ssm_scan_amd import inputs

from .gpu_helpers import BF16_TOL, run_gpu, say, to_device

pytestmark = pytest.mark.gpu


def sample_rows(T, C, n_random, seed):
    rows = {0, 1, C - 1, C, C + 1, T - 1, T - C, T // 2, T // 2 - 1}
    k = 1
    while (1 << k) <= T:
        rows.update({(1 << k) - 1, min(T - 1, 1 << k)})
        k += 1
    rng = np.random.default_rng(seed)
    rows.update(rng.integers(0, T, size=n_random).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < T))


@pytest.mark.parametrize("name,heads,n_random", [
    ("t8k_bf16", (0, 1, 17, 47), 24),
    ("t32k_bf16", (0, 5, 30, 47), 16),
    ("t131k_bf16", (0, 47), 8),
])
def test_full_size_sampled_rows(name, heads, n_random):
    cfg = inputs.CONFIGS[name]
    say(f"[full] {name}: generating inputs")
    d = inputs.make_inputs(cfg, 0)
    t = to_device(d, cfg)
    say(f"[full] {name}: running loglin_fwd")
    out = run_gpu(cfg, t)
    torch.cuda.synchronize()
    rows = sample_rows(cfg.seqlen, cfg.chunk, n_random, seed=len(name))
    worst = 0.0
    for h in heads:
        ref = loglin_ref.loglin_rows(d["X"], d["B"], d["C"], d["log_a"], d["lam"], 0, h, rows)
        got = out[0, torch.from_numpy(rows).cuda(), h, :].float().cpu().numpy()
        assert np.isfinite(got).all()
        err = float(np.abs(got - ref).max() / np.abs(ref).max())
        say(f"[full] {name} head {h}: {len(rows)} rows, max_rel_err={err:.3e}")
        worst = max(worst, err)
    assert worst <= BF16_TOL
    o = out.float()
    assert torch.isfinite(o).all()
