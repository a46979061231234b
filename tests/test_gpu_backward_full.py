"""Backward pass at the full 32K-token workload (48 heads in groups of 2,
P = 64, N = 128, chunk 64, bf16) in the launch configuration the benchmark
times.  The oracle computes sampled gradient entries one by one from one
row or column of the T x T matrices: key positions for dX and dB, query
positions for dC and dlambda (chunk and power-of-two boundaries, the ends,
seeded random positions), and dlog_a at positions near both ends (its
double sum costs (T - r) r there).  Bar: 2e-2 of the largest sampled
reference value per head or group."""
import numpy as np
import pytest
import torch

from oracle import loglin_grad
from ssm_scan_amd import inputs
from ssm_scan_amd import loglin as L

from .gpu_helpers import BF16_TOL, say, to_device
from .test_gpu_full import boundary_rows

pytestmark = pytest.mark.gpu


def rel(got, ref):
    return float(np.abs(np.asarray(got) - ref).max() / np.abs(ref).max())


def test_backward_t32k_sampled():
    cfg = inputs.CONFIGS["t32k_bf16"]
    T, C = cfg.seqlen, cfg.chunk
    say("[bwd-full] generating inputs")
    d = inputs.make_inputs(cfg, 0)
    dOv, dOb = inputs.make_grad_output(cfg, 0)
    t = to_device(d, cfg)
    dO = torch.from_numpy(np.ascontiguousarray(dOb).view(np.int16)).cuda().view(torch.bfloat16)
    g = dict(dX=torch.empty_like(t["X"]), dB=torch.empty_like(t["B"]),
             dC=torch.empty_like(t["C"]), dlog_a=torch.empty_like(t["log_a"]),
             dlam=torch.empty_like(t["lam"]))
    say("[bwd-full] running loglin_bwd")
    L.loglin_bwd(t["X"], t["B"], t["C"], t["log_a"], t["lam"], dO, C, g["dX"], g["dB"], g["dC"],
                 g["dlog_a"], g["dlam"])
    torch.cuda.synchronize()
    for k, v in g.items():
        assert torch.isfinite(v.float()).all(), k
    pos = np.array(sorted(boundary_rows(T, C, 8, seed=32)))
    idx = torch.from_numpy(pos).cuda()
    args = (d["X"], d["B"], d["C"], d["log_a"], d["lam"], dOv, 0)
    worst = {}
    for grp in (0, 15):
        heads = (2 * grp, 2 * grp + 1)
        dB_ref = 0.0
        dC_ref = 0.0
        for h in heads:
            dX, dBh = loglin_grad.grad_key_columns(*args, h, pos)
            dCh, dlam = loglin_grad.grad_query_rows(*args, h, pos)
            dB_ref = dB_ref + dBh
            dC_ref = dC_ref + dCh
            e_x = rel(g["dX"][0, idx, h].float().cpu().numpy(), dX)
            e_l = rel(g["dlam"][0, idx, h].float().cpu().numpy(), dlam)
            say(f"[bwd-full] head {h}: dX {e_x:.3e} dlam {e_l:.3e} ({len(pos)} positions)")
            worst["dX"] = max(worst.get("dX", 0), e_x)
            worst["dlam"] = max(worst.get("dlam", 0), e_l)
        e_b = rel(g["dB"][0, idx, grp].float().cpu().numpy(), dB_ref)
        e_c = rel(g["dC"][0, idx, grp].float().cpu().numpy(), dC_ref)
        say(f"[bwd-full] group {grp}: dB {e_b:.3e} dC {e_c:.3e}")
        worst["dB"] = max(worst.get("dB", 0), e_b)
        worst["dC"] = max(worst.get("dC", 0), e_c)
    rs = [1, 2, C - 1, C, C + 1, T - C - 1, T - C, T - 2, T - 1]
    for h in (0, 31):
        ref = np.array([loglin_grad.grad_log_a_at(*args, h, r) for r in rs])
        got = g["dlog_a"][0, torch.tensor(rs).cuda(), h].cpu().numpy()
        e = rel(got, ref)
        say(f"[bwd-full] head {h}: dlog_a {e:.3e} at {rs}")
        worst["dlog_a"] = max(worst.get("dlog_a", 0), e)
    for k, v in worst.items():
        assert v <= BF16_TOL, (k, v)
