"""loglin_fwd_noalloc (the forward with the library's fixed scratch array
as its workspace, for callers that cannot allocate) against loglin_fwd with
a workspace of the caller's, through the C ABI: the same kernels, so the
outputs must be bit-identical.  Two calls in a row, the second smaller:
the array keeps the first call's contents, which the forward never reads.
The host-side rejection of problems too large for the array, and that the
32K-token workload fits, are tested on the CPU in test_abi.py."""
import pytest
import torch

from ssm_scan_amd import inputs
from ssm_scan_amd import loglin as L

from .gpu_helpers import max_rel_err, say, small_cfg, to_device

pytestmark = pytest.mark.gpu


def _with_workspace(cfg, t):
    dims = L.dims_of(t["X"], t["B"], t["lam"])
    ws = torch.empty(max(1, L.loglin_workspace_bytes(dims, cfg.chunk)), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(t["X"])
    L.loglin_fwd(t["X"], t["B"], t["C"], t["log_a"], t["lam"], cfg.chunk, out, workspace=ws)
    return out


def _noalloc(cfg, t):
    out = torch.empty_like(t["X"])
    L.loglin_fwd_noalloc(t["X"], t["B"], t["C"], t["log_a"], t["lam"], cfg.chunk, out)
    return out


def test_noalloc_matches_fwd_two_calls():
    big = small_cfg(T=8192, H=8, G=4)
    small = small_cfg(T=1344, H=2, G=1)
    for cfg, seed in ((big, 0), (small, 1)):
        d = inputs.make_inputs(cfg, seed, variant="slow_decay")
        t = to_device(d, cfg)
        dims = L.dims_of(t["X"], t["B"], t["lam"])
        need = L.loglin_workspace_bytes(dims, cfg.chunk)
        say(f"[noalloc] {cfg.name}: workspace {need} of {L.loglin_noalloc_scratch_bytes()} bytes")
        assert 0 < need <= L.loglin_noalloc_scratch_bytes()
        ref = _with_workspace(cfg, t)
        got = _noalloc(cfg, t)
        torch.cuda.synchronize()
        assert torch.isfinite(got.float()).all()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), max_rel_err(
            got.float().cpu().numpy(), ref.float().cpu().numpy())
