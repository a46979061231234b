"""The binding's own workspaces on a side stream.

When the caller passes no workspace, the binding allocates one for the
kernels it enqueues on the caller's stream and drops it on return.  These
tests enqueue the forward, the backward and the gated DeltaNet forward on a
side stream held back by a sleep, then allocate and fill buffers of the
workspace's size on torch's current stream while those kernels wait.  A
workspace taken from the current stream's pool would be handed to the
fills and overwritten before the kernels read it; the results must instead
match, bit for bit, a run on the current stream with a workspace of its
own (every kernel is deterministic).
"""
import numpy as np
import pytest
import torch

from ssm_scan_amd import inputs
from ssm_scan_amd import loglin as L

from .gpu_helpers import say, small_cfg, to_device

pytestmark = pytest.mark.gpu


def _scribble(nbytes, rounds=4):
    """Allocate and fill buffers of `nbytes` on the current stream."""
    keep = []
    for _ in range(rounds):
        b = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        b.fill_(0xFF)  # NaN in every float view
        keep.append(b)
    return keep


def _side_run(fn, nbytes):
    cur = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(cur)
    with torch.cuda.stream(side):
        torch.cuda._sleep(20_000_000)  # hold the side stream's kernels back
    res = fn(side)
    junk = _scribble(nbytes)
    cur.wait_stream(side)
    torch.cuda.synchronize()
    del junk
    return res


def test_forward_side_stream_workspace():
    cfg = small_cfg(T=2048, H=4, G=2)
    d = inputs.make_inputs(cfg, 0)
    t = to_device(d, cfg)
    dims = L.dims_of(t["X"], t["B"], t["lam"])
    need = L.loglin_workspace_bytes(dims, cfg.chunk)
    say(f"[streams] forward {cfg.name}: workspace {need} bytes")
    assert need > 0
    ref = torch.empty_like(t["X"])
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    L.loglin_fwd(t["X"], t["B"], t["C"], t["log_a"], t["lam"], cfg.chunk, ref, workspace=ws)
    torch.cuda.synchronize()

    def fn(side):
        out = torch.empty_like(t["X"])
        L.loglin_fwd(t["X"], t["B"], t["C"], t["log_a"], t["lam"], cfg.chunk, out, stream=side)
        return out

    out = _side_run(fn, need)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_backward_side_stream_workspace():
    cfg = small_cfg(T=1024, H=4, G=2)
    d = inputs.make_inputs(cfg, 0)
    t = to_device(d, cfg)
    _, bits = inputs.make_grad_output(cfg, 0)
    dO = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)
    dims = L.dims_of(t["X"], t["B"], t["lam"])
    need = L.loglin_bwd_workspace_bytes(dims, cfg.chunk)
    say(f"[streams] backward {cfg.name}: workspace {need} bytes")

    def grads():
        return dict(dX=torch.empty_like(t["X"]), dB=torch.empty_like(t["B"]),
                    dC=torch.empty_like(t["C"]), dlog_a=torch.empty_like(t["log_a"]),
                    dlam=torch.empty_like(t["lam"]))

    ref = grads()
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    L.loglin_bwd(t["X"], t["B"], t["C"], t["log_a"], t["lam"], dO, cfg.chunk, ref["dX"],
                 ref["dB"], ref["dC"], ref["dlog_a"], ref["dlam"], workspace=ws)
    torch.cuda.synchronize()

    def fn(side):
        g = grads()
        L.loglin_bwd(t["X"], t["B"], t["C"], t["log_a"], t["lam"], dO, cfg.chunk, g["dX"],
                     g["dB"], g["dC"], g["dlog_a"], g["dlam"], stream=side)
        return g

    got = _side_run(fn, need)
    for k in ref:
        a, b = got[k], ref[k]
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), k


def test_gdn_side_stream_workspace():
    cfg = inputs.Config("gdn_streams", 1, 512, 2, 2, 64, 128, 32, inputs.num_levels(512), "bf16",
                        "mamba2")
    d = inputs.make_gdn_inputs(cfg, 0)
    t = {}
    for k in ("q", "k", "v", "lam"):
        t[k] = torch.from_numpy(np.ascontiguousarray(d["bits"][k]).view(np.int16)).cuda().view(
            torch.bfloat16)
    t["log_alpha"] = torch.from_numpy(d["log_alpha"]).cuda()
    t["beta"] = torch.from_numpy(d["beta"]).cuda()
    need = L.loglin_gdn_workspace_bytes(L.gdn_dims(t["q"], t["v"], t["lam"]))
    say(f"[streams] gated DeltaNet {cfg.name}: workspace {need} bytes")
    ref = torch.empty_like(t["v"])
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    L.loglin_gdn_fwd(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], t["lam"], ref, workspace=ws)
    torch.cuda.synchronize()

    def fn(side):
        out = torch.empty_like(t["v"])
        L.loglin_gdn_fwd(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], t["lam"], out,
                         stream=side)
        return out

    out = _side_run(fn, need)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
