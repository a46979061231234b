"""One-token decode steps (Fenwick recurrence) on the GPU vs the fp64
oracle: step t must return row t of the dense definition, for every t of a
sequence, through the C ABI.  Same bars as the forward: max relative error
<= 2e-2 for bf16 inputs, <= 1e-4 for fp32."""
import numpy as np
import pytest
import torch

from oracle import loglin_ref
from ssm_scan_amd import inputs
from ssm_scan_amd import loglin as L

from .gpu_helpers import max_rel_err, run_gpu, say, small_cfg, to_device, tol_of

pytestmark = pytest.mark.gpu


def run_decode(t, cfg, state=None, seqlen=None):
    """All T steps of one sequence; returns [Bt, T, H, P] on the host."""
    Bt, T = t["X"].shape[:2]
    seqlen = seqlen or T
    dims = L.decode_dims(t["X"][:, 0], t["B"][:, 0], t["lam"][:, 0], seqlen)
    if state is None:
        state = torch.empty(L.loglin_decode_state_bytes(dims), dtype=torch.uint8, device="cuda")
    outs = []
    for s in range(T):
        tok = {k: t[k][:, s].contiguous() for k in ("X", "B", "C", "log_a", "lam")}
        o = torch.empty_like(tok["X"])
        L.loglin_decode_step(state, s, tok["X"], tok["B"], tok["C"], tok["log_a"], tok["lam"], o,
                             seqlen=seqlen)
        outs.append(o)
    torch.cuda.synchronize()
    return torch.stack(outs, dim=1).float().cpu().numpy(), state


def check_decode(cfg, seed=0, variant=None):
    say(f"[decode] {cfg.name} seed={seed} variant={variant}")
    d = inputs.make_inputs(cfg, seed, variant=variant)
    t = to_device(d, cfg)
    got, _ = run_decode(t, cfg)
    ref = loglin_ref.loglin_forward(d["X"], d["B"], d["C"], d["log_a"], d["lam"])
    err = max_rel_err(got, ref)
    say(f"         max_rel_err={err:.3e} (tol {tol_of(cfg):.0e})")
    assert np.isfinite(got).all()
    assert err <= tol_of(cfg), err
    return got, ref, t


def test_decode_tiny_fp32():
    """256 tokens, 1 head, P=N=16, fp32 (1e-4 bar)."""
    check_decode(inputs.CONFIGS["tiny_fp32"])


@pytest.mark.parametrize("T", [1, 2, 7, 64, 300])
def test_decode_headline_shape(T):
    """Headline head shape (P=64, N=128, groups of 2), bf16; ragged lengths."""
    check_decode(small_cfg(T=T, H=4, G=2))


@pytest.mark.parametrize("dtype,P,N", [("bf16", 16, 32), ("bf16", 32, 64), ("bf16", 64, 32),
                                       ("fp32", 64, 128), ("fp32", 32, 16)])
def test_decode_shapes(dtype, P, N):
    check_decode(small_cfg(dtype=dtype, T=200, H=2, G=1, P=P, N=N, C=16, decay="softplus"))


@pytest.mark.parametrize("variant", ["slow_decay", "no_decay", "lam_onehot_0", "lam_onehot_3",
                                     "lam_onehot_8"])
def test_decode_variants(variant):
    """Slow / no decay reach the old buckets; one-hot lambda isolates a level."""
    check_decode(small_cfg(T=300, H=2, G=1), variant=variant)


@pytest.mark.parametrize("variant", ["slow_decay", "slow_decay+lam_onehot_10"])
def test_decode_long_context(variant):
    """2100 steps: buckets up to level 12 occupied, with weight (slow decay),
    and a deep level alone (one-hot level weights)."""
    check_decode(small_cfg(T=2100, H=2, G=1), variant=variant)


def test_decode_batch_and_matches_forward():
    """Batch of 3; the decode outputs agree with the chunked forward's."""
    cfg = small_cfg(T=256, H=4, G=2, Bt=3)
    got, ref, t = check_decode(cfg, variant="slow_decay")
    fwd = run_gpu(cfg, t).float().cpu().numpy()
    assert max_rel_err(fwd, ref) <= tol_of(cfg)
    assert max_rel_err(got, fwd) <= 2 * tol_of(cfg)


def test_decode_state_reuse():
    """A state buffer reused for a second sequence needs no clearing: step 0
    re-initialises it."""
    cfg = small_cfg(T=130, H=2, G=1)
    d1 = inputs.make_inputs(cfg, 1, variant="no_decay")
    d2 = inputs.make_inputs(cfg, 2)
    t1, t2 = to_device(d1, cfg), to_device(d2, cfg)
    _, state = run_decode(t1, cfg)
    got, _ = run_decode(t2, cfg, state=state)
    fresh, _ = run_decode(t2, cfg)
    assert np.array_equal(got, fresh)
    ref = loglin_ref.loglin_forward(d2["X"], d2["B"], d2["C"], d2["log_a"], d2["lam"])
    assert max_rel_err(got, ref) <= tol_of(cfg)


def test_decode_longer_state_than_sequence():
    """A state sized for more positions (more levels) than the tokens fed."""
    cfg = small_cfg(T=100, H=2, G=1)
    d = inputs.make_inputs(cfg, 0)
    t = to_device(d, cfg)
    lam2 = torch.cat([t["lam"], torch.zeros_like(t["lam"][..., :4])], dim=-1).contiguous()
    t2 = dict(t, lam=lam2)
    got, _ = run_decode(t2, cfg, seqlen=1500)
    ref = loglin_ref.loglin_forward(d["X"], d["B"], d["C"], d["log_a"], d["lam"])
    assert max_rel_err(got, ref) <= tol_of(cfg)
