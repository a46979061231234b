"""C ABI of libloglin.so on the CPU: the library loads, exports every
function include/loglin.h declares, and every argument check fires on the
host.  No test here reaches a HIP call: each call is invalid on purpose and
the library validates before touching the device, or only plans."""
import ctypes
import os
import re

import pytest

from ssm_scan_amd import loglin as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "loglin.h")

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH),
                                reason="libloglin.so not built")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(loglin_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported():
    names = header_functions()
    assert "loglin_fwd" in names and "loglin_workspace_bytes" in names
    lib = L.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.EXPORTS)


def good_dims(**kw):
    d = dict(batch=1, seqlen=32768, nheads=48, ngroups=24, headdim=64, dstate=128,
             nlevels=16, io_dtype=L.LOGLIN_BF16)
    d.update(kw)
    return L.make_dims(**d)


FAKE = 1 << 20  # aligned, never dereferenced: every call below fails validation


def validate(dims, chunk=64, ws_bytes=None, ptrs=None, opts=None, ws=FAKE):
    p = dict(X=FAKE, B=FAKE, C=FAKE, log_a=FAKE, lam=FAKE, out=FAKE)
    p.update(ptrs or {})
    need = L.loglin_workspace_bytes(dims, chunk) if ws_bytes is None else ws_bytes
    o = ctypes.byref(opts) if opts is not None else None
    return L.lib().loglin_validate(p["X"], p["B"], p["C"], p["log_a"], p["lam"], chunk,
                                   p["out"], ctypes.byref(dims), ws, need, o)


def test_valid_arguments_pass_validation():
    assert validate(good_dims()) == 0
    assert validate(good_dims(io_dtype=L.LOGLIN_F32, seqlen=256, nheads=1, ngroups=1,
                              headdim=16, dstate=16, nlevels=9), chunk=16) == 0


@pytest.mark.parametrize("kw,chunk,code", [
    (dict(batch=0), 64, -2), (dict(seqlen=-64), 64, -2), (dict(nheads=0), 64, -2),
    (dict(headdim=0), 64, -2), (dict(nlevels=0), 64, -2),
    (dict(), 48, -3), (dict(), 128, -3), (dict(), 0, -3),
    (dict(seqlen=32768 + 16), 64, -4),
    (dict(ngroups=5), 64, -5),
    (dict(nlevels=15), 64, -6),
    (dict(io_dtype=7), 64, -7),
    (dict(headdim=48), 64, -10), (dict(dstate=96), 64, -10),
    (dict(dstate=16), 64, -10),
    # upper bounds the kernels' 24- and 32-bit offset arithmetic relies on
    (dict(nheads=8192, ngroups=4096), 64, -2), (dict(nlevels=65), 64, -2),
    (dict(batch=2048), 64, -2),
])
def test_dimension_errors(kw, chunk, code):
    assert validate(good_dims(**kw), chunk=chunk, ws_bytes=1 << 40) == code
    assert L.loglin_strerror(code) != "unknown error code"


@pytest.mark.parametrize("name", ["X", "B", "C", "log_a", "lam", "out"])
def test_null_and_misaligned_pointers(name):
    assert validate(good_dims(), ptrs={name: None}) == -1
    assert validate(good_dims(), ptrs={name: FAKE + 8}) == -9


def test_workspace_errors():
    d = good_dims()
    need = L.loglin_workspace_bytes(d, 64)
    assert need > 0
    assert validate(d, ws_bytes=need - 1) == -8
    assert validate(d, ws=None) == -8
    assert validate(d, ws=FAKE + 16) == -9


def test_options_errors():
    o = L.loglin_opts()
    o.seg_log2, o.heads_per_block = -2, 0
    assert validate(good_dims(), opts=o) == -12
    o.seg_log2, o.heads_per_block = 0, 3
    assert validate(good_dims(), opts=o) == -12
    o.seg_log2, o.heads_per_block = 4, 0  # deeper than the on-chip stack
    assert validate(good_dims(), opts=o) == -12
    o.seg_log2 = 2  # deeper than log2 of the chunk count (2 chunks)
    assert validate(good_dims(seqlen=128, nlevels=8), opts=o) == -12
    o.seg_log2 = 1
    assert validate(good_dims(seqlen=128, nlevels=8), opts=o) == 0


@pytest.mark.parametrize("kw,ok", [
    (dict(), True), (dict(ngroups=48), False), (dict(ngroups=16), False),
    (dict(ngroups=12), True), (dict(headdim=32), False),
    (dict(io_dtype=L.LOGLIN_F32), False),
])
def test_head_pairs_option(kw, ok):
    """Two heads per work-group need bf16, 64 columns and an even number of
    heads per group; one head is always accepted."""
    o = L.loglin_opts()
    o.seg_log2 = -1
    for hp in (0, 1):
        o.heads_per_block = hp
        assert validate(good_dims(**kw), opts=o) == 0
    o.heads_per_block = 2
    assert validate(good_dims(**kw), opts=o) == (0 if ok else -12)


def test_null_dims():
    assert L.lib().loglin_validate(FAKE, FAKE, FAKE, FAKE, FAKE, 64, FAKE, None, FAKE,
                                   1 << 40, None) == -1
    assert L.lib().loglin_workspace_bytes(None, 64) == 0


def test_fwd_rejects_before_any_device_call():
    """loglin_fwd runs the same checks first: an invalid call returns its
    code without a HIP call (this container has no GPU)."""
    d = good_dims(nlevels=3)
    rc = L.lib().loglin_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, 64, FAKE, ctypes.byref(d),
                            FAKE, 1 << 40, None)
    assert rc == -6


def test_workspace_size_formula():
    """Workspace: io-typed segment states and slots per (batch, head,
    segment), plus small decay arrays; zero when there is a single chunk."""
    d = good_dims()
    assert L.loglin_plan_seg_log2(d, 64) == 3
    for seg in (None, 0, 1, 2, 3):
        m = 3 if seg is None else seg
        need = L.loglin_workspace_bytes(d, 64, seg)
        ns = 32768 // 64 >> m
        core = 48 * ns * 64 * 128 * (2 + 2)
        assert core <= need <= core + 48 * ns * 4 * 32 + 4 * 256, (seg, need, core)
    # one chunk, or one segment: no level above a segment, no workspace
    assert L.loglin_workspace_bytes(good_dims(seqlen=64, nlevels=7), 64) == 0
    assert L.loglin_workspace_bytes(good_dims(seqlen=512, nlevels=10), 64) == 0
    assert L.loglin_workspace_bytes(good_dims(seqlen=512, nlevels=10), 64, 0) > 0
    assert L.loglin_plan_seg_log2(good_dims(seqlen=128, nlevels=8), 64) == 1


def test_strerror_all_codes():
    for code in L.ERRORS:
        assert isinstance(L.loglin_strerror(code), str)
        assert L.loglin_strerror(code) != "unknown error code", code
    assert L.loglin_strerror(-99) == "unknown error code"


def test_noalloc_host_checks():
    """loglin_fwd_noalloc validates on the host before its first HIP call:
    argument errors as for loglin_fwd, and LOGLIN_ERR_SCRATCH for a problem
    whose workspace exceeds the fixed array (the 32K-token, 48-head
    workload fits)."""
    lib = L.lib()
    cap = lib.loglin_noalloc_scratch_bytes()
    assert cap == 192 << 20
    assert L.loglin_workspace_bytes(good_dims(), 64) <= cap
    big = good_dims(seqlen=131072, nlevels=18, nheads=96, ngroups=48)
    assert L.loglin_workspace_bytes(big, 64) > cap

    def call(d, chunk=64, **ptrs):
        p = dict(X=FAKE, B=FAKE, C=FAKE, log_a=FAKE, lam=FAKE, out=FAKE)
        p.update(ptrs)
        return lib.loglin_fwd_noalloc(p["X"], p["B"], p["C"], p["log_a"], p["lam"], chunk,
                                      p["out"], ctypes.byref(d), None)

    assert call(big) == -13
    assert call(good_dims(nlevels=3)) == -6
    assert call(good_dims(), chunk=48) == -3
    assert call(good_dims(), X=None) == -1
    assert call(good_dims(), out=FAKE + 8) == -9
    assert lib.loglin_fwd_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, 64, FAKE, None, None) == -1


def decode_dims(**kw):
    d = dict(batch=1, seqlen=32768, nheads=48, ngroups=24, headdim=64, dstate=128,
             nlevels=16, io_dtype=L.LOGLIN_BF16)
    d.update(kw)
    return L.make_dims(**d)


def test_decode_state_bytes_formula():
    """Level states fp32 [B,H,LL,N,P] then two banks of decay factors
    [B,H,2,LL], each 256-byte aligned; LL = ceil(log2 seqlen) + 1."""
    d = decode_dims()
    need = L.loglin_decode_state_bytes(d)
    core = 48 * 16 * 128 * 64 * 4
    assert core + 48 * 2 * 16 * 4 <= need <= core + 48 * 2 * 16 * 4 + 512
    assert L.loglin_decode_state_bytes(decode_dims(seqlen=1, nlevels=1)) > 0
    assert L.loglin_decode_state_bytes(decode_dims(nlevels=15)) == 0
    assert L.lib().loglin_decode_state_bytes(None) == 0


def decode_step(dims, t=0, state=1 << 20, ptrs=None):
    p = dict(X=FAKE, B=FAKE, C=FAKE, log_a=FAKE, lam=FAKE, out=FAKE)
    p.update(ptrs or {})
    return L.lib().loglin_decode_step(state, t, p["X"], p["B"], p["C"], p["log_a"], p["lam"],
                                      p["out"], ctypes.byref(dims), None)


@pytest.mark.parametrize("kw,t,code", [
    (dict(), -1, -2), (dict(), 32768, -2), (dict(batch=0), 0, -2),
    (dict(nlevels=15), 0, -6), (dict(ngroups=5), 0, -5), (dict(io_dtype=9), 0, -7),
    (dict(headdim=48), 0, -10),
])
def test_decode_step_errors(kw, t, code):
    """Invalid decode steps fail on the host, before any HIP call."""
    assert decode_step(decode_dims(**kw), t=t) == code


@pytest.mark.parametrize("name", ["X", "B", "C", "log_a", "lam", "out"])
def test_decode_null_and_misaligned(name):
    assert decode_step(decode_dims(), ptrs={name: None}) == -1
    assert decode_step(decode_dims(), ptrs={name: FAKE + 1}) == -9
    if name == "out":
        assert decode_step(decode_dims(), ptrs={name: FAKE + 4}) == -9
    assert decode_step(decode_dims(), state=None) == -1
    assert decode_step(decode_dims(), state=FAKE + 64) == -9


def test_gdn_argument_errors():
    """loglin_gdn_fwd rejects bad dims on the host (no GPU needed)."""
    import ctypes
    lib = L.lib()
    fake = ctypes.c_void_p(0x10000)
    def call(dims, ptr=fake, ws=fake, nbytes=1 << 40):
        return lib.loglin_gdn_fwd(ptr, ptr, ptr, ptr, ptr, ptr, ptr, ctypes.byref(dims), ws, nbytes,
                                  None)
    ok = L.make_dims(1, 64, 2, 2, 64, 128, 7, L.LOGLIN_BF16)
    assert call(L.make_dims(1, 64, 2, 1, 64, 128, 7, L.LOGLIN_BF16)) == -5  # ngroups != nheads
    assert call(L.make_dims(1, 48, 2, 2, 64, 128, 7, L.LOGLIN_BF16)) == -4  # T % 32
    assert call(L.make_dims(1, 64, 2, 2, 64, 128, 6, L.LOGLIN_BF16)) == -6  # too few levels
    assert call(L.make_dims(1, 64, 2, 2, 48, 128, 7, L.LOGLIN_BF16)) == -10  # headdim
    assert call(L.make_dims(1, 64, 2, 2, 64, 96, 7, L.LOGLIN_BF16)) == -10  # dstate
    assert call(L.make_dims(1, 64, 2, 2, 64, 128, 7, 5)) == -7  # dtype
    assert call(ok, ptr=None) == -1
    assert call(ok, ptr=ctypes.c_void_p(0x10004)) == -9  # alignment
    need = lib.loglin_gdn_workspace_bytes(ctypes.byref(ok))
    # 4 (head, chunk) items: Qe and W 32 x 128, U and intra outputs 32 x 64,
    # 32 decay ratios, one total decay; fp32, each region 256-byte aligned
    assert need == 2 * 4 * 32 * 128 * 4 + 2 * 4 * 32 * 64 * 4 + 4 * 32 * 4 + 256
    assert call(ok, ws=None) == -8
    assert call(ok, nbytes=need - 1) == -8
    assert call(ok, ws=ctypes.c_void_p(0x10010)) == -9  # workspace alignment
    assert lib.loglin_gdn_workspace_bytes(ctypes.byref(L.make_dims(1, 48, 2, 2, 64, 128, 7, 1))) == 0


def test_seqlen_upper_bound():
    """The header's size bounds, shared by the forward and the backward:
    seqlen <= 2^30 and at most 2^16 segments of 8 chunks (2^19 chunks).  The
    largest valid length plans a workspace; one chunk more is
    LOGLIN_ERR_DIM before any device call, as is a length past 2^30."""
    lim = 64 << 19
    ok = good_dims(seqlen=lim, nheads=1, ngroups=1, nlevels=26)
    for bad in (good_dims(seqlen=lim + 64, nheads=1, ngroups=1, nlevels=27),
                good_dims(seqlen=(1 << 30) + 64, nheads=1, ngroups=1, nlevels=32)):
        assert validate(bad, ws_bytes=1 << 62) == -2
        assert L.lib().loglin_bwd_workspace_bytes(ctypes.byref(bad), 64) == 0
        rc = L.lib().loglin_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, FAKE, FAKE, FAKE, FAKE,
                                FAKE, ctypes.byref(bad), FAKE, 1 << 62, None)
        assert rc == -2
    assert validate(ok, ws_bytes=1 << 62) == 0
    assert L.lib().loglin_bwd_workspace_bytes(ctypes.byref(ok), 64) > 0
