"""ctypes binding of libloglin.so (the C ABI in include/loglin.h).

Argument marshalling only: every step of the forward pass, the backward pass
and the decode step runs in the HIP kernels of the library.  PyTorch supplies device memory and the stream.
There is no fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# LOGLIN_LIB selects another build of the same library (the host-sanitizer
# build the ABI tests run against); by default the in-tree one.
LIB_PATH = os.environ.get("LOGLIN_LIB") or os.path.join(_HERE, "_lib", "libloglin.so")

LOGLIN_F32 = 0
LOGLIN_BF16 = 1
LOGLIN_NUM_STAGES = 3
STAGES = ("chunk_state", "level_scan", "output")

ERRORS = {
    0: "LOGLIN_OK", -1: "LOGLIN_ERR_NULL", -2: "LOGLIN_ERR_DIM",
    -3: "LOGLIN_ERR_CHUNK", -4: "LOGLIN_ERR_SEQ_CHUNK", -5: "LOGLIN_ERR_GROUPS",
    -6: "LOGLIN_ERR_LEVELS", -7: "LOGLIN_ERR_DTYPE", -8: "LOGLIN_ERR_WORKSPACE",
    -9: "LOGLIN_ERR_ALIGN", -10: "LOGLIN_ERR_SHAPE", -11: "LOGLIN_ERR_HIP",
    -12: "LOGLIN_ERR_OPTS", -13: "LOGLIN_ERR_SCRATCH",
}


class loglin_dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("nheads", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64),
                ("nlevels", ctypes.c_int64), ("io_dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class loglin_opts(ctypes.Structure):
    _fields_ = [("seg_log2", ctypes.c_int32), ("heads_per_block", ctypes.c_int32),
                ("stage_events", ctypes.POINTER(ctypes.c_void_p)),
                ("level_mask", ctypes.c_uint64)]


class LoglinError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


_lib = None

EXPORTS = (
    "loglin_workspace_bytes", "loglin_workspace_bytes_ex", "loglin_fwd",
    "loglin_fwd_ex", "loglin_validate", "loglin_strerror",
    "loglin_plan_seg_log2", "loglin_event_create", "loglin_event_destroy",
    "loglin_event_elapsed_ms", "loglin_decode_state_bytes", "loglin_decode_step",
    "loglin_bwd_workspace_bytes", "loglin_bwd", "loglin_gdn_workspace_bytes", "loglin_gdn_fwd",
    "loglin_noalloc_scratch_bytes", "loglin_fwd_noalloc",
)


def lib():
    """Load libloglin.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it first "
            "(python -c 'import __graft_entry__; __graft_entry__.build()')")
    L = ctypes.CDLL(LIB_PATH)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    pd, po = ctypes.POINTER(loglin_dims), ctypes.POINTER(loglin_opts)
    L.loglin_workspace_bytes.argtypes = [pd, i32]
    L.loglin_workspace_bytes.restype = sz
    L.loglin_workspace_bytes_ex.argtypes = [pd, i32, po]
    L.loglin_workspace_bytes_ex.restype = sz
    L.loglin_fwd.argtypes = [vp, vp, vp, vp, vp, i32, vp, pd, vp, sz, vp]
    L.loglin_fwd.restype = i32
    L.loglin_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i32, vp, pd, vp, sz, vp, po]
    L.loglin_fwd_ex.restype = i32
    L.loglin_validate.argtypes = [vp, vp, vp, vp, vp, i32, vp, pd, vp, sz, po]
    L.loglin_validate.restype = i32
    L.loglin_strerror.argtypes = [i32]
    L.loglin_strerror.restype = ctypes.c_char_p
    L.loglin_plan_seg_log2.argtypes = [pd, i32, po]
    L.loglin_plan_seg_log2.restype = i32
    L.loglin_event_create.argtypes = [ctypes.POINTER(vp)]
    L.loglin_event_create.restype = i32
    L.loglin_event_destroy.argtypes = [vp]
    L.loglin_event_destroy.restype = i32
    L.loglin_event_elapsed_ms.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_float)]
    L.loglin_event_elapsed_ms.restype = i32
    L.loglin_decode_state_bytes.argtypes = [pd]
    L.loglin_decode_state_bytes.restype = sz
    L.loglin_decode_step.argtypes = [vp, ctypes.c_int64, vp, vp, vp, vp, vp, vp, pd, vp]
    L.loglin_decode_step.restype = i32
    L.loglin_bwd_workspace_bytes.argtypes = [pd, i32]
    L.loglin_bwd_workspace_bytes.restype = sz
    L.loglin_bwd.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, pd, vp, sz, vp]
    L.loglin_bwd.restype = i32
    L.loglin_gdn_workspace_bytes.argtypes = [pd]
    L.loglin_gdn_workspace_bytes.restype = sz
    L.loglin_gdn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, pd, vp, sz, vp]
    L.loglin_gdn_fwd.restype = i32
    L.loglin_noalloc_scratch_bytes.argtypes = []
    L.loglin_noalloc_scratch_bytes.restype = sz
    L.loglin_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, vp, pd, vp]
    L.loglin_fwd_noalloc.restype = i32
    _lib = L
    return L


def loglin_strerror(code: int) -> str:
    return lib().loglin_strerror(int(code)).decode()


def _check(code: int):
    if code != 0:
        raise LoglinError(code, loglin_strerror(code))


def make_dims(batch, seqlen, nheads, ngroups, headdim, dstate, nlevels, io_dtype):
    return loglin_dims(batch, seqlen, nheads, ngroups, headdim, dstate, nlevels,
                       io_dtype, 0)


def _opts(seg_log2, events, heads_per_block=None, level_mask=None):
    if seg_log2 is None and events is None and heads_per_block is None and level_mask is None:
        return None
    o = loglin_opts()
    o.level_mask = 0 if level_mask is None else int(level_mask)
    o.seg_log2 = -1 if seg_log2 is None else int(seg_log2)
    o.heads_per_block = 0 if heads_per_block is None else int(heads_per_block)
    if events is not None:
        arr = (ctypes.c_void_p * len(events))(*[e.handle for e in events])
        o.stage_events = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
        o._keep = arr
    return o


def dims_of(X, B, lam) -> loglin_dims:
    Bt, T, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    if X.dtype == torch.bfloat16:
        dt = LOGLIN_BF16
    elif X.dtype == torch.float32:
        dt = LOGLIN_F32
    else:
        raise TypeError(f"unsupported dtype {X.dtype}")
    return make_dims(Bt, T, H, G, P, N, lam.shape[3], dt)


def loglin_workspace_bytes(dims: loglin_dims, chunk: int, seg_log2=None) -> int:
    o = _opts(seg_log2, None)
    if o is None:
        return int(lib().loglin_workspace_bytes(ctypes.byref(dims), int(chunk)))
    return int(lib().loglin_workspace_bytes_ex(ctypes.byref(dims), int(chunk), ctypes.byref(o)))


def loglin_plan_seg_log2(dims: loglin_dims, chunk: int, seg_log2=None) -> int:
    o = _opts(seg_log2, None)
    r = lib().loglin_plan_seg_log2(ctypes.byref(dims), int(chunk),
                                   ctypes.byref(o) if o is not None else None)
    _check(r if r < 0 else 0)
    return r


class Event:
    """A hipEvent_t created through the library (timing enabled)."""

    def __init__(self):
        h = ctypes.c_void_p()
        _check(lib().loglin_event_create(ctypes.byref(h)))
        self.handle = h.value

    def elapsed_ms(self, stop: "Event") -> float:
        ms = ctypes.c_float()
        _check(lib().loglin_event_elapsed_ms(self.handle, stop.handle, ctypes.byref(ms)))
        return float(ms.value)

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.loglin_event_destroy(self.handle)
            self.handle = None


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _check_tensor(name, t, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_workspace(need, dev, stream):
    """A uint8 device buffer of `need` bytes for kernels enqueued on
    `stream`, allocated from that stream's pool: once the caller drops it,
    the caching allocator hands the block only to later work on the same
    stream, which runs after those kernels."""
    with torch.cuda.stream(stream):
        return torch.empty(need, dtype=torch.uint8, device=dev)


def loglin_fwd(X, B, C, log_a, lam, chunk, out, *, workspace=None, stream=None,
               seg_log2=None, stage_events=None, heads_per_block=None, level_mask=None):
    """Enqueue O = (C B^T . M^H) X into `out` on `stream` (default: torch's
    current stream).  Tensors: X/out [Bt,T,H,P], B/C [Bt,T,G,N], log_a
    [Bt,T,H] float32, lam [Bt,T,H,L]; X, B, C, lam, out share one dtype
    (bfloat16 or float32), all on one GPU and contiguous.  `workspace` is a
    uint8 device tensor of at least loglin_workspace_bytes bytes (allocated
    here when None).  Returns `out`."""
    dev = X.device
    if dev.type != "cuda":
        raise ValueError("loglin_fwd needs GPU tensors")
    dims = dims_of(X, B, lam)
    io = X.dtype
    Bt, T, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    _check_tensor("X", X, (Bt, T, H, P), io, dev)
    _check_tensor("B", B, (Bt, T, G, N), io, dev)
    _check_tensor("C", C, (Bt, T, G, N), io, dev)
    _check_tensor("log_a", log_a, (Bt, T, H), torch.float32, dev)
    _check_tensor("lam", lam, (Bt, T, H, lam.shape[3]), io, dev)
    _check_tensor("out", out, (Bt, T, H, P), io, dev)
    opts = _opts(seg_log2, stage_events, heads_per_block, level_mask)
    popts = ctypes.byref(opts) if opts is not None else None
    need = int(lib().loglin_workspace_bytes_ex(ctypes.byref(dims), int(chunk), popts))
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    if workspace is None and need > 0:
        workspace = _stream_workspace(need, dev, stream)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    sptr = ctypes.c_void_p(stream.cuda_stream)
    rc = lib().loglin_fwd_ex(_ptr(X), _ptr(B), _ptr(C), _ptr(log_a), _ptr(lam), int(chunk),
                             _ptr(out), ctypes.byref(dims), _ptr(workspace), ws_bytes, sptr,
                             popts)
    _check(rc)
    return out


def loglin_noalloc_scratch_bytes() -> int:
    return int(lib().loglin_noalloc_scratch_bytes())


def loglin_fwd_noalloc(X, B, C, log_a, lam, chunk, out, *, stream=None):
    """loglin_fwd with the library's fixed scratch array as the workspace:
    nothing is allocated on the device, here or in the library.  Same
    tensors as loglin_fwd; `stream` must belong to the current device.
    Returns `out`."""
    dev = X.device
    if dev.type != "cuda":
        raise ValueError("loglin_fwd_noalloc needs GPU tensors")
    dims = dims_of(X, B, lam)
    io = X.dtype
    Bt, T, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    _check_tensor("X", X, (Bt, T, H, P), io, dev)
    _check_tensor("B", B, (Bt, T, G, N), io, dev)
    _check_tensor("C", C, (Bt, T, G, N), io, dev)
    _check_tensor("log_a", log_a, (Bt, T, H), torch.float32, dev)
    _check_tensor("lam", lam, (Bt, T, H, lam.shape[3]), io, dev)
    _check_tensor("out", out, (Bt, T, H, P), io, dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    rc = lib().loglin_fwd_noalloc(_ptr(X), _ptr(B), _ptr(C), _ptr(log_a), _ptr(lam), int(chunk),
                                  _ptr(out), ctypes.byref(dims),
                                  ctypes.c_void_p(stream.cuda_stream))
    _check(rc)
    return out


def decode_dims(X, B, lam, seqlen) -> loglin_dims:
    """Dims of a decode state for tokens X [Bt,H,P], B [Bt,G,N], lam
    [Bt,H,L] and `seqlen` positions."""
    Bt, H, P = X.shape
    G, N = B.shape[1], B.shape[2]
    if X.dtype == torch.bfloat16:
        dt = LOGLIN_BF16
    elif X.dtype == torch.float32:
        dt = LOGLIN_F32
    else:
        raise TypeError(f"unsupported dtype {X.dtype}")
    return make_dims(Bt, seqlen, H, G, P, N, lam.shape[2], dt)


def loglin_decode_state_bytes(dims: loglin_dims) -> int:
    return int(lib().loglin_decode_state_bytes(ctypes.byref(dims)))


def loglin_decode_step(state, t, X, B, C, log_a, lam, out, *, seqlen, stream=None):
    """Enqueue decode step t: advance `state` (a uint8 device tensor of
    loglin_decode_state_bytes bytes, reused across the steps t = 0, 1, ...)
    by token t and write its output to `out`.  Tensors: X/out [Bt,H,P], B/C
    [Bt,G,N], log_a [Bt,H] float32, lam [Bt,H,L]; `seqlen` is the number of
    positions the state was sized for.  Returns `out`."""
    dev = X.device
    if dev.type != "cuda":
        raise ValueError("loglin_decode_step needs GPU tensors")
    dims = decode_dims(X, B, lam, seqlen)
    io = X.dtype
    Bt, H, P = X.shape
    G, N = B.shape[1], B.shape[2]
    _check_tensor("X", X, (Bt, H, P), io, dev)
    _check_tensor("B", B, (Bt, G, N), io, dev)
    _check_tensor("C", C, (Bt, G, N), io, dev)
    _check_tensor("log_a", log_a, (Bt, H), torch.float32, dev)
    _check_tensor("lam", lam, (Bt, H, lam.shape[2]), io, dev)
    _check_tensor("out", out, (Bt, H, P), io, dev)
    need = loglin_decode_state_bytes(dims)
    if state.numel() * state.element_size() < need:
        raise ValueError(f"state holds {state.numel() * state.element_size()} bytes, needs {need}")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    rc = lib().loglin_decode_step(_ptr(state), int(t), _ptr(X), _ptr(B), _ptr(C), _ptr(log_a),
                                  _ptr(lam), _ptr(out), ctypes.byref(dims),
                                  ctypes.c_void_p(stream.cuda_stream))
    _check(rc)
    return out


def loglin_bwd_workspace_bytes(dims: loglin_dims, chunk: int) -> int:
    return int(lib().loglin_bwd_workspace_bytes(ctypes.byref(dims), int(chunk)))


def loglin_bwd(X, B, C, log_a, lam, dO, chunk, dX, dB, dC, dlog_a, dlam, *, workspace=None,
               stream=None):
    """Enqueue the gradients of O = (C B^T . M^H) X for the upstream gradient
    dO [Bt,T,H,P]: dX [Bt,T,H,P], dB and dC [Bt,T,G,N] (summed over each
    group's heads), dlog_a [Bt,T,H] float32 and dlam [Bt,T,H,L] (zero on levels
    the sequence does not reach).  Inputs as for loglin_fwd; dO, dX, dB, dC and
    dlam in the io dtype.  `workspace` is a uint8 device tensor of at least
    loglin_bwd_workspace_bytes bytes (allocated here when None).  Returns
    (dX, dB, dC, dlog_a, dlam)."""
    dev = X.device
    if dev.type != "cuda":
        raise ValueError("loglin_bwd needs GPU tensors")
    dims = dims_of(X, B, lam)
    io = X.dtype
    Bt, T, H, P = X.shape
    G, N = B.shape[2], B.shape[3]
    L = lam.shape[3]
    for name, t, shape, dt in (("X", X, (Bt, T, H, P), io), ("B", B, (Bt, T, G, N), io),
                               ("C", C, (Bt, T, G, N), io),
                               ("log_a", log_a, (Bt, T, H), torch.float32),
                               ("lam", lam, (Bt, T, H, L), io), ("dO", dO, (Bt, T, H, P), io),
                               ("dX", dX, (Bt, T, H, P), io), ("dB", dB, (Bt, T, G, N), io),
                               ("dC", dC, (Bt, T, G, N), io),
                               ("dlog_a", dlog_a, (Bt, T, H), torch.float32),
                               ("dlam", dlam, (Bt, T, H, L), io)):
        _check_tensor(name, t, shape, dt, dev)
    need = loglin_bwd_workspace_bytes(dims, chunk)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    if workspace is None and need > 0:
        workspace = _stream_workspace(need, dev, stream)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().loglin_bwd(_ptr(X), _ptr(B), _ptr(C), _ptr(log_a), _ptr(lam), _ptr(dO), int(chunk),
                          _ptr(dX), _ptr(dB), _ptr(dC), _ptr(dlog_a), _ptr(dlam),
                          ctypes.byref(dims), _ptr(workspace), ws_bytes,
                          ctypes.c_void_p(stream.cuda_stream))
    _check(rc)
    return dX, dB, dC, dlog_a, dlam


def gdn_dims(q, v, lam) -> loglin_dims:
    Bt, T, H, N = q.shape
    if q.dtype == torch.bfloat16:
        dt = LOGLIN_BF16
    elif q.dtype == torch.float32:
        dt = LOGLIN_F32
    else:
        raise TypeError(f"unsupported dtype {q.dtype}")
    return make_dims(Bt, T, H, H, v.shape[3], N, lam.shape[3], dt)


def loglin_gdn_workspace_bytes(dims: loglin_dims) -> int:
    return int(lib().loglin_gdn_workspace_bytes(ctypes.byref(dims)))


def loglin_gdn_fwd(q, k, v, log_alpha, beta, lam, out, *, workspace=None, stream=None):
    """Enqueue the log-linear gated DeltaNet forward into `out` on `stream`.
    Tensors: q, k [Bt,T,H,N], v and out [Bt,T,H,P], log_alpha and beta
    [Bt,T,H] float32, lam [Bt,T,H,L]; q, k, v, lam and out share one dtype
    (bfloat16 or float32), all on one GPU and contiguous.  `workspace` is a
    uint8 device tensor of at least loglin_gdn_workspace_bytes bytes
    (allocated here when None).  Returns `out`."""
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("loglin_gdn_fwd needs GPU tensors")
    Bt, T, H, N = q.shape
    P = v.shape[3]
    L = lam.shape[3]
    io = q.dtype
    if io == torch.bfloat16:
        dt = LOGLIN_BF16
    elif io == torch.float32:
        dt = LOGLIN_F32
    else:
        raise TypeError(f"unsupported dtype {io}")
    for name, t, shape, d in (("q", q, (Bt, T, H, N), io), ("k", k, (Bt, T, H, N), io),
                              ("v", v, (Bt, T, H, P), io),
                              ("log_alpha", log_alpha, (Bt, T, H), torch.float32),
                              ("beta", beta, (Bt, T, H), torch.float32),
                              ("lam", lam, (Bt, T, H, L), io), ("out", out, (Bt, T, H, P), io)):
        _check_tensor(name, t, shape, d, dev)
    dims = make_dims(Bt, T, H, H, P, N, L, dt)
    need = loglin_gdn_workspace_bytes(dims)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    if workspace is None and need > 0:
        workspace = _stream_workspace(need, dev, stream)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().loglin_gdn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(lam),
                              _ptr(out), ctypes.byref(dims), _ptr(workspace), ws_bytes,
                              ctypes.c_void_p(stream.cuda_stream))
    _check(rc)
    return out
