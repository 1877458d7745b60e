"""ctypes binding of libnaju.so (argument marshalling only).

Every step of the computation runs in the HIP kernels of ``libnaju.so``;
this module checks tensor shapes/dtypes, allocates outputs and the
workspace with PyTorch, and passes raw device pointers plus the current
HIP stream through the C ABI declared in ``include/naju.h``.  If the
library is missing the import of any entry point raises -- there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnaju.so")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = range(5)
F32, BF16 = 0, 1
OP_SCAN_FWD, OP_SCAN_BWD, OP_BLOCK_FWD, OP_BLOCK_BWD = range(4)
D_CONV = 4

# every function the header declares (the CPU tests check the exports)
EXPORTS = ("naju_workspace_bytes", "naju_ckpt_bytes", "naju_workspace_init",
           "naju_workspace_check", "naju_scan_fwd", "naju_scan_bwd", "naju_block_fwd",
           "naju_block_bwd", "naju_scan_step", "naju_block_step", "naju_mixer_workspace_bytes",
           "naju_mixer_fwd", "naju_mixer_bwd_workspace_bytes", "naju_mixer_bwd",
           "naju_scan_fwd_noalloc", "naju_last_error", "naju_version")


class NajuError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("naju status %d: %s" % (status, msg))
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("d_inner", ctypes.c_int64), ("d_state", ctypes.c_int64),
                ("d_conv", ctypes.c_int32), ("io", ctypes.c_int32)]


_lib = None
_lock = threading.Lock()


def lib() -> ctypes.CDLL:
    """Loads libnaju.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise ImportError("libnaju.so not found at %s; build it with "
                              "`python -m selective_state_space_naju_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, st = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        dp = ctypes.POINTER(Dims)
        L.naju_workspace_bytes.argtypes = [ctypes.c_int, dp]
        L.naju_workspace_bytes.restype = sz
        L.naju_ckpt_bytes.argtypes = [dp]
        L.naju_ckpt_bytes.restype = sz
        L.naju_workspace_init.argtypes = [vp, sz, vp]
        L.naju_workspace_init.restype = st
        L.naju_workspace_check.argtypes = [vp, sz, vp, ctypes.POINTER(ctypes.c_uint32)]
        L.naju_workspace_check.restype = st
        L.naju_scan_fwd.argtypes = [dp] + [vp] * 11 + [sz, vp]
        L.naju_scan_fwd.restype = st
        L.naju_block_fwd.argtypes = [dp] + [vp] * 15 + [sz, vp]
        L.naju_block_fwd.restype = st
        L.naju_scan_bwd.argtypes = [dp] + [vp] * 18 + [sz, vp]
        L.naju_scan_bwd.restype = st
        L.naju_block_bwd.argtypes = [dp] + [vp] * 24 + [sz, vp]
        L.naju_block_bwd.restype = st
        L.naju_scan_step.argtypes = [dp] + [vp] * 9
        L.naju_scan_step.restype = st
        L.naju_block_step.argtypes = [dp] + [vp] * 12
        L.naju_block_step.restype = st
        L.naju_mixer_workspace_bytes.argtypes = [dp, ctypes.c_int64]
        L.naju_mixer_workspace_bytes.restype = sz
        L.naju_mixer_fwd.argtypes = [dp, ctypes.c_int64] + [vp] * 16 + [sz, vp]
        L.naju_mixer_fwd.restype = st
        L.naju_mixer_bwd_workspace_bytes.argtypes = [dp, ctypes.c_int64]
        L.naju_mixer_bwd_workspace_bytes.restype = sz
        L.naju_mixer_bwd.argtypes = [dp, ctypes.c_int64] + [vp] * 28 + [sz, vp, sz, vp]
        L.naju_mixer_bwd.restype = st
        L.naju_scan_fwd_noalloc.argtypes = [dp] + [vp] * 12
        L.naju_scan_fwd_noalloc.restype = st
        L.naju_last_error.argtypes = []
        L.naju_last_error.restype = ctypes.c_char_p
        L.naju_version.argtypes = []
        L.naju_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def last_error() -> str:
    return lib().naju_last_error().decode()


def check(status: int) -> None:
    if status != OK:
        raise NajuError(status, last_error())


def check_workspace(ws) -> None:
    """Raises if a cross-workgroup wait of a call that used `ws` gave up (its
    results are then invalid).  Synchronises the workspace's device."""
    flags = ws.error_flags()
    if flags:
        raise NajuError(EHIP, "a cross-workgroup wait gave up (workspace error flags 0x%x): "
                              "results invalid" % flags)


def make_dims(batch, seqlen, d_inner, d_state, io, d_conv=D_CONV) -> Dims:
    return Dims(int(batch), int(seqlen), int(d_inner), int(d_state), int(d_conv), int(io))


def workspace_bytes(op: int, dims: Dims) -> int:
    return int(lib().naju_workspace_bytes(op, ctypes.byref(dims)))


def ckpt_bytes(dims: Dims) -> int:
    return int(lib().naju_ckpt_bytes(ctypes.byref(dims)))


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def stream_handle(device=None):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


class Workspace:
    """A zero-initialised device workspace (reused across calls on one stream)."""

    def __init__(self, nbytes: int, device):
        n = max(256, (int(nbytes) + 255) // 256 * 256)
        self.tensor = torch.zeros(n, dtype=torch.uint8, device=device)
        self.nbytes = n

    @property
    def ptr(self):
        return ctypes.c_void_p(self.tensor.data_ptr())

    def error_flags(self) -> int:
        out = ctypes.c_uint32(0)
        check(lib().naju_workspace_check(self.ptr, self.nbytes, stream_handle(self.tensor.device),
                                         ctypes.byref(out)))
        return int(out.value)


_ws_cache: dict = {}


def workspace(op: int, dims: Dims, device) -> Workspace:
    """Cached workspace per (device, stream, op, dims): a workspace is only ever
    reused by calls with the same layout, on one stream."""
    dev = torch.device(device)
    key = (dev.index, torch.cuda.current_stream(dev).cuda_stream, op, dims.batch, dims.seqlen,
           dims.d_inner, dims.d_state, dims.d_conv, dims.io)
    ws = _ws_cache.get(key)
    if ws is None:
        ws = Workspace(workspace_bytes(op, dims), dev)
        _ws_cache[key] = ws
    return ws


def _io_of(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("activations must be float32 or bfloat16, got %s" % t.dtype)


def _req(t, name, shape, dtype, device):
    if t is None:
        raise ValueError("%s is required" % name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s: expected shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if t.dtype != dtype:
        raise TypeError("%s: expected %s, got %s" % (name, dtype, t.dtype))
    if t.device != device:
        raise ValueError("%s must be on %s" % (name, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _opt(t, name, shape, dtype, device):
    return None if t is None else _req(t, name, shape, dtype, device)


# ------------------------------------------------------------------ entry points
def scan_fwd(h, a, b, B, C, D, x0=None, *, return_ckpt=False, ws=None, check_errors=False):
    """y, x_final (, ckpt) = naju_scan_fwd(h, a, b, B, C, D, x0).

    check_errors=True synchronises and raises if a look-back wait gave up (the
    library sets an error bit in the workspace instead of hanging)."""
    Bt, L, Di = h.shape
    N = B.shape[-1]
    dt, dev = h.dtype, h.device
    io = _io_of(h)
    for nm, t in (("h", h), ("a", a), ("b", b)):
        _req(t, nm, (Bt, L, Di), dt, dev)
    _req(B, "B", (Bt, L, N), dt, dev)
    _req(C, "C", (Bt, L, N), dt, dev)
    _req(D, "D", (Di,), torch.float32, dev)
    _opt(x0, "x0", (Bt, Di, N), torch.float32, dev)
    dims = make_dims(Bt, L, Di, N, io)
    y = torch.empty((Bt, L, Di), dtype=dt, device=dev)
    xf = torch.empty((Bt, Di, N), dtype=torch.float32, device=dev)
    ck = None
    if return_ckpt:
        ck = torch.empty(ckpt_bytes(dims) // 4, dtype=torch.float32, device=dev)
    ws = ws or workspace(OP_SCAN_FWD, dims, dev)
    check(lib().naju_scan_fwd(ctypes.byref(dims), _p(h), _p(a), _p(b), _p(B), _p(C), _p(D),
                              _p(x0), _p(y), _p(xf), _p(ck), ws.ptr, ws.nbytes,
                              stream_handle(dev)))
    if check_errors:
        check_workspace(ws)
    return (y, xf, ck) if return_ckpt else (y, xf)


def block_fwd(u, z, conv_w, a, b, B, C, D, x0=None, conv_state=None, *, return_ckpt=False,
              ws=None, check_errors=False):
    """y, x_final, conv_state_out (, ckpt) = naju_block_fwd(...) (check_errors: as for
    scan_fwd)."""
    Bt, L, Di = u.shape
    N = B.shape[-1]
    dt, dev = u.dtype, u.device
    io = _io_of(u)
    for nm, t in (("u", u), ("z", z), ("a", a), ("b", b)):
        _req(t, nm, (Bt, L, Di), dt, dev)
    _req(B, "B", (Bt, L, N), dt, dev)
    _req(C, "C", (Bt, L, N), dt, dev)
    _req(D, "D", (Di,), torch.float32, dev)
    _req(conv_w, "conv_w", (Di, D_CONV), torch.float32, dev)
    _opt(x0, "x0", (Bt, Di, N), torch.float32, dev)
    _opt(conv_state, "conv_state", (Bt, D_CONV - 1, Di), dt, dev)
    dims = make_dims(Bt, L, Di, N, io)
    y = torch.empty((Bt, L, Di), dtype=dt, device=dev)
    xf = torch.empty((Bt, Di, N), dtype=torch.float32, device=dev)
    cso = torch.empty((Bt, D_CONV - 1, Di), dtype=dt, device=dev)
    ck = None
    if return_ckpt:
        ck = torch.empty(ckpt_bytes(dims) // 4, dtype=torch.float32, device=dev)
    ws = ws or workspace(OP_BLOCK_FWD, dims, dev)
    check(lib().naju_block_fwd(ctypes.byref(dims), _p(u), _p(z), _p(conv_w), _p(conv_state),
                               _p(a), _p(b), _p(B), _p(C), _p(D), _p(x0), _p(y), _p(xf),
                               _p(cso), _p(ck), ws.ptr, ws.nbytes, stream_handle(dev)))
    if check_errors:
        check_workspace(ws)
    return (y, xf, cso, ck) if return_ckpt else (y, xf, cso)


def scan_bwd(h, a, b, B, C, D, dy, x0=None, dx_final=None, ckpt=None, *, want_dx0=True,
             ws=None):
    """Gradients of naju_scan_fwd: dict(dh, da, db, dB, dC, dD, dx0)."""
    Bt, L, Di = h.shape
    N = B.shape[-1]
    dt, dev = h.dtype, h.device
    io = _io_of(h)
    for nm, t in (("h", h), ("a", a), ("b", b), ("dy", dy)):
        _req(t, nm, (Bt, L, Di), dt, dev)
    _req(B, "B", (Bt, L, N), dt, dev)
    _req(C, "C", (Bt, L, N), dt, dev)
    _req(D, "D", (Di,), torch.float32, dev)
    _opt(x0, "x0", (Bt, Di, N), torch.float32, dev)
    _opt(dx_final, "dx_final", (Bt, Di, N), torch.float32, dev)
    dims = make_dims(Bt, L, Di, N, io)
    out = {k: torch.empty((Bt, L, Di), dtype=dt, device=dev) for k in ("dh", "da", "db")}
    out["dB"] = torch.empty((Bt, L, N), dtype=dt, device=dev)
    out["dC"] = torch.empty((Bt, L, N), dtype=dt, device=dev)
    out["dD"] = torch.empty((Di,), dtype=torch.float32, device=dev)
    out["dx0"] = torch.empty((Bt, Di, N), dtype=torch.float32, device=dev) if want_dx0 else None
    ws = ws or workspace(OP_SCAN_BWD, dims, dev)
    check(lib().naju_scan_bwd(ctypes.byref(dims), _p(h), _p(a), _p(b), _p(B), _p(C), _p(D),
                              _p(x0), _p(ckpt), _p(dy), _p(dx_final), _p(out["dh"]),
                              _p(out["da"]), _p(out["db"]), _p(out["dB"]), _p(out["dC"]),
                              _p(out["dD"]), _p(out["dx0"]), ws.ptr, ws.nbytes,
                              stream_handle(dev)))
    return out


def block_bwd(u, z, conv_w, a, b, B, C, D, dy, x0=None, dx_final=None, conv_state=None,
              ckpt=None, *, want_dx0=True, want_dconv_state=True, ws=None):
    """Gradients of naju_block_fwd: dict(du, dz, dconv_w, dconv_state, da, db, dB, dC, dD, dx0)."""
    Bt, L, Di = u.shape
    N = B.shape[-1]
    dt, dev = u.dtype, u.device
    io = _io_of(u)
    for nm, t in (("u", u), ("z", z), ("a", a), ("b", b), ("dy", dy)):
        _req(t, nm, (Bt, L, Di), dt, dev)
    _req(B, "B", (Bt, L, N), dt, dev)
    _req(C, "C", (Bt, L, N), dt, dev)
    _req(D, "D", (Di,), torch.float32, dev)
    _req(conv_w, "conv_w", (Di, D_CONV), torch.float32, dev)
    _opt(x0, "x0", (Bt, Di, N), torch.float32, dev)
    _opt(dx_final, "dx_final", (Bt, Di, N), torch.float32, dev)
    _opt(conv_state, "conv_state", (Bt, D_CONV - 1, Di), dt, dev)
    dims = make_dims(Bt, L, Di, N, io)
    out = {k: torch.empty((Bt, L, Di), dtype=dt, device=dev) for k in ("du", "dz", "da", "db")}
    out["dB"] = torch.empty((Bt, L, N), dtype=dt, device=dev)
    out["dC"] = torch.empty((Bt, L, N), dtype=dt, device=dev)
    out["dD"] = torch.empty((Di,), dtype=torch.float32, device=dev)
    out["dconv_w"] = torch.empty((Di, D_CONV), dtype=torch.float32, device=dev)
    out["dconv_state"] = (torch.empty((Bt, D_CONV - 1, Di), dtype=dt, device=dev)
                          if want_dconv_state else None)
    out["dx0"] = torch.empty((Bt, Di, N), dtype=torch.float32, device=dev) if want_dx0 else None
    ws = ws or workspace(OP_BLOCK_BWD, dims, dev)
    check(lib().naju_block_bwd(ctypes.byref(dims), _p(u), _p(z), _p(conv_w), _p(conv_state),
                               _p(a), _p(b), _p(B), _p(C), _p(D), _p(x0), _p(ckpt), _p(dy),
                               _p(dx_final), _p(out["du"]), _p(out["dz"]), _p(out["dconv_w"]),
                               _p(out["dconv_state"]), _p(out["da"]), _p(out["db"]),
                               _p(out["dB"]), _p(out["dC"]), _p(out["dD"]), _p(out["dx0"]),
                               ws.ptr, ws.nbytes, stream_handle(dev)))
    return out


def scan_step(h, a, b, B, C, D, x):
    """y = naju_scan_step(h, a, b, B, C, D, x); x ([Bt, Di, N] fp32) is updated in place."""
    Bt, Di = h.shape
    N = B.shape[-1]
    dt, dev = h.dtype, h.device
    io = _io_of(h)
    for nm, t in (("h", h), ("a", a), ("b", b)):
        _req(t, nm, (Bt, Di), dt, dev)
    _req(B, "B", (Bt, N), dt, dev)
    _req(C, "C", (Bt, N), dt, dev)
    _req(D, "D", (Di,), torch.float32, dev)
    _req(x, "x", (Bt, Di, N), torch.float32, dev)
    dims = make_dims(Bt, 1, Di, N, io)
    y = torch.empty((Bt, Di), dtype=dt, device=dev)
    check(lib().naju_scan_step(ctypes.byref(dims), _p(h), _p(a), _p(b), _p(B), _p(C), _p(D),
                               _p(x), _p(y), stream_handle(dev)))
    return y


def block_step(u, z, conv_w, conv_state, a, b, B, C, D, x):
    """y = naju_block_step(...); x and conv_state ([Bt, K-1, Di]) are updated in place."""
    Bt, Di = u.shape
    N = B.shape[-1]
    dt, dev = u.dtype, u.device
    io = _io_of(u)
    for nm, t in (("u", u), ("z", z), ("a", a), ("b", b)):
        _req(t, nm, (Bt, Di), dt, dev)
    _req(B, "B", (Bt, N), dt, dev)
    _req(C, "C", (Bt, N), dt, dev)
    _req(D, "D", (Di,), torch.float32, dev)
    _req(conv_w, "conv_w", (Di, D_CONV), torch.float32, dev)
    _req(conv_state, "conv_state", (Bt, D_CONV - 1, Di), dt, dev)
    _req(x, "x", (Bt, Di, N), torch.float32, dev)
    dims = make_dims(Bt, 1, Di, N, io)
    y = torch.empty((Bt, Di), dtype=dt, device=dev)
    check(lib().naju_block_step(ctypes.byref(dims), _p(u), _p(z), _p(conv_w), _p(conv_state),
                                _p(a), _p(b), _p(B), _p(C), _p(D), _p(x), _p(y),
                                stream_handle(dev)))
    return y


def mixer_fwd(xn, W_u, W_z, conv_w, W_a, a_bias, W_b, b_bias, W_B, W_C, D, W_out, res=None,
              conv_state=None, *, ws=None):
    """out = naju_mixer_fwd(...): the mixer layer around the block scan (bf16)."""
    Bt, L, dm = xn.shape
    Di = W_u.shape[1]
    N = W_B.shape[1]
    dt, dev = xn.dtype, xn.device
    if dt != torch.bfloat16:
        raise TypeError("the mixer layer takes bfloat16 activations and weights")
    _req(xn, "xn", (Bt, L, dm), dt, dev)
    _opt(res, "res", (Bt, L, dm), dt, dev)
    _req(W_u, "W_u", (dm, Di), dt, dev)
    _req(W_z, "W_z", (dm, Di), dt, dev)
    _req(conv_w, "conv_w", (Di, D_CONV), torch.float32, dev)
    _opt(conv_state, "conv_state", (Bt, D_CONV - 1, Di), dt, dev)
    _req(W_a, "W_a", (Di, Di), dt, dev)
    _req(W_b, "W_b", (Di, Di), dt, dev)
    _req(a_bias, "a_bias", (Di,), torch.float32, dev)
    _req(b_bias, "b_bias", (Di,), torch.float32, dev)
    _req(W_B, "W_B", (Di, N), dt, dev)
    _req(W_C, "W_C", (Di, N), dt, dev)
    _req(D, "D", (Di,), torch.float32, dev)
    _req(W_out, "W_out", (Di, dm), dt, dev)
    dims = make_dims(Bt, L, Di, N, BF16)
    out = torch.empty((Bt, L, dm), dtype=dt, device=dev)
    if ws is None:
        d = torch.device(dev)
        key = (d.index, torch.cuda.current_stream(d).cuda_stream, "mixer", Bt, L, dm, Di, N)
        ws = _ws_cache.get(key)
        if ws is None:
            ws = Workspace(int(lib().naju_mixer_workspace_bytes(ctypes.byref(dims), dm)), d)
            _ws_cache[key] = ws
    check(lib().naju_mixer_fwd(ctypes.byref(dims), dm, _p(xn), _p(res), _p(W_u), _p(W_z),
                               _p(conv_w), _p(conv_state), _p(W_a), _p(a_bias), _p(W_b),
                               _p(b_bias), _p(W_B), _p(W_C), _p(D), _p(W_out), _p(out), ws.ptr,
                               ws.nbytes, stream_handle(dev)))
    return out


def mixer_bwd(xn, W_u, W_z, conv_w, W_a, a_bias, W_b, b_bias, W_B, W_C, D, W_out, d_out,
              conv_state=None, *, fwd_ws=None, ws=None):
    """Gradients of naju_mixer_fwd for upstream d_out (the residual's is d_out); fwd_ws:
    the Workspace a mixer_fwd call on the same inputs used (its intermediates are reused):
    dict(dxn, dW_u, dW_z, dconv_w, dconv_state, dW_a, da_bias, dW_b, db_bias, dW_B, dW_C,
    dD, dW_out), fp32 except dconv_state (bf16, only with conv_state)."""
    Bt, L, dm = xn.shape
    Di = W_u.shape[1]
    N = W_B.shape[1]
    dt, dev = xn.dtype, xn.device
    if dt != torch.bfloat16:
        raise TypeError("the mixer layer takes bfloat16 activations and weights")
    _req(d_out, "d_out", (Bt, L, dm), dt, dev)
    for nm, t, shp in (("xn", xn, (Bt, L, dm)), ("W_u", W_u, (dm, Di)), ("W_z", W_z, (dm, Di)),
                       ("W_a", W_a, (Di, Di)), ("W_b", W_b, (Di, Di)), ("W_B", W_B, (Di, N)),
                       ("W_C", W_C, (Di, N)), ("W_out", W_out, (Di, dm))):
        _req(t, nm, shp, dt, dev)
    for nm, t, shp in (("conv_w", conv_w, (Di, D_CONV)), ("a_bias", a_bias, (Di,)),
                       ("b_bias", b_bias, (Di,)), ("D", D, (Di,))):
        _req(t, nm, shp, torch.float32, dev)
    _opt(conv_state, "conv_state", (Bt, D_CONV - 1, Di), dt, dev)
    dims = make_dims(Bt, L, Di, N, BF16)
    f32 = lambda *shape: torch.empty(shape, dtype=torch.float32, device=dev)  # noqa: E731
    g = dict(dxn=f32(Bt, L, dm), dW_u=f32(dm, Di), dW_z=f32(dm, Di), dconv_w=f32(Di, D_CONV),
             dW_a=f32(Di, Di), da_bias=f32(Di), dW_b=f32(Di, Di), db_bias=f32(Di),
             dW_B=f32(Di, N), dW_C=f32(Di, N), dD=f32(Di), dW_out=f32(Di, dm))
    g["dconv_state"] = (torch.empty((Bt, D_CONV - 1, Di), dtype=dt, device=dev)
                        if conv_state is not None else None)
    if ws is None:
        d = torch.device(dev)
        key = (d.index, torch.cuda.current_stream(d).cuda_stream, "mixer_bwd", Bt, L, dm, Di, N)
        ws = _ws_cache.get(key)
        if ws is None:
            ws = Workspace(int(lib().naju_mixer_bwd_workspace_bytes(ctypes.byref(dims), dm)), d)
            _ws_cache[key] = ws
    check(lib().naju_mixer_bwd(ctypes.byref(dims), dm, _p(xn), _p(W_u), _p(W_z), _p(conv_w),
                               _p(conv_state), _p(W_a), _p(a_bias), _p(W_b), _p(b_bias),
                               _p(W_B), _p(W_C), _p(D), _p(W_out), _p(d_out), _p(g["dxn"]),
                               _p(g["dW_u"]), _p(g["dW_z"]), _p(g["dconv_w"]),
                               _p(g["dconv_state"]), _p(g["dW_a"]), _p(g["da_bias"]),
                               _p(g["dW_b"]), _p(g["db_bias"]), _p(g["dW_B"]), _p(g["dW_C"]),
                               _p(g["dD"]), _p(g["dW_out"]),
                               fwd_ws.ptr if fwd_ws is not None else None,
                               fwd_ws.nbytes if fwd_ws is not None else 0, ws.ptr, ws.nbytes,
                               stream_handle(dev)))
    return g
