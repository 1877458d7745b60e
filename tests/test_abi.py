"""CPU checks of the C ABI: the library loads, exports every function that
include/naju.h declares, the binding's argument counts match the header, and
argument validation rejects bad calls before anything is enqueued (no GPU is
touched by any call here)."""
import ctypes
import os
import re

import pytest

from selective_state_space_naju_amd import binding as nb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "naju.h")


def header_prototypes():
    """name -> number of parameters, for every function declared in naju.h."""
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    protos = {}
    for m in re.finditer(r"\b(naju_\w+)\s*\(([^;{]*?)\)\s*;", src, flags=re.S):
        name, params = m.group(1), m.group(2).strip()
        protos[name] = 0 if params in ("", "void") else params.count(",") + 1
    return protos


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(nb.LIB_PATH):
        pytest.fail("libnaju.so is not built (run __graft_entry__.build())")
    return nb.lib()


def test_library_exports_every_declared_symbol(lib):
    protos = header_prototypes()
    assert set(protos) == set(nb.EXPORTS)
    for name in protos:
        assert hasattr(lib, name), name


def test_binding_argument_counts_match_header(lib):
    for name, n in header_prototypes().items():
        assert len(getattr(lib, name).argtypes) == n, name


def test_version(lib):
    assert b"gfx950" in lib.naju_version()


def dims(**kw):
    d = dict(batch=2, seqlen=300, d_inner=100, d_state=16, io=nb.BF16)
    d.update(kw)
    return nb.make_dims(d["batch"], d["seqlen"], d["d_inner"], d["d_state"], d["io"],
                        d.get("d_conv", 4))


FAKE = 0x100000  # a 256-byte aligned non-null address; never dereferenced


def call_scan_fwd(lib, d, **over):
    args = dict(h=FAKE, a=FAKE, b=FAKE, B=FAKE, C=FAKE, D=FAKE, x0=None, y=FAKE, xf=None,
                ck=None, ws=FAKE, wsb=1 << 40)
    args.update(over)
    v = [args[k] for k in ("h", "a", "b", "B", "C", "D", "x0", "y", "xf", "ck", "ws")]
    return lib.naju_scan_fwd(ctypes.byref(d) if d is not None else None, *v, args["wsb"], None)


def test_validation_errors_scan_fwd(lib):
    assert call_scan_fwd(lib, None) == nb.EINVAL
    assert call_scan_fwd(lib, dims(batch=-1)) == nb.EINVAL
    assert call_scan_fwd(lib, dims(d_state=32)) == nb.EUNSUPPORTED
    assert call_scan_fwd(lib, dims(d_state=0)) == nb.EINVAL
    assert call_scan_fwd(lib, dims(io=7)) == nb.EINVAL
    assert call_scan_fwd(lib, dims(), h=None) == nb.EINVAL
    assert "h is NULL" in nb.last_error()
    assert call_scan_fwd(lib, dims(), C=FAKE + 1) == nb.EINVAL
    assert "aligned" in nb.last_error()
    assert call_scan_fwd(lib, dims(), ws=None) == nb.EWORKSPACE
    assert call_scan_fwd(lib, dims(), wsb=16) == nb.EWORKSPACE
    assert call_scan_fwd(lib, dims(), ws=FAKE + 64) == nb.EINVAL
    # empty problems are valid no-ops (nothing to enqueue)
    assert call_scan_fwd(lib, dims(batch=0), h=None, ws=None) == nb.OK
    assert call_scan_fwd(lib, dims(d_inner=0), h=None, ws=None) == nb.OK


def test_validation_errors_block(lib):
    d = dims(d_conv=3)
    v = [FAKE] * 15
    assert lib.naju_block_fwd(ctypes.byref(d), *v, 1 << 40, None) == nb.EUNSUPPORTED
    d = dims(d_conv=0)
    assert lib.naju_block_fwd(ctypes.byref(d), *v, 1 << 40, None) == nb.EINVAL
    d = dims()
    v2 = list(v)
    v2[1] = None  # z
    assert lib.naju_block_fwd(ctypes.byref(d), *v2, 1 << 40, None) == nb.EINVAL
    assert "z is NULL" in nb.last_error()
    vb = [FAKE] * 24
    vb[13] = None  # du
    assert lib.naju_block_bwd(ctypes.byref(d), *vb, 1 << 40, None) == nb.EINVAL
    assert "du is NULL" in nb.last_error()


def test_validation_errors_step(lib):
    d = dims()
    v = [FAKE] * 9  # h, a, b, B, C, D, x, y, stream
    v[-1] = None
    vx = list(v)
    vx[6] = None  # x
    assert lib.naju_scan_step(ctypes.byref(d), *vx) == nb.EINVAL
    assert "x is NULL" in nb.last_error()
    vx[6] = FAKE + 4  # x must be 16-byte aligned (float4 state rows)
    assert lib.naju_scan_step(ctypes.byref(d), *vx) == nb.EINVAL
    assert "aligned" in nb.last_error()
    assert lib.naju_scan_step(ctypes.byref(dims(d_state=32)), *vx) == nb.EUNSUPPORTED
    assert lib.naju_scan_step(ctypes.byref(dims(batch=70000)), *v) == nb.EINVAL
    assert lib.naju_scan_step(ctypes.byref(dims(batch=0)), *([None] * 9)) == nb.OK
    vb = [FAKE] * 12  # u, z, conv_w, conv_state, a, b, B, C, D, x, y, stream
    vb[-1] = None
    vb[3] = None  # conv_state is required (it is updated in place)
    assert lib.naju_block_step(ctypes.byref(d), *vb) == nb.EINVAL
    assert "conv_state is NULL" in nb.last_error()
    assert lib.naju_block_step(ctypes.byref(dims(d_conv=3)), *vb) == nb.EUNSUPPORTED


def test_validation_errors_mixer(lib):
    # dims, d_model, xn, res, W_u, W_z, conv_w, conv_state, W_a, a_bias, W_b, b_bias, W_B, W_C,
    # D, W_out, out, ws, ws_bytes, stream
    def call(d, dm=64, **over):
        args = dict(xn=FAKE, res=None, W_u=FAKE, W_z=FAKE, conv_w=FAKE, conv_state=None,
                    W_a=FAKE, a_bias=FAKE, W_b=FAKE, b_bias=FAKE, W_B=FAKE, W_C=FAKE, D=FAKE,
                    W_out=FAKE, out=FAKE, ws=FAKE, wsb=1 << 40)
        args.update(over)
        v = [args[k] for k in ("xn", "res", "W_u", "W_z", "conv_w", "conv_state", "W_a",
                               "a_bias", "W_b", "b_bias", "W_B", "W_C", "D", "W_out", "out",
                               "ws")]
        return lib.naju_mixer_fwd(ctypes.byref(d), dm, *v, args["wsb"], None)
    d = dims(d_inner=128)
    assert call(dims(d_inner=128, io=nb.F32)) == nb.EUNSUPPORTED
    assert call(dims(d_inner=100)) == nb.EUNSUPPORTED  # d_inner % 8
    assert call(d, dm=60) == nb.EUNSUPPORTED
    assert call(d, dm=0) == nb.EINVAL
    assert call(dims(d_inner=128, d_conv=3)) == nb.EUNSUPPORTED
    assert call(d, W_a=None) == nb.EINVAL
    assert "W_a is NULL" in nb.last_error()
    assert call(d, W_out=FAKE + 2) == nb.EINVAL
    assert "aligned" in nb.last_error()
    assert call(d, ws=None) == nb.EWORKSPACE
    assert call(d, wsb=1024) == nb.EWORKSPACE
    assert call(dims(d_inner=128, batch=0), xn=None, ws=None) == nb.OK
    # the workspace holds u, z, h, a, b, y, B, C, the GEMM workspace and the block forward's
    w = lib.naju_mixer_workspace_bytes(ctypes.byref(dims(batch=8, seqlen=2048, d_inner=1536)), 768)
    assert w > 6 * 8 * 2048 * 1536 * 2 + 2 * 8 * 2048 * 16 * 2
    assert lib.naju_mixer_workspace_bytes(ctypes.byref(dims(d_state=48)), 64) == 0


def test_validation_errors_mixer_bwd(lib):
    # dims, d_model, 14 inputs (xn .. d_out), 13 gradients, ws, ws_bytes, stream
    def call(d, dm=64, **over):
        ins = dict(xn=FAKE, W_u=FAKE, W_z=FAKE, conv_w=FAKE, conv_state=None, W_a=FAKE,
                   a_bias=FAKE, W_b=FAKE, b_bias=FAKE, W_B=FAKE, W_C=FAKE, D=FAKE, W_out=FAKE,
                   d_out=FAKE)
        outs = dict(dxn=FAKE, dW_u=FAKE, dW_z=FAKE, dconv_w=FAKE, dconv_state=None, dW_a=FAKE,
                    da_bias=FAKE, dW_b=FAKE, db_bias=FAKE, dW_B=FAKE, dW_C=FAKE, dD=FAKE,
                    dW_out=FAKE)
        for k, v in over.items():
            if k not in ("ws", "wsb", "fws", "fwsb"):
                (ins if k in ins else outs)[k] = v
        return lib.naju_mixer_bwd(ctypes.byref(d), dm, *ins.values(), *outs.values(),
                                  over.get("fws", None), over.get("fwsb", 0),
                                  over.get("ws", FAKE), over.get("wsb", 1 << 40), None)
    d = dims(d_inner=128)
    assert call(d, d_out=None) == nb.EINVAL
    assert "d_out is NULL" in nb.last_error()
    assert call(d, dW_a=None) == nb.EINVAL
    assert "dW_a is NULL" in nb.last_error()
    assert call(d, dxn=FAKE + 4) == nb.EINVAL
    assert call(dims(d_inner=128, io=nb.F32)) == nb.EUNSUPPORTED
    assert call(dims(d_inner=128, batch=0), xn=None) == nb.OK
    assert call(d, fws=FAKE, fwsb=16) == nb.EWORKSPACE  # a forward workspace too small
    assert call(d, fws=FAKE + 8, fwsb=1 << 40) == nb.EINVAL
    fwd = lib.naju_mixer_workspace_bytes(ctypes.byref(d), 64)
    assert lib.naju_mixer_bwd_workspace_bytes(ctypes.byref(d), 64) > fwd


def test_workspace_and_ckpt_sizes(lib):
    d = dims(batch=8, seqlen=2048, d_inner=1536)
    for op in range(4):
        assert nb.workspace_bytes(op, d) > 256
    assert nb.workspace_bytes(nb.OP_SCAN_BWD, d) > nb.workspace_bytes(nb.OP_SCAN_FWD, d)
    # checkpoints: one fp32 state per 32-token chunk
    assert nb.ckpt_bytes(d) == 8 * (2048 // 32) * 16 * 1536 * 4
    assert nb.workspace_bytes(nb.OP_SCAN_FWD, dims(d_state=48)) == 0
    assert lib.naju_workspace_bytes(9, ctypes.byref(d)) == 0


def test_binding_requires_library_file(monkeypatch, tmp_path):
    monkeypatch.setattr(nb, "_lib", None)
    monkeypatch.setattr(nb, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        nb.lib()


def test_validation_errors_scan_fwd_noalloc(lib):
    """Rejected before anything is enqueued: bad dims, and a shape whose forward
    workspace exceeds the library's scratch (no GPU is touched)."""
    bad = nb.make_dims(1, 16, 64, 17, nb.BF16)
    st = lib.naju_scan_fwd_noalloc(ctypes.byref(bad), *([ctypes.c_void_p(256)] * 10), None, None)
    assert st != nb.OK
    big = nb.make_dims(64, 65536, 4096, 16, nb.BF16)
    assert nb.workspace_bytes(nb.OP_SCAN_FWD, big) > (64 << 20)
    st = lib.naju_scan_fwd_noalloc(ctypes.byref(big), *([ctypes.c_void_p(256)] * 10), None, None)
    assert st == nb.EWORKSPACE
    assert b"scratch" in lib.naju_last_error()
