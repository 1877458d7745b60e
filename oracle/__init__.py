"""fp64 CPU oracle of the Naju selective scan -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path never does, and this
package imports nothing from the product package.

The scan and block arithmetic lives in ``naju_oracle.c`` (plain C, fp64,
sequential time loops); this module builds it with gcc and marshals numpy
arrays.  It also holds the mixer layer's oracle (``mixer_fwd`` /
``mixer_bwd``): the block flowchart's projections around the C block scan,
written as fp64 numpy matrix products, and the conv+SiLU reverse mode they
need.  Definitions followed (reproduction README of arXiv 2607.21000, "Core
equations" and the block flowchart):

    x_n  = sigma(a_n) x_{n-1} + sigma(b_n) h_n B_n^T
    ys_n = x_n C_n / sqrt(N) + D h_n
    block: h = SiLU(causal depthwise conv(u)),  y = ys * SiLU(z)

Parity pinning: every function here is pinned by ``tests/test_oracle_pins.py``
against closed forms, brute force, library routines (scipy lfilter, numpy
matmul) and central finite differences.  Nothing here is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "naju_oracle.c")
_LIB = os.path.join(_HERE, "libnaju_oracle.so")

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, no FMA contraction, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
               "-shared", "-std=c11", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = ctypes.CDLL(_LIB)
        i64 = ctypes.c_int64
        p = ctypes.c_void_p
        _lib.naju_oracle_scan_fwd.argtypes = [i64] * 4 + [p] * 9
        _lib.naju_oracle_scan_bwd.argtypes = [i64] * 4 + [p] * 16
        _lib.naju_oracle_conv_silu.argtypes = [i64] * 4 + [p] * 5
        _lib.naju_oracle_block_fwd.argtypes = [i64] * 5 + [p] * 13
        _lib.naju_oracle_block_bwd.argtypes = [i64] * 5 + [p] * 22
        for f in ("naju_oracle_scan_fwd", "naju_oracle_scan_bwd", "naju_oracle_conv_silu",
                  "naju_oracle_block_fwd", "naju_oracle_block_bwd"):
            getattr(_lib, f).restype = None
    return _lib


def _in(x, shape=None):
    """Read-only fp64 C-contiguous copy (or None)."""
    if x is None:
        return None
    arr = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    if shape is not None and arr.shape != tuple(shape):
        raise ValueError("oracle: expected shape %s, got %s" % (tuple(shape), arr.shape))
    return arr


def _p(arr):
    return None if arr is None else arr.ctypes.data_as(ctypes.c_void_p)


def _dims(h, B):
    Bt, L, Di = np.shape(h)
    N = np.shape(B)[-1]
    return int(Bt), int(L), int(Di), int(N)


def scan_fwd(h, a, b, B, C, D, x0=None):
    """Returns (ys [Bt,L,Di], x_final [Bt,Di,N]) in fp64."""
    lib = _load()
    Bt, L, Di, N = _dims(h, B)
    t3, tn, st = (Bt, L, Di), (Bt, L, N), (Bt, Di, N)
    h, a, b = _in(h, t3), _in(a, t3), _in(b, t3)
    B, C, D, x0 = _in(B, tn), _in(C, tn), _in(D, (Di,)), _in(x0, st)
    ys = np.empty(t3)
    xf = np.empty(st)
    lib.naju_oracle_scan_fwd(Bt, L, Di, N, _p(h), _p(a), _p(b), _p(B), _p(C), _p(D), _p(x0),
                             _p(ys), _p(xf))
    return ys, xf


def scan_bwd(h, a, b, B, C, D, x0, g, dx_final=None):
    """Reverse mode of scan_fwd for upstream gradient g = dLoss/dys.

    Returns dict with dh, da, db [Bt,L,Di]; dB, dC [Bt,L,N]; dD [Di]; dx0 [Bt,Di,N].
    """
    lib = _load()
    Bt, L, Di, N = _dims(h, B)
    t3, tn, st = (Bt, L, Di), (Bt, L, N), (Bt, Di, N)
    h, a, b, g = _in(h, t3), _in(a, t3), _in(b, t3), _in(g, t3)
    B, C, D = _in(B, tn), _in(C, tn), _in(D, (Di,))
    x0, dxf = _in(x0, st), _in(dx_final, st)
    out = {k: np.empty(t3) for k in ("dh", "da", "db")}
    out.update(dB=np.empty(tn), dC=np.empty(tn), dD=np.empty(Di), dx0=np.empty(st))
    lib.naju_oracle_scan_bwd(Bt, L, Di, N, _p(h), _p(a), _p(b), _p(B), _p(C), _p(D), _p(x0),
                             _p(g), _p(dxf), _p(out["dh"]), _p(out["da"]), _p(out["db"]),
                             _p(out["dB"]), _p(out["dC"]), _p(out["dD"]), _p(out["dx0"]))
    return out


def conv_silu(u, w, conv_state=None):
    """Returns (pre, h): causal depthwise conv of u with taps w [Di,K], then SiLU."""
    lib = _load()
    Bt, L, Di = np.shape(u)
    K = int(np.shape(w)[1])
    u, w = _in(u, (Bt, L, Di)), _in(w, (Di, K))
    cs = _in(conv_state, (Bt, K - 1, Di))
    pre = np.empty((Bt, L, Di))
    h = np.empty((Bt, L, Di))
    lib.naju_oracle_conv_silu(Bt, L, Di, K, _p(u), _p(w), _p(cs), _p(pre), _p(h))
    return pre, h


def block_fwd(u, z, w, a, b, B, C, D, x0=None, conv_state=None):
    """Returns (y, x_final, conv_state_out)."""
    lib = _load()
    Bt, L, Di, N = _dims(u, B)
    K = int(np.shape(w)[1])
    t3, tn, st = (Bt, L, Di), (Bt, L, N), (Bt, Di, N)
    u, z, a, b = _in(u, t3), _in(z, t3), _in(a, t3), _in(b, t3)
    w, cs = _in(w, (Di, K)), _in(conv_state, (Bt, K - 1, Di))
    B, C, D, x0 = _in(B, tn), _in(C, tn), _in(D, (Di,)), _in(x0, st)
    y = np.empty(t3)
    xf = np.empty(st)
    cso = np.empty((Bt, K - 1, Di))
    lib.naju_oracle_block_fwd(Bt, L, Di, N, K, _p(u), _p(z), _p(w), _p(cs), _p(a), _p(b),
                              _p(B), _p(C), _p(D), _p(x0), _p(y), _p(xf), _p(cso))
    return y, xf, cso


def block_bwd(u, z, w, a, b, B, C, D, x0, dy, dx_final=None, conv_state=None):
    """Reverse mode of block_fwd.  Returns dict with du, dz, dw, dconv_state, da, db,
    dB, dC, dD, dx0."""
    lib = _load()
    Bt, L, Di, N = _dims(u, B)
    K = int(np.shape(w)[1])
    t3, tn, st = (Bt, L, Di), (Bt, L, N), (Bt, Di, N)
    u, z, a, b, dy = _in(u, t3), _in(z, t3), _in(a, t3), _in(b, t3), _in(dy, t3)
    w, cs = _in(w, (Di, K)), _in(conv_state, (Bt, K - 1, Di))
    B, C, D = _in(B, tn), _in(C, tn), _in(D, (Di,))
    x0, dxf = _in(x0, st), _in(dx_final, st)
    out = {k: np.empty(t3) for k in ("du", "dz", "da", "db")}
    out.update(dw=np.empty((Di, K)), dconv_state=np.empty((Bt, K - 1, Di)),
               dB=np.empty(tn), dC=np.empty(tn), dD=np.empty(Di), dx0=np.empty(st))
    lib.naju_oracle_block_bwd(Bt, L, Di, N, K, _p(u), _p(z), _p(w), _p(cs), _p(a), _p(b),
                              _p(B), _p(C), _p(D), _p(x0), _p(dy), _p(dxf),
                              _p(out["du"]), _p(out["dz"]), _p(out["dw"]),
                              _p(out["dconv_state"]), _p(out["da"]), _p(out["db"]),
                              _p(out["dB"]), _p(out["dC"]), _p(out["dD"]), _p(out["dx0"]))
    return out


def _round(x):
    return round_bf16(x)


def round_bf16(x):
    """Values rounded to bfloat16 the way a device computing in fp32 stores them:
    first to the nearest fp32, then to the nearest bfloat16 (ties to the even
    significand).  Returns fp64 arrays holding the bf16 values."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    bits = f.view(np.uint32).astype(np.uint64)
    keep = bits >> np.uint64(16)
    rest = bits & np.uint64(0xFFFF)
    up = (rest > 0x8000) | ((rest == 0x8000) & ((keep & np.uint64(1)) == 1))
    keep = keep + up.astype(np.uint64)
    out = (keep << np.uint64(16)).astype(np.uint32).view(np.float32).astype(np.float64)
    return out.reshape(np.shape(x))


def mixer_fwd(xn, W_u, W_z, conv_w, W_a, a_bias, W_b, b_bias, W_B, W_C, D, W_out, res=None,
              conv_state=None, store_bf16=True):
    """The mixer layer of the block flowchart (reproduction README, "Background
    and main changes") around block_fwd, in fp64 with bf16 storage of the
    intermediates: returns a dict with u, z, h, a, b, B, C, y and out.

        u = xn W_u, z = xn W_z;  h = SiLU(conv(u));  a = h W_a + a_bias,
        b = h W_b + b_bias, B = h W_B, C = h W_C;  y = block_fwd(u, z, ...);
        out = y W_out + res
    Every intermediate is stored as bf16 (round_bf16) before its next use; the
    projections read the stored h, the scan recomputes h from u (block_fwd).
    The matrix products are numpy matmuls in fp64.  store_bf16=False skips the
    storage rounding (the smooth layer that finite differences can check)."""
    f = lambda t: None if t is None else np.asarray(t, dtype=np.float64)
    round_bf16 = _round if store_bf16 else (lambda t: np.asarray(t, dtype=np.float64))
    xn, W_u, W_z, W_a, W_b, W_B, W_C, W_out = map(f, (xn, W_u, W_z, W_a, W_b, W_B, W_C, W_out))
    u = round_bf16(xn @ W_u)
    z = round_bf16(xn @ W_z)
    _, h = conv_silu(u, conv_w, conv_state)
    h = round_bf16(h)
    a = round_bf16(h @ W_a + f(a_bias))
    b = round_bf16(h @ W_b + f(b_bias))
    B = round_bf16(h @ W_B)
    C = round_bf16(h @ W_C)
    y, _, _ = block_fwd(u, z, conv_w, a, b, B, C, D, conv_state=conv_state)
    y = round_bf16(y)
    o = y @ W_out
    if res is not None:
        o = o + f(res)
    return dict(u=u, z=z, h=h, a=a, b=b, B=B, C=C, y=y, out=round_bf16(o))


def _conv_silu_bwd(u, w, conv_state, dh):
    """Reverse mode of h = SiLU(conv(u)) (conv as conv_silu): returns
    (du, dw, dconv_state) for upstream dh, with SiLU'(p) = s (1 + p (1 - s))."""
    Bt, L, Di = u.shape
    K = w.shape[1]
    pre, _ = conv_silu(u, w, conv_state)
    s = 1.0 / (1.0 + np.exp(-pre))
    dpre = dh * s * (1.0 + pre * (1.0 - s))
    ext = np.concatenate([np.zeros((Bt, K - 1, Di)) if conv_state is None
                          else np.asarray(conv_state, dtype=np.float64), u], axis=1)
    du_ext = np.zeros_like(ext)
    dw = np.zeros((Di, K))
    for k in range(K):   # pre_n = sum_k w[:, k] ext[n + k]
        du_ext[:, k:k + L, :] += dpre * w[:, k]
        dw[:, k] = np.einsum("btc,btc->c", dpre, ext[:, k:k + L, :])
    return du_ext[:, K - 1:, :], dw, du_ext[:, :K - 1, :]


def mixer_bwd(xn, W_u, W_z, conv_w, W_a, a_bias, W_b, b_bias, W_B, W_C, D, W_out, d_out,
              res=None, conv_state=None, store_bf16=True):
    """Reverse mode of mixer_fwd for upstream gradient d_out = dLoss/dout.

    The stored bf16 intermediates pass gradients unchanged (rounding is taken
    as the identity); with store_bf16 the upstream gradients that the device
    stores in bf16 (dy, and the block backward's du, dz, da, db, dB, dC) are
    rounded the same way.  Returns a dict with dxn, dres, dW_u, dW_z, dconv_w,
    dconv_state, dW_a, da_bias, dW_b, db_bias, dW_B, dW_C, dD, dW_out."""
    f = lambda t: None if t is None else np.asarray(t, dtype=np.float64)
    rnd = _round if store_bf16 else (lambda t: np.asarray(t, dtype=np.float64))
    fw = mixer_fwd(xn, W_u, W_z, conv_w, W_a, a_bias, W_b, b_bias, W_B, W_C, D, W_out, res,
                   conv_state, store_bf16)
    xn, W_u, W_z, W_a, W_b, W_B, W_C, W_out, g = map(f, (xn, W_u, W_z, W_a, W_b, W_B, W_C,
                                                        W_out, d_out))
    w, cs = f(conv_w), f(conv_state)
    out = {"dres": g.copy() if res is not None else None}
    # out = y W_out + res
    dy = rnd(g @ W_out.T)
    out["dW_out"] = np.einsum("btk,btm->km", fw["y"], g)
    # y = block_fwd(u, z, conv_w, a, b, B, C, D)
    gb = block_bwd(fw["u"], fw["z"], w, fw["a"], fw["b"], fw["B"], fw["C"], D, None, dy,
                   conv_state=cs)
    da, db, dB, dC = (rnd(gb[k]) for k in ("da", "db", "dB", "dC"))
    du_blk, dz = rnd(gb["du"]), rnd(gb["dz"])
    out["dD"] = gb["dD"]
    # a = h W_a + a_bias, b = h W_b + b_bias, B = h W_B, C = h W_C (h: the stored one)
    h = fw["h"]
    dh = da @ W_a.T + db @ W_b.T + dB @ W_B.T + dC @ W_C.T
    out["dW_a"] = np.einsum("btk,btn->kn", h, da)
    out["dW_b"] = np.einsum("btk,btn->kn", h, db)
    out["dW_B"] = np.einsum("btk,btn->kn", h, dB)
    out["dW_C"] = np.einsum("btk,btn->kn", h, dC)
    out["da_bias"] = da.sum(axis=(0, 1))
    out["db_bias"] = db.sum(axis=(0, 1))
    # h = SiLU(conv(u)) on the projection path; the scan's own path is in gb
    du_p, dw_p, dcs_p = _conv_silu_bwd(fw["u"], w, cs, dh)
    du = rnd(du_blk + du_p)
    out["dconv_w"] = gb["dw"] + dw_p
    out["dconv_state"] = gb["dconv_state"] + dcs_p
    # u = xn W_u, z = xn W_z
    out["dxn"] = du @ W_u.T + dz @ W_z.T
    out["dW_u"] = np.einsum("btk,btn->kn", xn, du)
    out["dW_z"] = np.einsum("btk,btn->kn", xn, dz)
    return out
