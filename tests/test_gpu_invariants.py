"""GPU invariants of the hot path, and the edge cases of its gates, through the C ABI.

* Extreme gates: forget / write pre-activations near +-16, where sigma(-a) or
  sigma(-b) is about 1e-7 (the gate derivatives sigma(v) sigma(-v) must not
  cancel or underflow), for the scan and the block, forward and backward, on
  the matrix-core path and the fp32 register path; each output under the
  elementwise bound of gpu_helpers.assert_close.
* Homogeneity ("Core equations": the state and readout are linear in h and x0
  at fixed gates): y(2h, 2x0) = 2 y(h, x0) bit for bit when no look-back is
  involved (one 128-token chunk), within one bf16 ulp otherwise; the backward is
  linear in (dy, dx_final), bit for bit.
* Split invariance (the README's "Scope": the recurrence is an affine scan, so
  any split composes): one call equals two chained calls split at a token that
  is not a chunk boundary.
* Outputs written through raw pointers into sentinel-filled buffers leave the
  sentinels untouched (ragged tails, several batch rows).
* The forward's two ticket schedules give the same results.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import TOL, assert_agree, assert_close, f32_dev, host, to_dev
from selective_state_space_naju_amd import binding as nb
from selective_state_space_naju_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    nb.lib()


def _extreme(d, kind, seed):
    rng = np.random.default_rng(seed)
    shp = d["a"].shape
    noise = (0.5 * rng.standard_normal(shp)).astype(np.float32)
    if kind == "retain":     # f = 1 - ~1e-7: sigma(-a) ~ 1e-7 in da
        d["a"] = inputs.bf16_round(16.0 + noise)
    elif kind == "write":    # i = 1 - ~1e-7: sigma(-b) ~ 1e-7 in db
        d["b"] = inputs.bf16_round(16.0 + noise)
    elif kind == "forget":   # f ~ 1e-7: chunks leave the rescaled form's range
        d["a"] = inputs.bf16_round(-16.0 + noise)
    elif kind == "nowrite":  # i ~ 1e-7
        d["b"] = inputs.bf16_round(-16.0 + noise)
    return d


GATE_CASES = [
    # io, N, block, kind
    ("bf16", 16, False, "retain"), ("bf16", 16, False, "write"),
    ("bf16", 16, True, "retain"), ("bf16", 16, True, "write"),
    ("bf16", 16, False, "forget"), ("bf16", 16, True, "nowrite"),
    ("f32", 16, False, "retain"), ("f32", 16, True, "write"),
    ("bf16", 64, False, "retain"), ("bf16", 64, False, "write"),
]


@pytest.mark.parametrize("case", GATE_CASES, ids=lambda c: "%s_n%d_%s_%s" % (
    c[0], c[1], "block" if c[2] else "scan", c[3]))
def test_extreme_gates(case):
    io, N, block, kind = case
    Bt, L, Di = 2, 300, 128
    d = inputs.draw(Bt, L, Di, N, io=io, seed=31, x0=True, backward=True, dx_final=True,
                    block=block, conv_state=block)
    d = _extreme(d, kind, 32)
    print("extreme gates", case, flush=True)
    tol = TOL[io]
    D, x0, dxf = f32_dev(d["D"]), f32_dev(d["x0"]), f32_dev(d["dx_final"])
    if block:
        t = {k: to_dev(d[k], io) for k in ("u", "z", "a", "b", "B", "C", "dy", "conv_state")}
        w = f32_dev(d["conv_w"])
        y, xf, _, ck = nb.block_fwd(t["u"], t["z"], w, t["a"], t["b"], t["B"], t["C"], D, x0,
                                    t["conv_state"], return_ckpt=True, check_errors=True)
        g = nb.block_bwd(t["u"], t["z"], w, t["a"], t["b"], t["B"], t["C"], D, t["dy"], x0, dxf,
                         t["conv_state"], ck)
        torch.cuda.synchronize()
        yo, xfo, _ = oracle.block_fwd(d["u"], d["z"], d["conv_w"], d["a"], d["b"], d["B"],
                                      d["C"], d["D"], d["x0"], d["conv_state"])
        ref = oracle.block_bwd(d["u"], d["z"], d["conv_w"], d["a"], d["b"], d["B"], d["C"],
                               d["D"], d["x0"], d["dy"], d["dx_final"], d["conv_state"])
        ref["dconv_w"] = ref["dw"]
        names = ("du", "dz", "da", "db", "dB", "dC", "dD", "dx0", "dconv_w")
    else:
        t = {k: to_dev(d[k], io) for k in ("h", "a", "b", "B", "C", "dy")}
        y, xf, ck = nb.scan_fwd(t["h"], t["a"], t["b"], t["B"], t["C"], D, x0, return_ckpt=True,
                                check_errors=True)
        g = nb.scan_bwd(t["h"], t["a"], t["b"], t["B"], t["C"], D, t["dy"], x0, dxf, ck)
        torch.cuda.synchronize()
        yo, xfo = oracle.scan_fwd(d["h"], d["a"], d["b"], d["B"], d["C"], d["D"], d["x0"])
        ref = oracle.scan_bwd(d["h"], d["a"], d["b"], d["B"], d["C"], d["D"], d["x0"], d["dy"],
                              d["dx_final"])
        names = ("dh", "da", "db", "dB", "dC", "dD", "dx0")
    assert_close("y", host(y), yo, tol)
    assert_close("x_final", host(xf), xfo, tol)
    for k in names:
        assert_close(k, host(g[k]), ref[k], tol)


@pytest.mark.parametrize("L", [128, 1000], ids=["one_chunk", "look_back"])
def test_homogeneity(L):
    """y(2h, 2x0) = 2 y(h, x0); the backward is linear in (dy, dx_final)."""
    Bt, Di, N = 2, 136, 16
    d = inputs.draw(Bt, L, Di, N, io="bf16", seed=33, x0=True, backward=True, dx_final=True)
    t = {k: to_dev(d[k], "bf16") for k in ("h", "a", "b", "B", "C", "dy")}
    D, x0, dxf = f32_dev(d["D"]), f32_dev(d["x0"]), f32_dev(d["dx_final"])
    y1, xf1 = nb.scan_fwd(t["h"], t["a"], t["b"], t["B"], t["C"], D, x0, check_errors=True)
    y2, xf2 = nb.scan_fwd(t["h"] * 2, t["a"], t["b"], t["B"], t["C"], D, x0 * 2,
                          check_errors=True)
    torch.cuda.synchronize()
    if L <= 128:
        assert torch.equal(y2, y1 * 2) and torch.equal(xf2, xf1 * 2)
    else:
        assert_agree("y(2h, 2x0)", host(y2), 2 * host(y1))
        e = np.abs(host(xf2) - 2 * host(xf1)).max() / np.abs(2 * host(xf1)).max()
        assert e <= 1e-6, e
    # (one set of checkpoints for both: the backward itself has no look-back)
    _, _, ck = nb.scan_fwd(t["h"], t["a"], t["b"], t["B"], t["C"], D, x0, return_ckpt=True,
                           check_errors=True)
    g1 = nb.scan_bwd(t["h"], t["a"], t["b"], t["B"], t["C"], D, t["dy"], x0, dxf, ck)
    g2 = nb.scan_bwd(t["h"], t["a"], t["b"], t["B"], t["C"], D, t["dy"] * 2, x0, dxf * 2, ck)
    torch.cuda.synchronize()
    for k in ("dh", "da", "db", "dB", "dC", "dD", "dx0"):
        assert torch.equal(g2[k], g1[k] * 2), k


@pytest.mark.parametrize("block", [False, True], ids=["scan", "block"])
def test_split_invariance(block):
    """One call over L tokens equals two chained calls split at token 333 (not a
    boundary of the 32- or 128-token chunks), the state and conv window carried."""
    Bt, L, Di, N, m = 2, 1000, 136, 16, 333
    d = inputs.draw(Bt, L, Di, N, io="bf16", seed=34, x0=True, block=block, conv_state=block)
    hk = "u" if block else "h"
    keys = (hk, "a", "b", "B", "C") + (("z",) if block else ())
    t = {k: to_dev(d[k], "bf16") for k in keys}
    first = {k: v[:, :m].contiguous() for k, v in t.items()}
    second = {k: v[:, m:].contiguous() for k, v in t.items()}
    D, x0 = f32_dev(d["D"]), f32_dev(d["x0"])
    if block:
        w, cs = f32_dev(d["conv_w"]), to_dev(d["conv_state"], "bf16")
        run = lambda s, xi, c: nb.block_fwd(s["u"], s["z"], w, s["a"], s["b"], s["B"], s["C"],  # noqa: E731
                                            D, xi, c, check_errors=True)
        y, xf, cso = run(t, x0, cs)
        y1, xm, csm = run(first, x0, cs)
        y2, xf2, cso2 = run(second, xm, csm)
    else:
        run = lambda s, xi: nb.scan_fwd(s["h"], s["a"], s["b"], s["B"], s["C"], D, xi,  # noqa: E731
                                        check_errors=True)
        y, xf = run(t, x0)
        y1, xm = run(first, x0)
        y2, xf2 = run(second, xm)
    torch.cuda.synchronize()
    yc = torch.cat([y1, y2], dim=1)
    assert_agree("y(chained)", host(yc), host(y))
    e = np.abs(host(xf2) - host(xf)).max() / np.abs(host(xf)).max()
    assert e <= 1e-5, e
    if block:
        assert torch.equal(cso2, cso)
        yo, xfo, _ = oracle.block_fwd(d["u"], d["z"], d["conv_w"], d["a"], d["b"], d["B"], d["C"],
                                      d["D"], d["x0"], d["conv_state"])
    else:
        yo, xfo = oracle.scan_fwd(d["h"], d["a"], d["b"], d["B"], d["C"], d["D"], d["x0"])
    assert_close("y(chained)", host(yc), yo, TOL["bf16"])
    assert_close("x_final(chained)", host(xf2), xfo, TOL["bf16"])


SENT = -12288.0  # -1.5 * 2^13: exactly representable in bf16 and fp32


def _padded(n, dtype, pad=64):
    big = torch.full((n + 2 * pad,), SENT, dtype=dtype, device="cuda")
    return big, big[pad:pad + n]


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_outputs_stay_in_bounds(io):
    """Scan forward and backward into sentinel-padded buffers: 3 batch rows,
    L = 300 (a ragged last wave and chunk), d_inner 200 (a ragged channel tile)."""
    Bt, L, Di, N = 3, 300, 200, 16
    d = inputs.draw(Bt, L, Di, N, io=io, seed=35, x0=True, backward=True, dx_final=True)
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    t = {k: to_dev(d[k], io) for k in ("h", "a", "b", "B", "C", "dy")}
    D, x0, dxf = f32_dev(d["D"]), f32_dev(d["x0"]), f32_dev(d["dx_final"])
    dims = nb.make_dims(Bt, L, Di, N, nb.BF16 if io == "bf16" else nb.F32)
    L_ = nb.lib()
    p = lambda x: ctypes.c_void_p(x.data_ptr()) if x is not None else None  # noqa: E731
    ybig, y = _padded(Bt * L * Di, dt)
    xbig, xf = _padded(Bt * Di * N, torch.float32)
    ck = torch.empty(nb.ckpt_bytes(dims) // 4, dtype=torch.float32, device="cuda")
    ws = nb.Workspace(nb.workspace_bytes(nb.OP_SCAN_FWD, dims), torch.device("cuda"))
    nb.check(L_.naju_scan_fwd(ctypes.byref(dims), p(t["h"]), p(t["a"]), p(t["b"]), p(t["B"]),
                              p(t["C"]), p(D), p(x0), p(y), p(xf), p(ck), ws.ptr, ws.nbytes,
                              nb.stream_handle()))
    nb.check_workspace(ws)
    big = {k: _padded(Bt * L * Di, dt) for k in ("dh", "da", "db")}
    big.update({k: _padded(Bt * L * N, dt) for k in ("dB", "dC")})
    big["dD"] = _padded(Di, torch.float32)
    big["dx0"] = _padded(Bt * Di * N, torch.float32)
    wsb = nb.Workspace(nb.workspace_bytes(nb.OP_SCAN_BWD, dims), torch.device("cuda"))
    o = {k: v[1] for k, v in big.items()}
    nb.check(L_.naju_scan_bwd(ctypes.byref(dims), p(t["h"]), p(t["a"]), p(t["b"]), p(t["B"]),
                              p(t["C"]), p(D), p(x0), p(ck), p(t["dy"]), p(dxf), p(o["dh"]),
                              p(o["da"]), p(o["db"]), p(o["dB"]), p(o["dC"]), p(o["dD"]),
                              p(o["dx0"]), wsb.ptr, wsb.nbytes, nb.stream_handle()))
    torch.cuda.synchronize()
    for name, (bg, _) in [("y", (ybig, y)), ("x_final", (xbig, xf))] + list(big.items()):
        pad = bg[:64].float().cpu().numpy(), bg[-64:].float().cpu().numpy()
        assert (pad[0] == SENT).all() and (pad[1] == SENT).all(), name
    yo, xfo = oracle.scan_fwd(d["h"], d["a"], d["b"], d["B"], d["C"], d["D"], d["x0"])
    assert_close("y", host(y).reshape(Bt, L, Di), yo, TOL[io])
    assert_close("x_final", host(xf).reshape(Bt, Di, N), xfo, TOL[io])
    ref = oracle.scan_bwd(d["h"], d["a"], d["b"], d["B"], d["C"], d["D"], d["x0"], d["dy"],
                          d["dx_final"])
    for k in ("dh", "da", "db", "dB", "dC", "dD", "dx0"):
        assert_close(k, host(o[k]).reshape(ref[k].shape), ref[k], TOL[io])


@pytest.mark.parametrize("sched", ["static", "dynamic", "global"])
@pytest.mark.parametrize("block", [False, True], ids=["scan", "block"])
def test_ticket_schedules_agree(block, sched):
    """Every ticket schedule of the matrix-core forward -- static, per-XCD queues,
    one queue in ticket order (the default; NAJU_FWD_TICKETS, read at each call) --
    computes the same results."""
    Bt, L, Di, N = 4, 2100, 264, 16
    d = inputs.draw(Bt, L, Di, N, io="bf16", seed=36, x0=True, block=block, conv_state=block)
    hk = "u" if block else "h"
    t = {k: to_dev(d[k], "bf16") for k in (hk, "a", "b", "B", "C") + (("z", "conv_state") if block else ())}
    D, x0 = f32_dev(d["D"]), f32_dev(d["x0"])

    def run():
        if block:
            return nb.block_fwd(t["u"], t["z"], f32_dev(d["conv_w"]), t["a"], t["b"], t["B"],
                                t["C"], D, x0, t["conv_state"], check_errors=True)[:2]
        return nb.scan_fwd(t["h"], t["a"], t["b"], t["B"], t["C"], D, x0, check_errors=True)
    y0, xf0 = run()
    old = os.environ.get("NAJU_FWD_TICKETS")
    os.environ["NAJU_FWD_TICKETS"] = sched
    try:
        ys = [run() for _ in range(3)]
    finally:
        if old is None:
            del os.environ["NAJU_FWD_TICKETS"]
        else:
            os.environ["NAJU_FWD_TICKETS"] = old
    torch.cuda.synchronize()
    for y1, xf1 in ys:
        assert_agree("y(%s)" % sched, host(y1), host(y0))
        e = np.abs(host(xf1) - host(xf0)).max() / np.abs(host(xf0)).max()
        assert e <= 1e-6, e
