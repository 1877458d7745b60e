"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small cases span several channel tiles and sequence chunks with ragged tails
(d_inner not a multiple of 64, seqlen not a multiple of 32/256), both io
types and both state sizes, with and without initial/conv states.  Edge
cases: a single token, empty sequences, non-finite gates.  Tolerance:
normwise relative error max|gpu - ref| / max|ref| <= 1e-4 (fp32 io) and
<= 2e-2 (bf16 io, fp32 state).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import TOL, assert_agree, assert_close, dev, f32_dev, host, to_dev
from selective_state_space_naju_amd import binding as nb
from selective_state_space_naju_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    nb.lib()


SMALL = [
    # Bt, L, Di, N, io
    (2, 300, 100, 16, "f32"),
    (2, 300, 100, 16, "bf16"),
    (1, 77, 40, 64, "f32"),
    (2, 530, 70, 64, "bf16"),
    (3, 1, 64, 16, "f32"),
    (1, 513, 129, 16, "bf16"),
    # bf16 with d_inner % 8 == 0 takes the matrix-core kernels: ragged channel
    # tiles, a partial last chunk, several look-back predecessors, more
    # tickets than resident workgroups
    (2, 300, 200, 16, "bf16"),
    (3, 1000, 136, 16, "bf16"),
    (4, 2100, 264, 16, "bf16"),
    # bf16, d_state 64, d_inner % 8 == 0: the staged register forward (a ragged
    # 16-channel tile, a partial last chunk)
    (2, 333, 72, 64, "bf16"),
    # bf16, d_state 64 with at least 32 rows of 64 channels: the matrix-core
    # forward (a ragged last tile, a partial last chunk with an idle wave)
    (2, 333, 1000, 64, "bf16"),
    # bf16, d_state 16, two channel tiles and 33 chunks: every chunk's predecessor
    # is resident at the same time, so the look-back publishes aggregates first and
    # walks long chains of them
    (1, 4100, 128, 16, "bf16"),
]


def ids(c):
    return "b%d_l%d_d%d_n%d_%s" % c


def scan_inputs(Bt, L, Di, N, io, seed, **kw):
    d = inputs.draw(Bt, L, Di, N, io=io, seed=seed, x0=True, backward=True, dx_final=True, **kw)
    return d


@pytest.mark.parametrize("case", SMALL, ids=ids)
def test_scan_fwd_parity(case):
    Bt, L, Di, N, io = case
    d = scan_inputs(Bt, L, Di, N, io, seed=11)
    print("scan_fwd", case, flush=True)
    ys, xf = oracle.scan_fwd(d["h"], d["a"], d["b"], d["B"], d["C"], d["D"], d["x0"])
    t = {k: to_dev(d[k], io) for k in ("h", "a", "b", "B", "C")}
    y, xg, ck = nb.scan_fwd(t["h"], t["a"], t["b"], t["B"], t["C"], f32_dev(d["D"]),
                            f32_dev(d["x0"]), return_ckpt=True)
    torch.cuda.synchronize()
    assert_close("y", host(y), ys, TOL[io])
    assert_close("x_final", host(xg), xf, TOL[io])
    # zero initial state
    ys0, xf0 = oracle.scan_fwd(d["h"], d["a"], d["b"], d["B"], d["C"], d["D"], None)
    y0, xg0 = nb.scan_fwd(t["h"], t["a"], t["b"], t["B"], t["C"], f32_dev(d["D"]))
    assert_close("y(x0=0)", host(y0), ys0, TOL[io])
    assert_close("xf(x0=0)", host(xg0), xf0, TOL[io])


@pytest.mark.parametrize("case", SMALL, ids=ids)
def test_block_fwd_parity(case):
    Bt, L, Di, N, io = case
    d = scan_inputs(Bt, L, Di, N, io, seed=12, block=True, conv_state=True)
    print("block_fwd", case, flush=True)
    yo, xfo, cso = oracle.block_fwd(d["u"], d["z"], d["conv_w"], d["a"], d["b"], d["B"], d["C"],
                                    d["D"], d["x0"], d["conv_state"])
    t = {k: to_dev(d[k], io) for k in ("u", "z", "a", "b", "B", "C", "conv_state")}
    y, xf, cs = nb.block_fwd(t["u"], t["z"], f32_dev(d["conv_w"]), t["a"], t["b"], t["B"], t["C"],
                             f32_dev(d["D"]), f32_dev(d["x0"]), t["conv_state"])
    torch.cuda.synchronize()
    assert_close("y", host(y), yo, TOL[io])
    assert_close("x_final", host(xf), xfo, TOL[io])
    assert np.array_equal(host(cs), cso)
    # no conv_state / no x0
    yo2, xfo2, cso2 = oracle.block_fwd(d["u"], d["z"], d["conv_w"], d["a"], d["b"], d["B"],
                                       d["C"], d["D"])
    y2, xf2, cs2 = nb.block_fwd(t["u"], t["z"], f32_dev(d["conv_w"]), t["a"], t["b"], t["B"],
                                t["C"], f32_dev(d["D"]))
    torch.cuda.synchronize()
    assert_close("y(no state)", host(y2), yo2, TOL[io])
    assert_close("xf(no state)", host(xf2), xfo2, TOL[io])
    assert np.array_equal(host(cs2), cso2)


def _grad_checks(names, got, ref, io):
    for k in names:
        assert_close(k, host(got[k]), ref[k], TOL[io])


@pytest.mark.parametrize("case", SMALL, ids=ids)
@pytest.mark.parametrize("use_ckpt", [True, False], ids=["ckpt", "recompute"])
def test_scan_bwd_parity(case, use_ckpt):
    Bt, L, Di, N, io = case
    d = scan_inputs(Bt, L, Di, N, io, seed=13)
    print("scan_bwd", case, use_ckpt, flush=True)
    ref = oracle.scan_bwd(d["h"], d["a"], d["b"], d["B"], d["C"], d["D"], d["x0"], d["dy"],
                          d["dx_final"])
    t = {k: to_dev(d[k], io) for k in ("h", "a", "b", "B", "C", "dy")}
    D, x0, dxf = f32_dev(d["D"]), f32_dev(d["x0"]), f32_dev(d["dx_final"])
    ck = None
    if use_ckpt:
        _, _, ck = nb.scan_fwd(t["h"], t["a"], t["b"], t["B"], t["C"], D, x0, return_ckpt=True)
    g = nb.scan_bwd(t["h"], t["a"], t["b"], t["B"], t["C"], D, t["dy"], x0, dxf, ck)
    torch.cuda.synchronize()
    _grad_checks(("dh", "da", "db", "dB", "dC", "dD", "dx0"), g, ref, io)


@pytest.mark.parametrize("case", SMALL, ids=ids)
@pytest.mark.parametrize("use_ckpt", [True, False], ids=["ckpt", "recompute"])
def test_block_bwd_parity(case, use_ckpt):
    Bt, L, Di, N, io = case
    d = scan_inputs(Bt, L, Di, N, io, seed=14, block=True, conv_state=True)
    print("block_bwd", case, use_ckpt, flush=True)
    ref = oracle.block_bwd(d["u"], d["z"], d["conv_w"], d["a"], d["b"], d["B"], d["C"], d["D"],
                           d["x0"], d["dy"], d["dx_final"], d["conv_state"])
    ref["du"], ref["dconv_w"] = ref["du"], ref["dw"]
    t = {k: to_dev(d[k], io) for k in ("u", "z", "a", "b", "B", "C", "dy", "conv_state")}
    D, x0, dxf, w = (f32_dev(d["D"]), f32_dev(d["x0"]), f32_dev(d["dx_final"]),
                     f32_dev(d["conv_w"]))
    ck = None
    if use_ckpt:
        *_, ck = nb.block_fwd(t["u"], t["z"], w, t["a"], t["b"], t["B"], t["C"], D, x0,
                              t["conv_state"], return_ckpt=True)
    g = nb.block_bwd(t["u"], t["z"], w, t["a"], t["b"], t["B"], t["C"], D, t["dy"], x0, dxf,
                     t["conv_state"], ck)
    torch.cuda.synchronize()
    _grad_checks(("du", "dz", "da", "db", "dB", "dC", "dD", "dx0", "dconv_w", "dconv_state"),
                 g, ref, io)


def test_empty_sequence_and_empty_batch():
    d = inputs.draw(2, 1, 64, 16, io="f32", seed=15, x0=True, block=True, conv_state=True)
    t = {k: to_dev(d[k], "f32") for k in ("u", "z", "a", "b", "B", "C", "conv_state")}
    e = {k: v[:, :0].contiguous() for k, v in t.items() if k != "conv_state"}
    x0 = f32_dev(d["x0"])
    y, xf, cs = nb.block_fwd(e["u"], e["z"], f32_dev(d["conv_w"]), e["a"], e["b"], e["B"], e["C"],
                             f32_dev(d["D"]), x0, t["conv_state"])
    torch.cuda.synchronize()
    assert y.numel() == 0
    assert torch.equal(xf, x0) and torch.equal(cs, t["conv_state"])
    y, xf = nb.scan_fwd(e["u"], e["a"], e["b"], e["B"], e["C"], f32_dev(d["D"]))
    torch.cuda.synchronize()
    assert not xf.any()
    z3 = torch.empty((0, 5, 64), device=dev())
    y, xf = nb.scan_fwd(z3, z3, z3, torch.empty((0, 5, 16), device=dev()),
                        torch.empty((0, 5, 16), device=dev()), f32_dev(d["D"]))
    assert y.shape == (0, 5, 64)


def test_lossless_retention_and_feedthrough():
    """a = +inf, b = -inf: x_final == x0 exactly; C = 0: y = D h (one rounding)."""
    Bt, L, Di, N = 2, 300, 96, 16
    d = inputs.draw(Bt, L, Di, N, io="f32", seed=16, x0=True)
    t = {k: to_dev(d[k], "f32") for k in ("h", "B", "C")}
    a = torch.full((Bt, L, Di), float("inf"), device=dev())
    b = torch.full((Bt, L, Di), float("-inf"), device=dev())
    x0 = f32_dev(d["x0"])
    y, xf = nb.scan_fwd(t["h"], a, b, t["B"], t["C"], f32_dev(d["D"]), x0)
    torch.cuda.synchronize()
    assert torch.equal(xf, x0)
    ys, _ = oracle.scan_fwd(d["h"], np.full((Bt, L, Di), np.inf), np.full((Bt, L, Di), -np.inf),
                            d["B"], d["C"], d["D"], d["x0"])
    assert_close("y", host(y), ys, TOL["f32"])
    Cz = torch.zeros_like(t["C"])
    y2, _ = nb.scan_fwd(t["h"], to_dev(d["a"], "f32"), to_dev(d["b"], "f32"), t["B"], Cz,
                        f32_dev(d["D"]), x0)
    torch.cuda.synchronize()
    ref = d["D"].astype(np.float32) * d["h"]
    assert np.array_equal(host(y2), ref.astype(np.float64))


def test_nonfinite_gates_follow_oracle():
    """f = 0 (a = -inf) resets the state; NaN in a gate stays in its channel."""
    Bt, L, Di, N = 1, 100, 64, 16
    d = inputs.draw(Bt, L, Di, N, io="f32", seed=17, x0=True)
    d["a"][0, 40, :8] = -np.inf
    d["a"][0, 70, 9] = np.nan
    ys, xf = oracle.scan_fwd(d["h"], d["a"], d["b"], d["B"], d["C"], d["D"], d["x0"])
    t = {k: to_dev(d[k], "f32") for k in ("h", "a", "b", "B", "C")}
    y, xg = nb.scan_fwd(t["h"], t["a"], t["b"], t["B"], t["C"], f32_dev(d["D"]), f32_dev(d["x0"]))
    torch.cuda.synchronize()
    yg = host(y)
    assert np.isnan(yg[0, 70:, 9]).all() and not np.isnan(np.delete(yg, 9, axis=2)).any()
    assert not np.isnan(yg[0, :70, 9]).any()
    m = ~np.isnan(ys)
    assert_close("y", yg[m], ys[m], TOL["f32"])


def test_repeat_runs_agree_and_workspace_clean():
    Bt, L, Di, N = 2, 2048, 256, 16
    d = inputs.draw(Bt, L, Di, N, io="bf16", seed=18)
    t = {k: to_dev(d[k], "bf16") for k in ("h", "a", "b", "B", "C")}
    ws = nb.Workspace(nb.workspace_bytes(nb.OP_SCAN_FWD, nb.make_dims(Bt, L, Di, N, nb.BF16)),
                      dev())
    outs = [nb.scan_fwd(t["h"], t["a"], t["b"], t["B"], t["C"], f32_dev(d["D"]), ws=ws)
            for _ in range(3)]
    torch.cuda.synchronize()
    assert ws.error_flags() == 0
    # Repeats may fold a look-back predecessor's aggregate where another run found
    # its inclusive state, which only changes the fp32 rounding: x_final agrees to
    # 1e-6 of its size, and a bf16 output at most by a rounding flip (1 ulp).
    y0, x0f = host(outs[0][0]), host(outs[0][1])
    for y, xf in outs[1:]:
        assert_agree("y(repeat)", host(y), y0)
        assert np.abs(host(xf) - x0f).max() <= 1e-6 * np.abs(x0f).max()


@pytest.mark.parametrize("block", [False, True], ids=["scan", "block"])
def test_mfma64_rows_beyond_grid(block):
    """d_state 64 matrix-core forward with more (batch row, 32-channel tile) rows
    than resident workgroups, so workgroups walk a second row: the carried state,
    per-channel constants and conv window restart at each row."""
    Bt, L, Di, N = (3, 200, 5600, 64) if not block else (2, 130, 8200, 64)
    d = inputs.draw(Bt, L, Di, N, io="bf16", seed=21, x0=True, block=block, conv_state=block)
    print("mfma64 rows", block, flush=True)
    D, x0 = f32_dev(d["D"]), f32_dev(d["x0"])
    if block:
        yo, xfo, cso = oracle.block_fwd(d["u"], d["z"], d["conv_w"], d["a"], d["b"], d["B"],
                                        d["C"], d["D"], d["x0"], d["conv_state"])
        t = {k: to_dev(d[k], "bf16") for k in ("u", "z", "a", "b", "B", "C", "conv_state")}
        y, xf, cs = nb.block_fwd(t["u"], t["z"], f32_dev(d["conv_w"]), t["a"], t["b"], t["B"],
                                 t["C"], D, x0, t["conv_state"])
        torch.cuda.synchronize()
        assert np.array_equal(host(cs), cso)
    else:
        yo, xfo = oracle.scan_fwd(d["h"], d["a"], d["b"], d["B"], d["C"], d["D"], d["x0"])
        t = {k: to_dev(d[k], "bf16") for k in ("h", "a", "b", "B", "C")}
        y, xf = nb.scan_fwd(t["h"], t["a"], t["b"], t["B"], t["C"], D, x0)
        torch.cuda.synchronize()
    assert_close("y", host(y), yo, TOL["bf16"])
    assert_close("x_final", host(xf), xfo, TOL["bf16"])


@pytest.mark.parametrize("N", [16, 64])
@pytest.mark.parametrize("block", [False, True], ids=["scan", "block"])
def test_bf16_fallback_chunks(block, N):
    """bf16 runs on the matrix-core paths; chunks whose prod(1/f) leaves the safe
    range (a = -inf, or a drawn wide so f is often tiny) or that hold a NaN gate
    are recomputed by the register recurrence.  Both kinds mix in one call.  (At
    d_state 64, 2 x 1024 channels make the 32 rows that select the matrix-core form.)"""
    Bt, L, Di = (2, 700, 160) if N == 16 else (2, 400, 1024)
    d = inputs.draw(Bt, L, Di, N, io="bf16", seed=19, x0=True, block=block, conv_state=block)
    d["a"][0, 100, :10] = -np.inf                      # f = 0: full reset
    d["a"][1, 300:364, 64:] = inputs.bf16_round(       # wide gates: prod(1/f) overflows
        (np.random.default_rng(3).standard_normal((64, Di - 64)) * 6 - 6).astype(np.float32))
    d["a"][1, min(500, L - 1), 5] = np.nan
    print("fallback", block, N, flush=True)
    hk = "u" if block else "h"
    t = {k: to_dev(d[k], "bf16") for k in (hk, "a", "b", "B", "C") + (("z", "conv_state") if block else ())}
    D, x0 = f32_dev(d["D"]), f32_dev(d["x0"])
    if block:
        ys, xf, _ = oracle.block_fwd(d["u"], d["z"], d["conv_w"], d["a"], d["b"], d["B"], d["C"],
                                     d["D"], d["x0"], d["conv_state"])
        y, xg, _ = nb.block_fwd(t["u"], t["z"], f32_dev(d["conv_w"]), t["a"], t["b"], t["B"], t["C"],
                                D, x0, t["conv_state"])
    else:
        ys, xf = oracle.scan_fwd(d["h"], d["a"], d["b"], d["B"], d["C"], d["D"], d["x0"])
        y, xg = nb.scan_fwd(t["h"], t["a"], t["b"], t["B"], t["C"], D, x0)
    torch.cuda.synchronize()
    yg, xgh = host(y), host(xg)
    assert np.array_equal(np.isnan(yg), np.isnan(ys))
    m = ~np.isnan(ys)
    assert_close("y", yg[m], ys[m], TOL["bf16"])
    mx = ~np.isnan(xf)
    assert_close("x_final", xgh[mx], xf[mx], TOL["bf16"])


@pytest.mark.parametrize("N", [16, 64])
@pytest.mark.parametrize("block", [False, True], ids=["scan", "block"])
def test_bf16_strongly_forgetting_gates(block, N):
    """Forget pre-activations around -3.5 (f ~ 0.03): a 32-token chunk's decay spans
    about 2^160, which only the pivoted factorisation (each half-chunk's product of
    1/f bounded) keeps on the matrix cores; the few half-chunks past the bound take
    the register recurrence.  Forward and backward against the oracle (at d_state 64
    the forward takes its matrix-core form, 32 rows of 64 channels)."""
    Bt, L, Di = (2, 500, 128) if N == 16 else (2, 300, 1024)
    d = inputs.draw(Bt, L, Di, N, io="bf16", seed=29, a_mu=-3.5, x0=True, backward=True,
                    dx_final=True, block=block, conv_state=block)
    print("strongly forgetting", block, N, flush=True)
    D, x0, dxf = f32_dev(d["D"]), f32_dev(d["x0"]), f32_dev(d["dx_final"])
    if block:
        t = {k: to_dev(d[k], "bf16") for k in ("u", "z", "a", "b", "B", "C", "dy", "conv_state")}
        w = f32_dev(d["conv_w"])
        y, xf, _, ck = nb.block_fwd(t["u"], t["z"], w, t["a"], t["b"], t["B"], t["C"], D, x0,
                                    t["conv_state"], return_ckpt=True)
        g = nb.block_bwd(t["u"], t["z"], w, t["a"], t["b"], t["B"], t["C"], D, t["dy"], x0, dxf,
                         t["conv_state"], ck)
        ys, xs, _ = oracle.block_fwd(d["u"], d["z"], d["conv_w"], d["a"], d["b"], d["B"], d["C"],
                                     d["D"], d["x0"], d["conv_state"])
        ref = oracle.block_bwd(d["u"], d["z"], d["conv_w"], d["a"], d["b"], d["B"], d["C"], d["D"],
                               d["x0"], d["dy"], d["dx_final"], d["conv_state"])
        ref["dconv_w"] = ref["dw"]
        names = ("du", "dz", "da", "db", "dB", "dC", "dD", "dx0", "dconv_w", "dconv_state")
    else:
        t = {k: to_dev(d[k], "bf16") for k in ("h", "a", "b", "B", "C", "dy")}
        y, xf, ck = nb.scan_fwd(t["h"], t["a"], t["b"], t["B"], t["C"], D, x0, return_ckpt=True)
        g = nb.scan_bwd(t["h"], t["a"], t["b"], t["B"], t["C"], D, t["dy"], x0, dxf, ckpt=ck)
        ys, xs = oracle.scan_fwd(d["h"], d["a"], d["b"], d["B"], d["C"], d["D"], d["x0"])
        ref = oracle.scan_bwd(d["h"], d["a"], d["b"], d["B"], d["C"], d["D"], d["x0"], d["dy"],
                              d["dx_final"])
        names = ("dh", "da", "db", "dB", "dC", "dD", "dx0")
    torch.cuda.synchronize()
    assert_close("y", host(y), ys, TOL["bf16"])
    assert_close("x_final", host(xf), xs, TOL["bf16"])
    _grad_checks(names, g, ref, "bf16")


@pytest.mark.parametrize("block", [False, True], ids=["scan", "block"])
def test_bf16_bwd_fallback_chunks(block):
    """Backward on the matrix-core path with chunks it must hand to the plain reverse
    recurrence (f = 0 resets, very wide forget gates), mixed with ordinary chunks."""
    Bt, L, Di, N = 2, 300, 128, 16
    d = inputs.draw(Bt, L, Di, N, io="bf16", seed=23, x0=True, backward=True, dx_final=True,
                    block=block, conv_state=block)
    d["a"][0, 40, :5] = -np.inf
    d["a"][1, 130:160, 70:] = inputs.bf16_round(
        (np.random.default_rng(4).standard_normal((30, Di - 70)) * 6 - 6).astype(np.float32))
    print("bwd fallback", block, flush=True)
    D, x0, dxf = f32_dev(d["D"]), f32_dev(d["x0"]), f32_dev(d["dx_final"])
    if block:
        ref = oracle.block_bwd(d["u"], d["z"], d["conv_w"], d["a"], d["b"], d["B"], d["C"], d["D"],
                               d["x0"], d["dy"], d["dx_final"], d["conv_state"])
        ref["dconv_w"] = ref["dw"]
        t = {k: to_dev(d[k], "bf16") for k in ("u", "z", "a", "b", "B", "C", "dy", "conv_state")}
        g = nb.block_bwd(t["u"], t["z"], f32_dev(d["conv_w"]), t["a"], t["b"], t["B"], t["C"], D,
                         t["dy"], x0, dxf, t["conv_state"])
        names = ("du", "dz", "da", "db", "dB", "dC", "dD", "dx0", "dconv_w", "dconv_state")
    else:
        ref = oracle.scan_bwd(d["h"], d["a"], d["b"], d["B"], d["C"], d["D"], d["x0"], d["dy"],
                              d["dx_final"])
        t = {k: to_dev(d[k], "bf16") for k in ("h", "a", "b", "B", "C", "dy")}
        g = nb.scan_bwd(t["h"], t["a"], t["b"], t["B"], t["C"], D, t["dy"], x0, dxf)
        names = ("dh", "da", "db", "dB", "dC", "dD", "dx0")
    torch.cuda.synchronize()
    _grad_checks(names, g, ref, "bf16")
    # the workspace was left clean: a second call agrees with the first
    g2 = (nb.block_bwd(t["u"], t["z"], f32_dev(d["conv_w"]), t["a"], t["b"], t["B"], t["C"], D,
                       t["dy"], x0, dxf, t["conv_state"]) if block else
          nb.scan_bwd(t["h"], t["a"], t["b"], t["B"], t["C"], D, t["dy"], x0, dxf))
    torch.cuda.synchronize()
    # (the checkpoints are recomputed by the forward, whose look-back may fold a
    # predecessor's aggregate in one call and read its inclusive state in the other:
    # rounding only)
    for k in names:
        assert_agree(k + "(2nd)", host(g2[k]), host(g[k]), ulps=2.0)
