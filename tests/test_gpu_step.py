"""GPU parity of the one-token (decode) step entry points against the fp64 oracle.

The step is the sequence forward on one token with the state carried in
place, so the oracle is oracle.scan_fwd / oracle.block_fwd on a one-token
sequence with x0 = x (and conv_state), whose x_final (and conv_state_out) are
what the step leaves in x (and conv_state).  A run of T steps must also equal
the oracle's forward over the whole T-token sequence.  Tolerance as for the
sequence kernels: normwise relative error <= 1e-4 (fp32 io), <= 2e-2 (bf16 io).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import TOL, assert_close, dev, f32_dev, host, to_dev
from selective_state_space_naju_amd import binding as nb
from selective_state_space_naju_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    nb.lib()


CASES = [
    # Bt, Di, N, io: ragged channel counts (a partial last workgroup), both state sizes
    (3, 100, 16, "f32"),
    (2, 300, 16, "bf16"),
    (2, 70, 64, "bf16"),
    (1, 129, 64, "f32"),
]


def ids(c):
    return "b%d_d%d_n%d_%s" % c


@pytest.mark.parametrize("case", CASES, ids=ids)
def test_scan_step_one_token(case):
    Bt, Di, N, io = case
    d = inputs.draw(Bt, 1, Di, N, io=io, seed=31, x0=True)
    print("scan_step", case, flush=True)
    ys, xf = oracle.scan_fwd(d["h"], d["a"], d["b"], d["B"], d["C"], d["D"], d["x0"])
    x = f32_dev(d["x0"])
    y = nb.scan_step(to_dev(d["h"][:, 0], io), to_dev(d["a"][:, 0], io), to_dev(d["b"][:, 0], io),
                     to_dev(d["B"][:, 0], io), to_dev(d["C"][:, 0], io), f32_dev(d["D"]), x)
    torch.cuda.synchronize()
    assert_close("y", host(y), ys[:, 0], TOL[io])
    assert_close("x", host(x), xf, TOL[io])


@pytest.mark.parametrize("case", CASES, ids=ids)
def test_block_step_one_token(case):
    Bt, Di, N, io = case
    d = inputs.draw(Bt, 1, Di, N, io=io, seed=32, block=True, x0=True, conv_state=True)
    print("block_step", case, flush=True)
    yo, xfo, cso = oracle.block_fwd(d["u"], d["z"], d["conv_w"], d["a"], d["b"], d["B"], d["C"],
                                    d["D"], d["x0"], d["conv_state"])
    x = f32_dev(d["x0"])
    cs = to_dev(d["conv_state"], io)
    y = nb.block_step(to_dev(d["u"][:, 0], io), to_dev(d["z"][:, 0], io), f32_dev(d["conv_w"]), cs,
                      to_dev(d["a"][:, 0], io), to_dev(d["b"][:, 0], io), to_dev(d["B"][:, 0], io),
                      to_dev(d["C"][:, 0], io), f32_dev(d["D"]), x)
    torch.cuda.synchronize()
    assert_close("y", host(y), yo[:, 0], TOL[io])
    assert_close("x", host(x), xfo, TOL[io])
    # the shifted conv window holds input values: exact
    assert np.array_equal(host(cs), cso)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_steps_equal_the_sequence(io):
    """T decode steps = the forward over the T-token sequence (scan and block)."""
    Bt, T, Di, N = 2, 40, 96, 16
    d = inputs.draw(Bt, T, Di, N, io=io, seed=33, x0=True, block=True, conv_state=True)
    d["h"] = d["u"]
    print("steps", io, flush=True)
    ys, xf = oracle.scan_fwd(d["h"], d["a"], d["b"], d["B"], d["C"], d["D"], d["x0"])
    yo, xfo, cso = oracle.block_fwd(d["u"], d["z"], d["conv_w"], d["a"], d["b"], d["B"], d["C"],
                                    d["D"], d["x0"], d["conv_state"])
    t = {k: to_dev(d[k], io) for k in ("h", "u", "z", "a", "b", "B", "C")}
    D, cw = f32_dev(d["D"]), f32_dev(d["conv_w"])
    xs, xb = f32_dev(d["x0"]), f32_dev(d["x0"])
    cs = to_dev(d["conv_state"], io)
    gs, gb = [], []
    for n in range(T):
        col = lambda k: t[k][:, n].contiguous()
        gs.append(nb.scan_step(col("h"), col("a"), col("b"), col("B"), col("C"), D, xs))
        gb.append(nb.block_step(col("u"), col("z"), cw, cs, col("a"), col("b"), col("B"), col("C"),
                                D, xb))
    torch.cuda.synchronize()
    assert_close("scan y", host(torch.stack(gs, 1)), ys, TOL[io])
    assert_close("scan x", host(xs), xf, TOL[io])
    assert_close("block y", host(torch.stack(gb, 1)), yo, TOL[io])
    assert_close("block x", host(xb), xfo, TOL[io])
    assert np.array_equal(host(cs), cso)


def test_step_empty_batch_is_a_noop():
    x = torch.zeros((0, 64, 16), dtype=torch.float32, device=dev())
    e = torch.zeros((0, 64), dtype=torch.bfloat16, device=dev())
    eB = torch.zeros((0, 16), dtype=torch.bfloat16, device=dev())
    y = nb.scan_step(e, e, e, eB, eB, torch.zeros(64, device=dev()), x)
    torch.cuda.synchronize()
    assert y.shape == (0, 64)
