"""GPU parity of the mixer layer (naju_mixer_fwd) against the fp64 oracle.

The oracle (oracle.mixer_fwd) is the block flowchart of the reproduction
README around the pinned block forward, with the intermediates stored in bf16
at the same points as the device path.  Both sides read the same bf16 inputs
and weights.  Tolerance: normwise relative error <= 2e-2 on the bf16 output,
as for the other bf16 entry points (the device's fp32 accumulation can flip
a bf16 rounding of an intermediate, which then propagates).
"""
import ctypes

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


# (with a residual of unit size the output is dominated by it after bf16 rounding, so
# most cases run without one, where the output is the projected scan result itself)
CASES = [
    # Bt, L, d_model, d_inner, d_state, residual, conv_state: ragged lengths, both state sizes
    (2, 200, 64, 128, 16, False, False),
    (1, 333, 96, 64, 64, False, True),
    (3, 130, 128, 256, 16, True, True),
    (2, 257, 64, 2048, 64, True, False),   # d_state 64 matrix-core form (32 rows)
    (1, 1, 32, 64, 16, False, True),       # one token: conv window entirely from conv_state
    (3, 17, 40, 72, 16, False, False),     # one partial conv segment, d_inner not a multiple of 64
    (2, 50, 16, 8, 64, False, True),       # the smallest d_inner, register form of the scan
    (8, 2048, 64, 128, 16, False, False),  # the training batch shape (16384 tokens), narrow layer
    (2, 256, 768, 1536, 16, True, True),   # the benchmarked layer width, fewer tokens
]

FP32_KEYS = ("conv_w", "D", "a_bias", "b_bias")


def run_case(Bt, L, dm, Di, N, residual, conv_state, seed):
    d = inputs.draw_mixer(Bt, L, dm, Di, N, seed=seed, residual=residual, conv_state=conv_state)
    print("mixer case Bt=%d L=%d dm=%d Di=%d N=%d res=%s cs=%s" % (Bt, L, dm, Di, N, residual,
                                                                  conv_state), flush=True)
    t = {k: (f32_dev(v) if k in FP32_KEYS else to_dev(v, "bf16")) for k, v in d.items()}
    out = nb.mixer_fwd(t["xn"], t["W_u"], t["W_z"], t["conv_w"], t["W_a"], t["a_bias"],
                       t["W_b"], t["b_bias"], t["W_B"], t["W_C"], t["D"], t["W_out"],
                       res=t.get("res"), conv_state=t.get("conv_state"))
    torch.cuda.synchronize()
    ref = oracle.mixer_fwd(d["xn"], d["W_u"], d["W_z"], d["conv_w"], d["W_a"], d["a_bias"],
                           d["W_b"], d["b_bias"], d["W_B"], d["W_C"], d["D"], d["W_out"],
                           res=d.get("res"), conv_state=d.get("conv_state"))
    return host(out), ref


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b%d_l%d_dm%d_d%d_n%d" % c[:5])
def test_mixer_matches_oracle(case):
    got, ref = run_case(*case, seed=77)
    assert np.isfinite(got).all()
    assert np.abs(ref["y"]).max() > 0.1 and np.abs(ref["out"]).max() > 0.1  # a non-trivial case
    assert_close("out", got, ref["out"], TOL["bf16"])


def test_mixer_repeat_calls_are_identical():
    """A second call on the same workspace (cached GEMM plans, the block
    forward's epoch-tagged look-back words) repeats the first within rounding:
    the look-back may fold predecessor chunks in a different order."""
    Bt, L, dm, Di, N = 2, 300, 64, 128, 16
    d = inputs.draw_mixer(Bt, L, dm, Di, N, seed=5)
    t = {k: (f32_dev(v) if k in FP32_KEYS else to_dev(v, "bf16")) for k, v in d.items()}
    args = (t["xn"], t["W_u"], t["W_z"], t["conv_w"], t["W_a"], t["a_bias"], t["W_b"],
            t["b_bias"], t["W_B"], t["W_C"], t["D"], t["W_out"])
    o1 = host(nb.mixer_fwd(*args, res=t["res"]))
    o2 = host(nb.mixer_fwd(*args, res=t["res"]))
    # the GEMMs repeat exactly; a look-back that folds a predecessor's aggregate
    # instead of taking its inclusive state changes only the fp32 rounding of the
    # block forward, so an output moves by at most a bf16 rounding flip or two
    assert_agree("repeat", o2, o1, ulps=2.0)


BWD_CASES = [
    # Bt, L, d_model, d_inner, d_state, conv_state
    (2, 200, 64, 128, 16, False),
    (1, 333, 96, 64, 64, True),
    (2, 130, 32, 256, 16, True),
    (8, 2048, 64, 128, 16, False),  # the training batch shape (16384 tokens), narrow layer
    # 3000 tokens: the weight gradients split over 4 token slices of 750
    (2, 1500, 64, 128, 16, False),
    # the benchmarked layer width, fewer tokens: the layer's dh = dB W_B^T + dC W_C^T
    # spreads any error of dB / dC over every channel of a token, so this case holds
    # the channel contractions of the block backward to near-fp32 accuracy
    (2, 256, 768, 1536, 16, True),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "b%d_l%d_dm%d_d%d_n%d" % c[:5])
def test_mixer_backward_matches_oracle(case):
    Bt, L, dm, Di, N, cs = case
    print("mixer bwd case Bt=%d L=%d dm=%d Di=%d N=%d cs=%s" % case, flush=True)
    d = inputs.draw_mixer(Bt, L, dm, Di, N, seed=91, residual=False, conv_state=cs)
    g = inputs.bf16_round(np.random.default_rng(92).standard_normal((Bt, L, dm)).astype(np.float32))
    t = {k: (f32_dev(v) if k in FP32_KEYS else to_dev(v, "bf16")) for k, v in d.items()}
    got = nb.mixer_bwd(t["xn"], t["W_u"], t["W_z"], t["conv_w"], t["W_a"], t["a_bias"],
                       t["W_b"], t["b_bias"], t["W_B"], t["W_C"], t["D"], t["W_out"],
                       to_dev(g, "bf16"), conv_state=t.get("conv_state"))
    torch.cuda.synchronize()
    ref = oracle.mixer_bwd(d["xn"], d["W_u"], d["W_z"], d["conv_w"], d["W_a"], d["a_bias"],
                           d["W_b"], d["b_bias"], d["W_B"], d["W_C"], d["D"], d["W_out"], g,
                           conv_state=d.get("conv_state"))
    names = ["dxn", "dW_u", "dW_z", "dconv_w", "dW_a", "da_bias", "dW_b", "db_bias", "dW_B",
             "dW_C", "dD", "dW_out"] + (["dconv_state"] if cs else [])
    for k in names:
        assert_close(k, host(got[k]), ref[k], TOL["bf16"])


@pytest.mark.parametrize("case", [(2, 200, 64, 128, 16, True), (8, 2048, 64, 128, 16, False)],
                         ids=lambda c: "b%d_l%d_dm%d_d%d_n%d" % c[:5])
def test_mixer_backward_reusing_forward_workspace(case):
    """The backward given the forward call's workspace (no recomputation) matches
    the oracle like the recomputing one."""
    Bt, L, dm, Di, N, cs = case
    print("mixer bwd (saved forward) case Bt=%d L=%d dm=%d Di=%d N=%d cs=%s" % case, flush=True)
    d = inputs.draw_mixer(Bt, L, dm, Di, N, seed=93, residual=False, conv_state=cs)
    g = inputs.bf16_round(np.random.default_rng(94).standard_normal((Bt, L, dm)).astype(np.float32))
    t = {k: (f32_dev(v) if k in FP32_KEYS else to_dev(v, "bf16")) for k, v in d.items()}
    W = (t["W_u"], t["W_z"], t["conv_w"], t["W_a"], t["a_bias"], t["W_b"], t["b_bias"], t["W_B"],
         t["W_C"], t["D"], t["W_out"])
    dims = nb.make_dims(Bt, L, Di, N, nb.BF16)
    fws = nb.Workspace(int(nb.lib().naju_mixer_workspace_bytes(ctypes.byref(dims), dm)),
                       t["xn"].device)
    nb.mixer_fwd(t["xn"], *W, conv_state=t.get("conv_state"), ws=fws)
    got = nb.mixer_bwd(t["xn"], *W, to_dev(g, "bf16"), conv_state=t.get("conv_state"),
                       fwd_ws=fws)
    torch.cuda.synchronize()
    ref = oracle.mixer_bwd(d["xn"], d["W_u"], d["W_z"], d["conv_w"], d["W_a"], d["a_bias"],
                           d["W_b"], d["b_bias"], d["W_B"], d["W_C"], d["D"], d["W_out"], g,
                           conv_state=d.get("conv_state"))
    for k in ["dxn", "dW_u", "dW_z", "dconv_w", "dW_a", "da_bias", "dW_b", "db_bias", "dW_B",
              "dW_C", "dD", "dW_out"] + (["dconv_state"] if cs else []):
        assert_close(k, host(got[k]), ref[k], TOL["bf16"])
