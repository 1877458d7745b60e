"""Seeded synthetic inputs for the Naju scan workloads.

This module holds no arithmetic of the method: it only draws random numbers
and rounds them to the storage type.  It is the one module shared by the
tests, the benchmark and the oracle's callers; the oracle itself never
imports it and it imports neither the oracle nor the HIP binding.

Distributions follow the pages' workloads: preserve-first gate biases
(forget pre-activation around +5, write pre-activation around -2, from the
"Core equations" section of the Naju reproduction README), unit normals for
the token activations and the B/C directions, and std 0.5 normals for the
width-4 depthwise convolution taps.  The long single-sequence workload uses a
forget pre-activation around +7 (near-lossless retention, f ~ 0.999).

Every array is drawn in float32 from ``numpy.random.default_rng(seed)`` in a
fixed order, then (for bf16 workloads) rounded to bfloat16 with
round-to-nearest-even.  The returned float32 arrays hold exactly the values
the device receives, so quantisation of the inputs is shared by both sides.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# draw order of the named arrays; a workload draws the subset it needs, in this order
DRAW_ORDER = ("h", "u", "a", "b", "B", "C", "D", "z", "conv_w", "x0", "dy", "dx_final",
              "conv_state")


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even; NaN kept quiet."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = np.isnan(x)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + r) >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 values (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16 (RNE), returned as float32."""
    return bf16_to_f32(bf16_bits(x))


@dataclass(frozen=True)
class Workload:
    """A named synthetic workload: shapes, io type and value distributions."""
    name: str
    Bt: int
    L: int
    Di: int
    N: int
    io: str = "bf16"          # "f32" or "bf16"
    K: int = 4                # conv width
    a_mu: float = 5.0         # forget-gate pre-activation mean (std 1)
    b_mu: float = -2.0        # write-gate pre-activation mean (std 1)
    seed: int = 1000
    block: bool = False       # draws u, z, conv_w instead of h
    backward: bool = False    # also draws dy
    chain: int = 1            # number of equal-length calls the sequence is split into
    extra: dict = field(default_factory=dict)

    @property
    def tokens(self) -> int:
        return self.Bt * self.L


# The five workloads of the hot path (named by what they are).
WORKLOADS = {
    "scan_f32_b1_l256_d192_n16": Workload("scan_f32_b1_l256_d192_n16", 1, 256, 192, 16,
                                          io="f32", seed=1000),
    "block_bf16_b8_l2048_d1536_n16": Workload("block_bf16_b8_l2048_d1536_n16", 8, 2048, 1536,
                                              16, seed=1001, block=True),
    "scan_bf16_b4_l8192_d4096_n64": Workload("scan_bf16_b4_l8192_d4096_n64", 4, 8192, 4096,
                                             64, seed=1002, chain=4),
    "scan_bf16_b1_l65536_d2048_n16": Workload("scan_bf16_b1_l65536_d2048_n16", 1, 65536, 2048,
                                              16, a_mu=7.0, seed=1003),
    "train_bf16_b8_l2048_d1536_n16": Workload("train_bf16_b8_l2048_d1536_n16", 8, 2048, 1536,
                                              16, seed=1004, block=True, backward=True),
    # forgetful gates (forget pre-activation around -2, f ~ 0.12): the product of
    # 1/f over 32 tokens is far past 2^64, so every chunk leaves the rescaled
    # matrix-core form and takes the register recurrence
    "scan_bf16_b8_l2048_d1536_n16_forget": Workload("scan_bf16_b8_l2048_d1536_n16_forget", 8,
                                                    2048, 1536, 16, a_mu=-2.0, seed=1006),
}


def draw(Bt: int, L: int, Di: int, N: int, *, io: str = "bf16", K: int = 4,
         a_mu: float = 5.0, b_mu: float = -2.0, seed: int = 0, block: bool = False,
         backward: bool = False, x0: bool = False, dx_final: bool = False,
         conv_state: bool = False) -> dict:
    """Draw one input set.  Returns a dict of float32 numpy arrays.

    Keys: h (scan) or u, z, conv_w (block); a, b [Bt,L,Di]; B, C [Bt,L,N]; D [Di];
    optional x0 [Bt,Di,N], dy [Bt,L,Di], dx_final [Bt,Di,N], conv_state [Bt,K-1,Di].
    Token activations and their gradients are rounded to the io type; D, conv_w and
    the fp32 states stay float32.
    """
    if io not in ("f32", "bf16"):
        raise ValueError("io must be 'f32' or 'bf16'")
    rng = np.random.default_rng(seed)
    tok = (Bt, L, Di)
    shapes = {
        "h": tok, "u": tok, "a": tok, "b": tok, "B": (Bt, L, N), "C": (Bt, L, N), "D": (Di,),
        "z": tok, "conv_w": (Di, K), "x0": (Bt, Di, N), "dy": tok, "dx_final": (Bt, Di, N),
        "conv_state": (Bt, K - 1, Di),
    }
    want = {"a", "b", "B", "C", "D"}
    want |= {"u", "z", "conv_w"} if block else {"h"}
    if backward:
        want.add("dy")
    if x0:
        want.add("x0")
    if dx_final:
        want.add("dx_final")
    if conv_state and block:
        want.add("conv_state")
    io_round = {"h", "u", "a", "b", "B", "C", "z", "dy", "conv_state"}
    out = {}
    for name in DRAW_ORDER:
        if name not in want:
            continue
        x = rng.standard_normal(shapes[name], dtype=np.float32)
        if name == "a":
            x += np.float32(a_mu)
        elif name == "b":
            x += np.float32(b_mu)
        elif name == "conv_w":
            x *= np.float32(0.5)
        if io == "bf16" and name in io_round:
            x = bf16_round(x)
        out[name] = x
    return out


def draw_workload(w: Workload, **kw) -> dict:
    """Draw the input set of a named workload (keyword overrides allowed)."""
    args = dict(io=w.io, K=w.K, a_mu=w.a_mu, b_mu=w.b_mu, seed=w.seed, block=w.block,
                backward=w.backward)
    args.update(kw)
    return draw(w.Bt, w.L, w.Di, w.N, **args)


# ------------------------------------------------------------ mixer layer
# The layer's weights are drawn so that its activations follow the same
# distributions as the scan workloads: u ~ N(0, 1) (W_u, W_z std 1/sqrt(d_model)
# on unit-normal tokens), and a = h W_a + 5, b = h W_b - 2 with unit spread,
# where h = SiLU(conv(u)) has mean square ~0.355 for std 0.5 taps (so W_a, W_b,
# W_B, W_C have std 1/sqrt(0.355 d_inner)); the gate biases are the page's
# preserve-first initialisation (5 and -2); W_out has std 1/sqrt(d_inner).
MIXER_DRAW_ORDER = ("xn", "res", "W_u", "W_z", "conv_w", "W_a", "W_b", "W_B", "W_C", "D",
                    "W_out", "conv_state")

MIXER_WORKLOADS = {
    "mixer_bf16_b8_l2048_dm768_d1536_n16": dict(Bt=8, L=2048, dm=768, Di=1536, N=16, seed=1005),
}


def draw_mixer(Bt: int, L: int, dm: int, Di: int, N: int, *, seed: int = 0,
               residual: bool = True, conv_state: bool = False, K: int = 4) -> dict:
    """One input set of the mixer layer (float32 arrays; bf16 ones already rounded)."""
    rng = np.random.default_rng(seed)
    h_ms = 0.355
    shapes = {"xn": (Bt, L, dm), "res": (Bt, L, dm), "W_u": (dm, Di), "W_z": (dm, Di),
              "conv_w": (Di, K), "W_a": (Di, Di), "W_b": (Di, Di), "W_B": (Di, N),
              "W_C": (Di, N), "D": (Di,), "W_out": (Di, dm), "conv_state": (Bt, K - 1, Di)}
    scale = {"W_u": dm ** -0.5, "W_z": dm ** -0.5, "conv_w": 0.5, "W_a": (h_ms * Di) ** -0.5,
             "W_b": (h_ms * Di) ** -0.5, "W_B": (h_ms * Di) ** -0.5, "W_C": (h_ms * Di) ** -0.5,
             "W_out": Di ** -0.5}
    fp32 = {"conv_w", "D"}
    out = {}
    for name in MIXER_DRAW_ORDER:
        if (name == "res" and not residual) or (name == "conv_state" and not conv_state):
            continue
        x = rng.standard_normal(shapes[name], dtype=np.float32)
        if name in scale:
            x *= np.float32(scale[name])
        out[name] = x if name in fp32 else bf16_round(x)
    out["a_bias"] = np.full(Di, 5.0, dtype=np.float32)
    out["b_bias"] = np.full(Di, -2.0, dtype=np.float32)
    return out
