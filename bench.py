"""Benchmark of the Naju scan hot path on one MI355X.

A step is one pass of the whole hot path over one batch of the training
workload (batch 8, seqlen 2048, d_inner 1536, d_state 16, bf16 activations,
fp32 state): the fused block forward (conv+SiLU front end, gates, scan,
readout, SiLU(z) modulation, checkpoints) followed by the block backward
(reverse-time adjoint scan, every gradient).  Inputs are synthetic, drawn by
the seeded generator, and resident in HBM before timing starts; three input
sets rotate so the 256 MB Infinity Cache cannot hold a step's working set.

The same run also times, as ``parts`` (per-launch HIP events on the launch
stream; median, mean, p10 and p90 over at least 50 launches):

* the scan forward alone and the block forward / backward alone at the step's
  shape, and the one-token decode step at its batch and width;
* every other workload of the hot path: the fp32 1 x 256 x 192 scan, the
  4 x 8192 x 4096 d_state-64 scan (one call, and the same sequence as 4 chained
  calls of 2048 tokens carrying the state), the 1 x 65536 x 2048 long scan, the
  step's scan shape with forgetful gates (forget pre-activations ~ N(-2, 1)),
  and the mixer layer around the scan (8 x 2048, d_model 768, d_inner 1536);
* the CPU oracle (the cpu_baseline leg) on a bounded sample of each workload,
  on the host's cores and, for the fp32 1 x 256 x 192 scan, on one thread.

`--workload NAME` instead prints the line of one named scan workload
(naju_scan_fwd alone) or of the mixer workload (forward + backward step).

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "scan tokens/sec + achieved HBM GB/s (% peak), fwd and fwd+bwd, L=2048"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak
WORKLOAD = "train_bf16_b8_l2048_d1536_n16"
MIXER = "mixer_bf16_b8_l2048_dm768_d1536_n16"
# the other workloads of the hot path, timed as parts of the default run
SCAN_PARTS = ("scan_f32_b1_l256_d192_n16", "scan_bf16_b4_l8192_d4096_n64",
              "scan_bf16_b1_l65536_d2048_n16", "scan_bf16_b8_l2048_d1536_n16_forget")
NSETS = 3
MIN_LAUNCHES = 50

FWD_SRC = ("selective_state_space_naju_amd/csrc/naju_fwd_mfma.hip",
           "selective_state_space_naju_amd/csrc/naju_mfma.h",
           "selective_state_space_naju_amd/csrc/naju_device.h",
           "selective_state_space_naju_amd/csrc/naju_launch.h")
FWD64_SRC = ("selective_state_space_naju_amd/csrc/naju_fwd_mfma64.hip",) + FWD_SRC[1:]
BWD_SRC = ("selective_state_space_naju_amd/csrc/naju_bwd_mfma.hip",
           "selective_state_space_naju_amd/csrc/naju_bwd.hip",
           "selective_state_space_naju_amd/csrc/naju_device.h",
           "selective_state_space_naju_amd/csrc/naju_launch.h")


def alg_bytes(kind, Bt, L, Di, N, e, K=4):
    """Algorithmic HBM bytes of one call (what the method must move)."""
    tok, st = Bt * L * Di, Bt * Di * N
    if kind == "scan_fwd":     # read h, a, b; write y; B, C; x_final; D
        return tok * 4 * e + Bt * L * N * 2 * e + st * 4 + Di * 4
    if kind == "scan_fwd_x0":  # the same, also reading the initial state
        return tok * 4 * e + Bt * L * N * 2 * e + st * 8 + Di * 4
    if kind == "block_fwd":    # read u, z, a, b; write y; B, C; x_final; D, conv_w
        return tok * 5 * e + Bt * L * N * 2 * e + st * 4 + Di * 4 + Di * K * 4
    if kind == "block_bwd":    # read u, z, a, b, dy; write du, dz, da, db; B, C, dB, dC; D, dD, w, dw
        return tok * 9 * e + Bt * L * N * 4 * e + Di * 4 * 2 + Di * K * 4 * 2
    if kind == "block_step":   # state read + write, u z a b read, y write, conv window r + w, B C, D, w
        return Bt * Di * N * 8 + Bt * Di * 5 * e + Bt * (K - 1) * Di * e * 2 + Bt * N * 2 * e + Di * 4 * 5
    raise ValueError(kind)


def measured_traffic(md_name, sources):
    """Per-launch HBM bytes from a committed rocprofv3 counter summary, or None when
    there is none or the kernel sources changed since the counters were taken."""
    if not md_name:
        return None
    path = os.path.join(ROOT, "profiles", md_name)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.split(":")[0] in ("traffic_bytes_per_launch", "source_sha256_16"):
            k, v = line.split(":", 1)
            fields[k] = v.split()[0]
    h = hashlib.sha256()
    for f in sources:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if fields.get("source_sha256_16") != h.hexdigest()[:16]:
        return None
    return int(fields["traffic_bytes_per_launch"])


def stats_ms(tt):
    """Summary of per-launch durations in ms."""
    tt = np.asarray(tt, dtype=np.float64)
    r = lambda v: round(float(v), 4)  # noqa: E731
    return {"ms_median": r(np.median(tt)), "ms_mean": r(tt.mean()),
            "ms_p10": r(np.percentile(tt, 10)), "ms_p90": r(np.percentile(tt, 90)),
            "launches": int(tt.size)}


def hbm_part(tt, by, tokens, **extra):
    """A part bound by HBM: timing statistics, tokens/s and GB/s at the median."""
    e = dict(extra)
    e.update(stats_ms(tt))
    s = e["ms_median"] * 1e-3
    e.update(tokens_per_s=round(tokens / s, 1), alg_bytes=int(by),
             GB_per_s=round(by / s / 1e9, 1), pct_hbm_peak=round(100 * by / s / 1e9 / HBM_PEAK_GBS, 2))
    return e


def roofline_hbm(part, kernel, traffic=None):
    """Roofline of an HBM-bound part at its mean launch duration (the figure a
    rocprofv3 kernel trace averages)."""
    by, ms = part["alg_bytes"], part["ms_mean"]
    ach = by / (ms * 1e-3) / 1e9
    return {"kernel": kernel, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
            "ms_per_launch": round(ms, 4), "alg_bytes_per_launch": int(by)}


class Timer:
    """Per-launch GPU durations from HIP events recorded on torch's current stream
    (the stream every call below is launched on)."""

    def __init__(self, torch):
        self.torch = torch

    def launches(self, fn, count):
        torch = self.torch
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(count)]
        torch.cuda.synchronize()
        for k in range(count):
            ev[k][0].record()
            fn(k)
            ev[k][1].record()
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in ev])


def scan_workload_parts(name, torch, nb, inputs, warmup, launches, keep_sample=None):
    """naju_scan_fwd on a named scan workload (inputs resident in HBM, two input
    sets alternating), and for a chained workload the same sequence as equal
    calls carrying the state.  Returns (parts, roofline)."""
    w = inputs.WORKLOADS[name]
    Bt, L, Di, N = w.Bt, w.L, w.Di, w.N
    e = 2 if w.io == "bf16" else 4
    dev = torch.device("cuda:0")
    io_t = torch.bfloat16 if w.io == "bf16" else torch.float32
    d = inputs.draw_workload(w)
    if keep_sample is not None:
        keep_sample(d)
    base = {k: torch.from_numpy(d[k]).to(io_t).to(dev) for k in ("h", "a", "b", "B", "C")}
    D = torch.from_numpy(d["D"]).to(dev)
    del d
    sets = [base, {k: v.clone() for k, v in base.items()}]
    L_, stream = nb.lib(), nb.stream_handle(dev)
    p = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731
    dims = nb.make_dims(Bt, L, Di, N, nb.BF16 if w.io == "bf16" else nb.F32)
    ws = nb.Workspace(nb.workspace_bytes(nb.OP_SCAN_FWD, dims), dev)
    y = torch.empty((Bt, L, Di), dtype=io_t, device=dev)
    xf = torch.empty((Bt, Di, N), dtype=torch.float32, device=dev)

    def call(i):
        s = sets[i % 2]
        nb.check(L_.naju_scan_fwd(ctypes.byref(dims), p(s["h"]), p(s["a"]), p(s["b"]),
                                  p(s["B"]), p(s["C"]), p(D), None, p(y), p(xf), None, ws.ptr,
                                  ws.nbytes, stream))
    timer = Timer(torch)
    for k in range(warmup):
        call(k)
    tt = timer.launches(call, launches)
    parts = {}
    kind = "scan_fwd"
    parts["scan_fwd[%s]" % name] = hbm_part(tt, alg_bytes(kind, Bt, L, Di, N, e), Bt * L)
    if N == 64 and e == 2:
        kernel = "naju::fwd_mfma64_kernel<false> (naju_scan_fwd)"
        traffic = measured_traffic("hbm_traffic_fwd_mfma64_%s.md" % name, FWD64_SRC)
    elif N == 16 and e == 2:
        kernel = "naju::fwd_chunk_kernel<false> (naju_scan_fwd)"
        traffic = measured_traffic("hbm_traffic_fwd_chunk_%s.md" % name, FWD_SRC)
    else:
        kernel = "naju_scan_fwd, fp32 register recurrence (d_state %d)" % N
        traffic = None
    rf = roofline_hbm(parts["scan_fwd[%s]" % name], kernel, traffic)

    if w.chain > 1:
        # the same sequence as w.chain calls of L / chain tokens, each starting
        # from the previous call's final state
        Ls = L // w.chain
        seg = [[{k: v[:, c * Ls:(c + 1) * Ls].contiguous() for k, v in s.items()}
                for c in range(w.chain)] for s in sets]
        cd = nb.make_dims(Bt, Ls, Di, N, nb.BF16 if w.io == "bf16" else nb.F32)
        cws = nb.Workspace(nb.workspace_bytes(nb.OP_SCAN_FWD, cd), dev)
        ys = [torch.empty((Bt, Ls, Di), dtype=io_t, device=dev) for _ in range(w.chain)]
        xs = [torch.empty((Bt, Di, N), dtype=torch.float32, device=dev) for _ in range(w.chain)]

        def chain(i):
            for c in range(w.chain):
                s = seg[i % 2][c]
                nb.check(L_.naju_scan_fwd(ctypes.byref(cd), p(s["h"]), p(s["a"]), p(s["b"]),
                                          p(s["B"]), p(s["C"]), p(D),
                                          p(xs[c - 1]) if c else None, p(ys[c]), p(xs[c]), None,
                                          cws.ptr, cws.nbytes, stream))
        for k in range(warmup):
            chain(k)
        tc = timer.launches(chain, launches)
        by = w.chain * alg_bytes("scan_fwd_x0", Bt, Ls, Di, N, e)
        parts["scan_fwd_chain%d[%s]" % (w.chain, name)] = hbm_part(
            tc, by, Bt * L, what="%d chained naju_scan_fwd calls of %d tokens, state carried "
                                  "through x0 / x_final" % (w.chain, Ls))
        if cws.error_flags():
            raise RuntimeError("a cross-workgroup wait gave up: results invalid")
        del seg, ys, xs, cws
    if ws.error_flags():
        raise RuntimeError("a cross-workgroup wait gave up: results invalid")
    del sets, base, y, xf, ws
    torch.cuda.empty_cache()
    return parts, rf


def mixer_parts(torch, nb, inputs, warmup, launches, keep_sample=None):
    """naju_mixer_fwd, naju_mixer_bwd and a forward + backward step on the mixer
    workload, weights and inputs resident in HBM; also the block forward alone at
    the same shape (the scan inside the layer).  Returns (parts, roofline, t_step)."""
    c = inputs.MIXER_WORKLOADS[MIXER]
    Bt, L, dm, Di, N = c["Bt"], c["L"], c["dm"], c["Di"], c["N"]
    dev = torch.device("cuda:0")
    d = inputs.draw_mixer(Bt, L, dm, Di, N, seed=c["seed"])
    if keep_sample is not None:
        keep_sample(d)
    f32 = ("conv_w", "D", "a_bias", "b_bias")
    t = {k: torch.from_numpy(v).to(torch.float32 if k in f32 else torch.bfloat16).to(dev)
         for k, v in d.items()}
    del d
    sets = [t["xn"], t["xn"].roll(1, 0).contiguous()]
    res = [t["res"], t["res"].roll(1, 0).contiguous()]
    dims = nb.make_dims(Bt, L, Di, N, nb.BF16)
    fws = nb.Workspace(int(nb.lib().naju_mixer_workspace_bytes(ctypes.byref(dims), dm)), dev)
    g_out = [torch.randn_like(sets[0], dtype=torch.float32).to(torch.bfloat16) for _ in range(2)]
    W = [t[k] for k in ("W_u", "W_z", "conv_w", "W_a", "a_bias", "W_b", "b_bias", "W_B", "W_C",
                        "D", "W_out")]

    def fwd(i):
        nb.mixer_fwd(sets[i % 2], *W, res=res[i % 2], ws=fws)

    def bwd(i):
        nb.mixer_bwd(sets[i % 2], *W, g_out[i % 2])

    def step(i):  # a training step: the backward reuses the forward's workspace
        fwd(i)
        nb.mixer_bwd(sets[i % 2], *W, g_out[i % 2], fwd_ws=fws)
    timer = Timer(torch)
    for k in range(warmup):
        fwd(k)
        bwd(k)
    tf = timer.launches(fwd, launches)
    tb = timer.launches(bwd, launches)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(launches):
        step(k)
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t0) / launches
    ts = timer.launches(step, launches)
    # the block scan of the same shape alone (synthetic u, z, a, b, B, C)
    wb = inputs.Workload("mixer_scan_part", Bt, L, Di, N, seed=c["seed"] + 1, block=True)
    db = inputs.draw_workload(wb)
    bt = {k: torch.from_numpy(db[k]).to(torch.bfloat16).to(dev)
          for k in ("u", "z", "a", "b", "B", "C")}
    bD, bw = torch.from_numpy(db["D"]).to(dev), torch.from_numpy(db["conv_w"]).to(dev)
    del db
    blk = lambda i: nb.block_fwd(bt["u"], bt["z"], bw, bt["a"], bt["b"], bt["B"], bt["C"], bD)  # noqa: E731
    for k in range(warmup):
        blk(k)
    tk = timer.launches(blk, launches)
    flops = 2.0 * Bt * L * (2 * dm * Di + 2 * Di * Di + 2 * Di * N + Di * dm)
    ms, ms_b = float(tf.mean()), float(tk.mean())
    parts = {
        "mixer_fwd[%s]" % MIXER: dict(stats_ms(tf), tokens_per_s=round(Bt * L / (ms * 1e-3), 1),
                                      gemm_flops=int(flops),
                                      TFLOP_per_s_over_call=round(flops / (ms * 1e-3) / 1e12, 1)),
        "mixer_bwd[%s]" % MIXER: dict(stats_ms(tb), gemm_flops=int(3 * flops),
                                      what="naju_mixer_bwd alone (recomputes the forward)"),
        "mixer_step[%s]" % MIXER: dict(stats_ms(ts), tokens_per_s=round(Bt * L / t_step, 1),
                                       what="naju_mixer_fwd + naju_mixer_bwd reusing the "
                                            "forward's workspace"),
        "block_fwd_same_shape[%s]" % MIXER: stats_ms(tk),
    }
    ach_g = flops / ((ms - ms_b) * 1e-3) / 1e12
    rf = {"kernel": "the call's hipBLASLt projections (bf16, fp32 accumulation); time = mixer "
                    "call minus the block forward alone",
          "bound": "mfma", "achieved": round(ach_g, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
          "unit": "TFLOP/s", "frac": round(ach_g / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
          "ms_per_launch": round(ms - ms_b, 4), "alg_flops_per_launch": int(flops)}
    del t, sets, res, fws, g_out, W, bt
    torch.cuda.empty_cache()
    return parts, rf, t_step


# one-thread oracle timing of the fp32 1 x 256 x 192 scan, in a child process
# (the oracle's OpenMP team size is fixed when its library loads)
_ONE_THREAD = r"""
import sys, time, json
sys.path.insert(0, sys.argv[1])
import oracle
from selective_state_space_naju_amd import inputs
d = inputs.draw_workload(inputs.WORKLOADS["scan_f32_b1_l256_d192_n16"])
oracle.scan_fwd(d["h"], d["a"], d["b"], d["B"], d["C"], d["D"])
reps, t0 = 0, time.perf_counter()
while time.perf_counter() - t0 < 1.0:
    oracle.scan_fwd(d["h"], d["a"], d["b"], d["B"], d["C"], d["D"])
    reps += 1
print(json.dumps({"s_per_call": (time.perf_counter() - t0) / reps, "calls": reps}))
"""


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the cpu_baseline leg")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the parts of the other workloads (scan configs, mixer)")
    ap.add_argument("--only", choices=["all", "scan_fwd", "step", "copy"], default="all",
                    help="restrict the timed work (for profiling runs); 'copy' runs a plain "
                         "1 GiB device copy, the reference for HBM byte counters")
    ap.add_argument("--workload", default=WORKLOAD,
                    help="another named scan workload (naju_scan_fwd alone) or the mixer "
                         "workload (forward + backward step)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the Naju scan path has no multi-GPU "
              "implementation here (it would shard over batch rows, over channels with B and C "
              "replicated, or over sequence segments chained through the x0 input).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from selective_state_space_naju_amd import binding as nb
    from selective_state_space_naju_amd import inputs

    dev = torch.device("cuda:0")
    launches = max(args.steps, MIN_LAUNCHES)

    def plain_copy(nbytes, warmup, steps):
        """A plain device copy of nbytes (the HIP runtime's copy kernel): seconds per copy."""
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(warmup):
            dst.copy_(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / steps
        del src, dst
        return dt

    if args.only == "copy":
        nbytes = 1 << 30
        dt = plain_copy(nbytes, args.warmup, args.steps)
        print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes,
                          "ms": round(dt * 1e3, 4), "GB_per_s": round(2 * nbytes / dt / 1e9, 1)}))
        return
    if args.workload == MIXER:
        return bench_mixer_workload(args, torch, nb, inputs)
    if args.workload != WORKLOAD:
        return bench_scan_workload(args, torch, nb, inputs)
    w = inputs.WORKLOADS[WORKLOAD]
    Bt, L, Di, N = w.Bt, w.L, w.Di, w.N
    e = 2
    L_ = nb.lib()
    d = inputs.draw_workload(w)
    bf = lambda k: torch.from_numpy(d[k]).to(torch.bfloat16).to(dev)  # noqa: E731
    f32 = lambda k: torch.from_numpy(d[k]).to(dev)  # noqa: E731
    base = {k: bf(k) for k in ("u", "z", "a", "b", "B", "C", "dy")}
    D, cw = f32("D"), f32("conv_w")
    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(NSETS - 1)]
    dims = nb.make_dims(Bt, L, Di, N, nb.BF16)
    stream = nb.stream_handle(dev)
    p = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731

    def alloc_outs():
        o = {k: torch.empty((Bt, L, Di), dtype=torch.bfloat16, device=dev)
             for k in ("y", "du", "dz", "da", "db")}
        o["xf"] = torch.empty((Bt, Di, N), dtype=torch.float32, device=dev)
        o["dB"] = torch.empty((Bt, L, N), dtype=torch.bfloat16, device=dev)
        o["dC"] = torch.empty((Bt, L, N), dtype=torch.bfloat16, device=dev)
        o["dD"] = torch.empty((Di,), dtype=torch.float32, device=dev)
        o["dw"] = torch.empty((Di, 4), dtype=torch.float32, device=dev)
        o["ck"] = torch.empty(nb.ckpt_bytes(dims) // 4, dtype=torch.float32, device=dev)
        return o

    outs = [alloc_outs() for _ in range(NSETS)]
    ws_f = nb.Workspace(nb.workspace_bytes(nb.OP_BLOCK_FWD, dims), dev)
    ws_b = nb.Workspace(nb.workspace_bytes(nb.OP_BLOCK_BWD, dims), dev)
    ws_s = nb.Workspace(nb.workspace_bytes(nb.OP_SCAN_FWD, dims), dev)

    def block_fwd(i):
        s, o = sets[i % NSETS], outs[i % NSETS]
        nb.check(L_.naju_block_fwd(ctypes.byref(dims), p(s["u"]), p(s["z"]), p(cw), None,
                                   p(s["a"]), p(s["b"]), p(s["B"]), p(s["C"]), p(D), None,
                                   p(o["y"]), p(o["xf"]), None, p(o["ck"]), ws_f.ptr,
                                   ws_f.nbytes, stream))

    def block_bwd(i):
        s, o = sets[i % NSETS], outs[i % NSETS]
        nb.check(L_.naju_block_bwd(ctypes.byref(dims), p(s["u"]), p(s["z"]), p(cw), None,
                                   p(s["a"]), p(s["b"]), p(s["B"]), p(s["C"]), p(D), None,
                                   p(o["ck"]), p(s["dy"]), None, p(o["du"]), p(o["dz"]),
                                   p(o["dw"]), None, p(o["da"]), p(o["db"]), p(o["dB"]),
                                   p(o["dC"]), p(o["dD"]), None, ws_b.ptr, ws_b.nbytes, stream))

    def scan_fwd(i):
        s, o = sets[i % NSETS], outs[i % NSETS]
        nb.check(L_.naju_scan_fwd(ctypes.byref(dims), p(s["u"]), p(s["a"]), p(s["b"]),
                                  p(s["B"]), p(s["C"]), p(D), None, p(o["y"]), p(o["xf"]), None,
                                  ws_s.ptr, ws_s.nbytes, stream))
    timer = Timer(torch)

    # ---------------------------------------------------------------- warmup
    for k in range(args.warmup):
        if args.only in ("all", "step"):
            block_fwd(k)
            block_bwd(k)
        if args.only in ("all", "scan_fwd"):
            scan_fwd(k)
    torch.cuda.synchronize()

    # ---------------------------------------------------------- timed steps
    t_step = float("nan")
    if args.only in ("all", "step"):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            block_fwd(k)
            block_bwd(k)
        torch.cuda.synchronize()
        t_step = (time.perf_counter() - t0) / args.steps
    # per-kernel timing (after the timed steps, same inputs)
    n_ev = args.steps if args.only != "all" else launches
    t_sf = timer.launches(scan_fwd, n_ev) if args.only in ("all", "scan_fwd") else None
    t_bf = timer.launches(block_fwd, n_ev) if args.only in ("all", "step") else None
    t_bb = timer.launches(block_bwd, n_ev) if args.only in ("all", "step") else None
    for ws in (ws_f, ws_b, ws_s):
        if ws.error_flags():
            raise RuntimeError("a cross-workgroup wait gave up: results invalid")

    tokens = Bt * L
    parts = {}
    for name, tt in (("scan_fwd", t_sf), ("block_fwd", t_bf), ("block_bwd", t_bb)):
        if tt is not None:
            parts[name] = hbm_part(tt, alg_bytes(name, Bt, L, Di, N, e), tokens)

    # decode step (one token per call, state and conv window carried in place) at the
    # workload's batch and width
    if args.only == "all":
        xs = torch.zeros((Bt, Di, N), dtype=torch.float32, device=dev)
        cst = torch.zeros((Bt, 3, Di), dtype=torch.bfloat16, device=dev)
        yst = torch.empty((Bt, Di), dtype=torch.bfloat16, device=dev)
        dec = [{k: sets[i][k][:, i].contiguous() for k in ("u", "z", "a", "b", "B", "C")}
               for i in range(NSETS)]

        def block_step(i):
            s = dec[i % NSETS]
            nb.check(L_.naju_block_step(ctypes.byref(dims), p(s["u"]), p(s["z"]), p(cw), p(cst),
                                        p(s["a"]), p(s["b"]), p(s["B"]), p(s["C"]), p(D), p(xs),
                                        p(yst), stream))
        for k in range(10):
            block_step(k)
        t_ds = timer.launches(block_step, max(launches, 100))
        parts["block_step"] = hbm_part(t_ds, alg_bytes("block_step", Bt, L, Di, N, e), Bt,
                                       what="naju_block_step, one token for each of the %d rows"
                                            % Bt)

    rf_scan = (roofline_hbm(parts["scan_fwd"], "naju::fwd_chunk_kernel<false> (naju_scan_fwd)",
                            measured_traffic("hbm_traffic_fwd_chunk_scan_bf16_b8_l2048_d1536_n16.md",
                                             FWD_SRC))
               if "scan_fwd" in parts else None)
    # dominant part of the timed step
    rf = rf_scan
    if "block_bwd" in parts and "block_fwd" in parts:
        if parts["block_bwd"]["ms_mean"] >= parts["block_fwd"]["ms_mean"]:
            rf = roofline_hbm(parts["block_bwd"],
                              "naju_block_bwd call: bwd_carry + bwd_carry_scan + bwd_mfma<true> "
                              "(gradients) + bwd_fix + finish + dd_reduce2",
                              measured_traffic("hbm_traffic_block_bwd_train_bf16_b8_l2048_d1536_n16.md",
                                               BWD_SRC))
        else:
            rf = roofline_hbm(parts["block_fwd"], "naju::fwd_chunk_kernel<true> (naju_block_fwd)",
                              measured_traffic("hbm_traffic_fwd_chunk_block_train_bf16_b8_l2048_d1536_n16.md",
                                               FWD_SRC))
    # the training step's input set stays on the host for the CPU leg; the device
    # buffers are freed before the other workloads
    del sets, base, outs, ws_f, ws_b, ws_s
    torch.cuda.empty_cache()

    # ----------------------------------------------- the other workloads
    rooflines = {}
    samples = {}
    if args.only == "all" and not args.no_configs:
        for name in SCAN_PARTS:
            def keep(dd, name=name):
                # the CPU leg's bounded sample: the first batch row, up to 1024 tokens
                n = min(inputs.WORKLOADS[name].L, 1024)
                samples[name] = {k: np.ascontiguousarray(dd[k][:1, :n]) if dd[k].ndim == 3
                                 else dd[k] for k in ("h", "a", "b", "B", "C", "D")}
            pp, rr = scan_workload_parts(name, torch, nb, inputs, args.warmup, launches, keep)
            parts.update(pp)
            rooflines[name] = rr

        def keep_mixer(dd):
            samples[MIXER] = {k: (np.ascontiguousarray(dd[k][:1, :256]) if k in ("xn", "res") else dd[k])
                              for k in dd}
        pp, rr, _ = mixer_parts(torch, nb, inputs, args.warmup, launches, keep_mixer)
        parts.update(pp)
        rooflines[MIXER] = rr

    cpu = None
    if not args.no_cpu:
        import oracle
        cores = len(os.sched_getaffinity(0))
        if os.environ.get("OMP_NUM_THREADS", "").isdigit():  # the oracle's OpenMP team
            cores = min(cores, int(os.environ["OMP_NUM_THREADS"]))
        # the whole step's workload (every batch row), a few seconds on the host cores
        t0 = time.perf_counter()
        oracle.block_fwd(d["u"], d["z"], d["conv_w"], d["a"], d["b"], d["B"], d["C"], d["D"])
        oracle.block_bwd(d["u"], d["z"], d["conv_w"], d["a"], d["b"], d["B"], d["C"], d["D"],
                         None, d["dy"])
        tc = time.perf_counter() - t0
        per = {}
        for name, s in samples.items():
            t0 = time.perf_counter()
            if name == MIXER:
                oracle.mixer_fwd(s["xn"], s["W_u"], s["W_z"], s["conv_w"], s["W_a"], s["a_bias"],
                                 s["W_b"], s["b_bias"], s["W_B"], s["W_C"], s["D"], s["W_out"],
                                 res=s["res"])
                what = "mixer forward, 1 x 256 tokens"
            else:
                oracle.scan_fwd(s["h"], s["a"], s["b"], s["B"], s["C"], s["D"])
                what = "scan forward, 1 x %d tokens" % s["h"].shape[1]
            dt = time.perf_counter() - t0
            ntok = s["xn"].shape[1] if name == MIXER else s["h"].shape[1]
            per[name] = {"sample": what, "s": round(dt, 4), "tokens_per_s": round(ntok / dt, 1),
                         "threads": cores}
        one = None
        try:
            r = subprocess.run([sys.executable, "-c", _ONE_THREAD, ROOT], capture_output=True,
                               text=True, timeout=120, env=dict(os.environ, OMP_NUM_THREADS="1"))
            if r.returncode == 0:
                o = json.loads(r.stdout.strip().splitlines()[-1])
                one = {"sample": "scan forward, the whole 1 x 256 x 192 fp32 workload",
                       "s_per_call": round(o["s_per_call"], 6),
                       "tokens_per_s": round(256 / o["s_per_call"], 1), "threads": 1}
        except (subprocess.TimeoutExpired, ValueError):
            one = None
        per["scan_f32_b1_l256_d192_n16 (1 thread)"] = one
        cpu = {"value": round(Bt * L / tc, 1), "unit": "tokens/s", "cores": cores,
               "kind": "oracle", "cpu_model": cpu_model(),
               "sample": "block fwd+bwd of the whole step workload (%d x %d tokens x %d channels, "
                         "d_state %d), fp64, %.2f s wall on %d threads" % (Bt, L, Di, N, tc, cores),
               "per_workload": per}

    # the practical HBM ceiling on this machine: a plain 1 GiB device copy (read + write)
    copy_ceiling = None
    if args.only == "all":
        dt = plain_copy(1 << 30, 3, 10)
        copy_ceiling = {"what": "plain 1 GiB device copy (HIP runtime copy kernel), read + write",
                        "GB_per_s": round(2 * (1 << 30) / dt / 1e9, 1),
                        "frac_of_peak": round(2 * (1 << 30) / dt / 1e9 / HBM_PEAK_GBS, 4)}

    out = {
        "metric": METRIC,
        "value": round(tokens / t_step, 1) if t_step == t_step else None,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 4) if t_step == t_step else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "batch": Bt, "seq_len": L, "d_inner": Di,
                   "d_state": N, "io": "bf16", "state": "f32",
                   "step": "block fwd (with checkpoints) + block bwd"},
        "roofline": rf,
        "roofline_scan_fwd": rf_scan,
        "rooflines_other_workloads": rooflines or None,
        "cpu_baseline": cpu,
        "hbm_copy_ceiling": copy_ceiling,
        "parts": parts,
    }
    print(json.dumps(out), flush=True)


def bench_mixer_workload(args, torch, nb, inputs):
    """The mixer workload's own line: a forward + backward step of the layer."""
    parts, rf, t_step = mixer_parts(torch, nb, inputs, args.warmup, max(args.steps, MIN_LAUNCHES))
    c = inputs.MIXER_WORKLOADS[MIXER]
    Bt, L = c["Bt"], c["L"]
    out = {
        "metric": "mixer layer tokens/sec, forward + backward step (forward alone in parts)",
        "value": round(Bt * L / t_step, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": max(args.steps, MIN_LAUNCHES),
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": MIXER, "batch": Bt, "seq_len": L, "d_model": c["dm"],
                   "d_inner": c["Di"], "d_state": c["N"], "io": "bf16",
                   "step": "naju_mixer_fwd + naju_mixer_bwd reusing the forward's workspace"},
        "roofline": rf,
        "cpu_baseline": None,
        "parts": parts,
    }
    print(json.dumps(out), flush=True)


def bench_scan_workload(args, torch, nb, inputs):
    """A named scan workload's own line: naju_scan_fwd alone, inputs resident in HBM."""
    w = inputs.WORKLOADS[args.workload]
    if w.block or w.backward:
        raise SystemExit("--workload takes a scan workload or the mixer workload")
    launches = max(args.steps, MIN_LAUNCHES)
    torch.cuda.synchronize()
    parts, rf = scan_workload_parts(w.name, torch, nb, inputs, args.warmup, launches)
    main_part = parts["scan_fwd[%s]" % w.name]
    out = {
        "metric": METRIC,
        "value": main_part["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": launches,
        "warmup": args.warmup,
        "ms_per_step": main_part["ms_median"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.Bt, "seq_len": w.L, "d_inner": w.Di,
                   "d_state": w.N, "io": w.io, "state": "f32", "step": "scan fwd"},
        "roofline": rf,
        "cpu_baseline": None,
        "parts": parts,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
