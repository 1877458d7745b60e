"""Benchmark of the Naju scan hot path on one MI355X.

A step is one pass of the whole hot path over one batch of the training
workload (batch 8, seqlen 2048, d_inner 1536, d_state 16, bf16 activations,
fp32 state): the fused block forward (conv+SiLU front end, gates, scan,
readout, SiLU(z) modulation, checkpoints) followed by the block backward
(reverse-time adjoint scan, every gradient).  Inputs are synthetic, drawn by
the seeded generator, and resident in HBM before timing starts; three input
sets rotate so the 256 MB Infinity Cache cannot hold a step's working set.

Also timed in the same run: the scan forward alone (the kernel with the
70%-of-HBM-peak target), the block forward alone, and the CPU oracle on a
bounded sample of the same workload (the cpu_baseline leg).

`--workload NAME` instead times naju_scan_fwd alone on another named workload
of the hot path (for instance the 4 x 8192 x 4096, d_state 64 scan), with its
roofline, or, for a mixer workload (mixer_bf16_b8_l2048_dm768_d1536_n16), the
whole mixer layer forward (naju_mixer_fwd: projections on the matrix cores
around the block scan); the default run is the training step above.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "scan tokens/sec + achieved HBM GB/s (% peak), fwd and fwd+bwd, L=2048"
HBM_PEAK_GBS = 8000.0
WORKLOAD = "train_bf16_b8_l2048_d1536_n16"
NSETS = 3


def alg_bytes(kind, Bt, L, Di, N, e, K=4):
    """Algorithmic HBM bytes of one call (what the method must move)."""
    tok, st = Bt * L * Di, Bt * Di * N
    if kind == "scan_fwd":     # read h, a, b; write y; B, C; x_final; D
        return tok * 4 * e + Bt * L * N * 2 * e + st * 4 + Di * 4
    if kind == "block_fwd":    # read u, z, a, b; write y; B, C; x_final; D, conv_w
        return tok * 5 * e + Bt * L * N * 2 * e + st * 4 + Di * 4 + Di * K * 4
    if kind == "block_bwd":    # read u, z, a, b, dy; write du, dz, da, db; B, C, dB, dC; D, dD, w, dw
        return tok * 9 * e + Bt * L * N * 4 * e + Di * 4 * 2 + Di * K * 4 * 2
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the cpu_baseline leg")
    ap.add_argument("--only", choices=["all", "scan_fwd", "step", "copy"], default="all",
                    help="restrict the timed work (for profiling runs); 'copy' runs a plain "
                         "1 GiB device copy, the reference for HBM byte counters")
    ap.add_argument("--workload", default=WORKLOAD,
                    help="another named scan workload (naju_scan_fwd alone) or a mixer "
                         "workload (naju_mixer_fwd)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the Naju scan path has no multi-GPU "
              "implementation here (see DESIGN.md for how it would shard).", file=sys.stderr)
        sys.exit(2)

    import torch
    from selective_state_space_naju_amd import binding as nb
    from selective_state_space_naju_amd import inputs

    dev = torch.device("cuda:0")
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
    if args.workload in inputs.MIXER_WORKLOADS:
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
        s, o = sets[i], outs[i]
        nb.check(L_.naju_block_fwd(ctypes.byref(dims), p(s["u"]), p(s["z"]), p(cw), None,
                                   p(s["a"]), p(s["b"]), p(s["B"]), p(s["C"]), p(D), None,
                                   p(o["y"]), p(o["xf"]), None, p(o["ck"]), ws_f.ptr,
                                   ws_f.nbytes, stream))

    def block_bwd(i):
        s, o = sets[i], outs[i]
        nb.check(L_.naju_block_bwd(ctypes.byref(dims), p(s["u"]), p(s["z"]), p(cw), None,
                                   p(s["a"]), p(s["b"]), p(s["B"]), p(s["C"]), p(D), None,
                                   p(o["ck"]), p(s["dy"]), None, p(o["du"]), p(o["dz"]),
                                   p(o["dw"]), None, p(o["da"]), p(o["db"]), p(o["dB"]),
                                   p(o["dC"]), p(o["dD"]), None, ws_b.ptr, ws_b.nbytes, stream))

    def scan_fwd(i):
        s, o = sets[i], outs[i]
        nb.check(L_.naju_scan_fwd(ctypes.byref(dims), p(s["u"]), p(s["a"]), p(s["b"]),
                                  p(s["B"]), p(s["C"]), p(D), None, p(o["y"]), p(o["xf"]), None,
                                  ws_s.ptr, ws_s.nbytes, stream))

    def timed_launches(fn, count):
        """Per-launch GPU durations (ms) from events on the launch stream."""
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(count)]
        torch.cuda.synchronize()
        for k in range(count):
            ev[k][0].record()
            fn(k % NSETS)
            ev[k][1].record()
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in ev])

    # ---------------------------------------------------------------- warmup
    for k in range(args.warmup):
        if args.only in ("all", "step"):
            block_fwd(k % NSETS)
            block_bwd(k % NSETS)
        if args.only in ("all", "scan_fwd"):
            scan_fwd(k % NSETS)
    torch.cuda.synchronize()

    # ---------------------------------------------------------- timed steps
    t_step = float("nan")
    if args.only in ("all", "step"):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            block_fwd(k % NSETS)
            block_bwd(k % NSETS)
        torch.cuda.synchronize()
        t_step = (time.perf_counter() - t0) / args.steps
    # per-kernel timing (after the timed steps, same inputs)
    n_ev = args.steps if args.only != "all" else max(args.steps, 10)
    t_sf = timed_launches(scan_fwd, n_ev) if args.only in ("all", "scan_fwd") else None
    t_bf = timed_launches(block_fwd, n_ev) if args.only in ("all", "step") else None
    t_bb = timed_launches(block_bwd, n_ev) if args.only in ("all", "step") else None
    for ws in (ws_f, ws_b, ws_s):
        if ws.error_flags():
            raise RuntimeError("a cross-workgroup wait gave up: results invalid")

    # decode step (one token per call, state and conv window carried in place) at the
    # workload's batch and width: per-call latency and bytes moved
    t_ds = None
    if args.only == "all":
        xs = torch.zeros((Bt, Di, N), dtype=torch.float32, device=dev)
        cst = torch.zeros((Bt, 3, Di), dtype=torch.bfloat16, device=dev)
        yst = torch.empty((Bt, Di), dtype=torch.bfloat16, device=dev)
        dec = [{k: sets[i][k][:, i].contiguous() for k in ("u", "z", "a", "b", "B", "C")}
               for i in range(NSETS)]

        def block_step(i):
            s = dec[i]
            nb.check(L_.naju_block_step(ctypes.byref(dims), p(s["u"]), p(s["z"]), p(cw), p(cst),
                                        p(s["a"]), p(s["b"]), p(s["B"]), p(s["C"]), p(D), p(xs),
                                        p(yst), stream))
        for k in range(10):
            block_step(k % NSETS)
        t_ds = timed_launches(block_step, 100)

    tokens = Bt * L
    parts = {}
    for name, tt, kind in (("scan_fwd", t_sf, "scan_fwd"), ("block_fwd", t_bf, "block_fwd"),
                           ("block_bwd", t_bb, "block_bwd")):
        if tt is None:
            continue
        ms = float(np.median(tt))
        by = alg_bytes(kind, Bt, L, Di, N, e)
        parts[name] = {"ms_median": round(ms, 4), "ms_mean": round(float(tt.mean()), 4),
                       "tokens_per_s": round(tokens / (ms * 1e-3), 1),
                       "alg_bytes": int(by), "GB_per_s": round(by / (ms * 1e-3) / 1e9, 1),
                       "pct_hbm_peak": round(100 * by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)}

    if t_ds is not None:
        ms = float(np.median(t_ds))
        # state read + write, u z a b read, y write, conv window read + write, B C, D, conv_w
        by = Bt * Di * N * 8 + Bt * Di * 5 * e + Bt * 3 * Di * e * 2 + Bt * N * 2 * e + Di * 4 * 5
        parts["block_step"] = {"what": "naju_block_step, one token for each of the %d rows" % Bt,
                               "us_median": round(ms * 1e3, 2),
                               "us_mean": round(float(t_ds.mean()) * 1e3, 2),
                               "tokens_per_s": round(Bt / (ms * 1e-3), 1), "alg_bytes": int(by),
                               "GB_per_s": round(by / (ms * 1e-3) / 1e9, 1)}

    def roofline(part, kernel, traffic_md=None, sources=()):
        by = parts[part]["alg_bytes"]
        ms = parts[part]["ms_mean"]
        ach = by / (ms * 1e-3) / 1e9
        return {"kernel": kernel, "bound": "hbm", "achieved": round(ach, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(traffic_md, sources),
                "ms_per_launch": round(ms, 4), "alg_bytes_per_launch": int(by)}

    fwd_src = ("selective_state_space_naju_amd/csrc/naju_fwd_mfma.hip",
               "selective_state_space_naju_amd/csrc/naju_mfma.h",
               "selective_state_space_naju_amd/csrc/naju_device.h",
               "selective_state_space_naju_amd/csrc/naju_launch.h")
    rf_scan = (roofline("scan_fwd", "naju::fwd_mfma_kernel<false> (naju_scan_fwd)",
                        "hbm_traffic_fwd_mfma_scan_bf16_b8_l2048_d1536_n16.md", fwd_src)
               if "scan_fwd" in parts else None)
    # dominant part of the timed step
    rf = rf_scan
    if "block_bwd" in parts and "block_fwd" in parts:
        if parts["block_bwd"]["ms_mean"] >= parts["block_fwd"]["ms_mean"]:
            bwd_src = ("selective_state_space_naju_amd/csrc/naju_bwd_mfma.hip",
                       "selective_state_space_naju_amd/csrc/naju_bwd.hip",
                       "selective_state_space_naju_amd/csrc/naju_device.h",
                       "selective_state_space_naju_amd/csrc/naju_launch.h")
            rf = roofline("block_bwd", "naju_block_bwd call: bwd_carry + bwd_carry_scan + "
                          "bwd_mfma<true> (gradients) + bwd_fix + 4 reduction kernels",
                          "hbm_traffic_block_bwd_train_bf16_b8_l2048_d1536_n16.md", bwd_src)
        else:
            rf = roofline("block_fwd", "naju::fwd_mfma_kernel<true> (naju_block_fwd)")

    cpu = None
    if not args.no_cpu:
        import oracle
        # the whole step's workload (every batch row), a few seconds on the host cores
        cores = len(os.sched_getaffinity(0))
        if os.environ.get("OMP_NUM_THREADS", "").isdigit():  # the oracle's OpenMP team
            cores = min(cores, int(os.environ["OMP_NUM_THREADS"]))
        t0 = time.perf_counter()
        oracle.block_fwd(d["u"], d["z"], d["conv_w"], d["a"], d["b"], d["B"], d["C"], d["D"])
        oracle.block_bwd(d["u"], d["z"], d["conv_w"], d["a"], d["b"], d["B"], d["C"], d["D"],
                         None, d["dy"])
        tc = time.perf_counter() - t0
        cpu = {"value": round(Bt * L / tc, 1), "unit": "tokens/s", "cores": cores,
               "kind": "oracle",
               "sample": "block fwd+bwd of the whole workload (%d x %d tokens x %d channels, "
                         "d_state %d), fp64, %.2f s wall on %d threads" % (Bt, L, Di, N, tc, cores)}

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
        "cpu_baseline": cpu,
        "hbm_copy_ceiling": copy_ceiling,
        "parts": parts,
    }
    print(json.dumps(out), flush=True)


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak


def bench_mixer_workload(args, torch, nb, inputs):
    """naju_mixer_fwd on a named mixer workload, inputs and weights resident in HBM;
    also the block forward alone on inputs of the same shape (the scan inside)."""
    c = inputs.MIXER_WORKLOADS[args.workload]
    Bt, L, dm, Di, N = c["Bt"], c["L"], c["dm"], c["Di"], c["N"]
    dev = torch.device("cuda:0")
    d = inputs.draw_mixer(Bt, L, dm, Di, N, seed=c["seed"])
    f32 = ("conv_w", "D", "a_bias", "b_bias")
    t = {k: torch.from_numpy(v).to(torch.float32 if k in f32 else torch.bfloat16).to(dev)
         for k, v in d.items()}
    del d
    sets = [t["xn"], t["xn"].roll(1, 0).contiguous()]
    res = [t["res"], t["res"].roll(1, 0).contiguous()]

    dims = nb.make_dims(Bt, L, Di, N, nb.BF16)
    fws = nb.Workspace(int(nb.lib().naju_mixer_workspace_bytes(ctypes.byref(dims), dm)), dev)

    def call(i):
        nb.mixer_fwd(sets[i % 2], t["W_u"], t["W_z"], t["conv_w"], t["W_a"], t["a_bias"],
                     t["W_b"], t["b_bias"], t["W_B"], t["W_C"], t["D"], t["W_out"],
                     res=res[i % 2], ws=fws)

    def timed(fn, steps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            ev[k][0].record()
            fn(k)
            ev[k][1].record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        return wall, np.array([a.elapsed_time(b) for a, b in ev])

    for k in range(args.warmup):
        call(k)
    t_all, tt = timed(call, args.steps)
    # the layer's backward (it recomputes the forward intermediates), and a step
    g_out = [torch.randn_like(sets[0], dtype=torch.float32).to(torch.bfloat16) for _ in range(2)]

    def call_bwd(i):
        nb.mixer_bwd(sets[i % 2], t["W_u"], t["W_z"], t["conv_w"], t["W_a"], t["a_bias"],
                     t["W_b"], t["b_bias"], t["W_B"], t["W_C"], t["D"], t["W_out"], g_out[i % 2])

    def call_step(i):  # a training step: the backward reuses the forward's workspace
        call(i)
        nb.mixer_bwd(sets[i % 2], t["W_u"], t["W_z"], t["conv_w"], t["W_a"], t["a_bias"],
                     t["W_b"], t["b_bias"], t["W_B"], t["W_C"], t["D"], t["W_out"], g_out[i % 2],
                     fwd_ws=fws)
    for k in range(args.warmup):
        call_bwd(k)
    _, tbw = timed(call_bwd, args.steps)
    t_step, tst = timed(call_step, args.steps)
    # the block scan of the same shape alone (synthetic u, z, a, b, B, C)
    w = inputs.Workload("mixer_scan_part", Bt, L, Di, N, seed=c["seed"] + 1, block=True)
    db = inputs.draw_workload(w)
    bt = {k: torch.from_numpy(db[k]).to(torch.bfloat16).to(dev)
          for k in ("u", "z", "a", "b", "B", "C")}
    bD, bw = torch.from_numpy(db["D"]).to(dev), torch.from_numpy(db["conv_w"]).to(dev)
    del db
    blk = lambda i: nb.block_fwd(bt["u"], bt["z"], bw, bt["a"], bt["b"], bt["B"], bt["C"], bD)  # noqa: E731
    for k in range(args.warmup):
        blk(k)
    _, tb = timed(blk, args.steps)
    ms, ms_b = float(tt.mean()), float(tb.mean())
    flops = 2.0 * Bt * L * (2 * dm * Di + 2 * Di * Di + 2 * Di * N + Di * dm)
    ach = flops / (ms * 1e-3) / 1e12
    ach_g = flops / ((ms - ms_b) * 1e-3) / 1e12
    out = {
        "metric": "mixer layer tokens/sec, forward + backward step (forward alone in parts)",
        "value": round(Bt * L / t_step, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": Bt, "seq_len": L, "d_model": dm,
                   "d_inner": Di, "d_state": N, "io": "bf16",
                   "step": "naju_mixer_fwd + naju_mixer_bwd reusing the forward's workspace "
                           "(parts.mixer_bwd: the backward alone, recomputing the forward)"},
        "roofline": {"kernel": "the call's hipBLASLt projections (bf16, fp32 accumulation); "
                               "time = mixer call minus the block forward alone",
                     "bound": "mfma", "achieved": round(ach_g, 1),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach_g / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "ms_per_launch": round(ms - ms_b, 4), "alg_flops_per_launch": int(flops)},
        "cpu_baseline": None,
        "parts": {"mixer_fwd": {"ms_median": round(float(np.median(tt)), 4),
                                "ms_mean": round(ms, 4),
                                "tokens_per_s": round(Bt * L / (ms * 1e-3), 1),
                                "gemm_flops": int(flops),
                                "TFLOP_per_s_over_call": round(ach, 1)},
                  "mixer_bwd": {"ms_median": round(float(np.median(tbw)), 4),
                                "ms_mean": round(float(tbw.mean()), 4),
                                "gemm_flops": int(3 * flops)},
                  "mixer_step": {"ms_median": round(float(np.median(tst)), 4),
                                 "ms_mean": round(float(tst.mean()), 4)},
                  "block_fwd_same_shape": {"ms_median": round(float(np.median(tb)), 4),
                                           "ms_mean": round(ms_b, 4)}},
    }
    print(json.dumps(out), flush=True)


def bench_scan_workload(args, torch, nb, inputs):
    """naju_scan_fwd alone on a named scan workload, inputs resident in HBM."""
    w = inputs.WORKLOADS[args.workload]
    if w.block or w.backward:
        raise SystemExit("--workload takes a scan workload")
    Bt, L, Di, N = w.Bt, w.L, w.Di, w.N
    e = 2 if w.io == "bf16" else 4
    dev = torch.device("cuda:0")
    io_t = torch.bfloat16 if w.io == "bf16" else torch.float32
    d = inputs.draw_workload(w)
    base = {k: torch.from_numpy(d[k]).to(io_t).to(dev) for k in ("h", "a", "b", "B", "C")}
    D = torch.from_numpy(d["D"]).to(dev)
    del d
    # two input sets (a third would not fit the point: each set is well past the
    # 256 MB Infinity Cache at this size)
    sets = [base, {k: v.clone() for k, v in base.items()}]
    dims = nb.make_dims(Bt, L, Di, N, nb.BF16 if w.io == "bf16" else nb.F32)
    ws = nb.Workspace(nb.workspace_bytes(nb.OP_SCAN_FWD, dims), dev)
    y = torch.empty((Bt, L, Di), dtype=io_t, device=dev)
    xf = torch.empty((Bt, Di, N), dtype=torch.float32, device=dev)
    L_, stream = nb.lib(), nb.stream_handle(dev)
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731

    def call(i):
        s = sets[i % 2]
        nb.check(L_.naju_scan_fwd(ctypes.byref(dims), p(s["h"]), p(s["a"]), p(s["b"]),
                                  p(s["B"]), p(s["C"]), p(D), None, p(y), p(xf), None, ws.ptr,
                                  ws.nbytes, stream))
    for k in range(args.warmup):
        call(k)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        ev[k][0].record()
        call(k)
        ev[k][1].record()
    torch.cuda.synchronize()
    t_all = (time.perf_counter() - t0) / args.steps
    if ws.error_flags():
        raise RuntimeError("a cross-workgroup wait gave up: results invalid")
    tt = np.array([a.elapsed_time(b) for a, b in ev])
    ms = float(tt.mean())
    by = alg_bytes("scan_fwd", Bt, L, Di, N, e)
    ach = by / (ms * 1e-3) / 1e9
    traffic = None
    if N == 64 and e == 2:
        kernel = "naju::fwd_mfma64_kernel<false> (naju_scan_fwd)"
        traffic = measured_traffic(
            "hbm_traffic_fwd_mfma64_%s.md" % w.name,
            ("selective_state_space_naju_amd/csrc/naju_fwd_mfma64.hip",
             "selective_state_space_naju_amd/csrc/naju_mfma.h",
             "selective_state_space_naju_amd/csrc/naju_device.h",
             "selective_state_space_naju_amd/csrc/naju_launch.h"))
    else:
        kernel = "naju_scan_fwd (d_state %d)" % N
    out = {
        "metric": METRIC,
        "value": round(Bt * L / (t_all), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_all * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": Bt, "seq_len": L, "d_inner": Di, "d_state": N,
                   "io": w.io, "state": "f32", "step": "scan fwd"},
        "roofline": {"kernel": kernel, "bound": "hbm", "achieved": round(ach, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "ms_per_launch": round(ms, 4),
                     "alg_bytes_per_launch": int(by)},
        "cpu_baseline": None,
        "parts": {"scan_fwd": {"ms_median": round(float(np.median(tt)), 4), "ms_mean": round(ms, 4),
                               "tokens_per_s": round(Bt * L / (ms * 1e-3), 1), "alg_bytes": int(by),
                               "GB_per_s": round(ach, 1),
                               "pct_hbm_peak": round(100 * ach / HBM_PEAK_GBS, 2)}},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
