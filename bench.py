#!/usr/bin/env python3
"""Throughput of the gated temporal scan (forward + backward) on one MI355X.

One step = one forward pass and one backward pass (both phases) over one
batch of the headline workload B=8192, K=8, SH2=256, D=16 (fp32), with all
inputs already resident in HBM.  Steps rotate over several distinct input
sets (together larger than the 256 MB Infinity Cache) so the timed traffic
is real HBM traffic.  Prints one JSON line.

Fields beyond the headline value:
  hbm_frac          algorithmic bytes per step / step time / 8 TB/s
  kernels_us        average duration of each kernel, HIP events on the
                    launch stream, measured in a second timed loop
  roofline          the dominant kernel against its bound
  cpu_baseline      the fp64 CPU oracle timed on a bounded sample of the
                    same workload on this host's cores
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
FP32_PEAK_TFLOPS = 157.3     # MI355X dense fp32 (matrix and vector)
METRIC = "fwd+bwd samples/sec at B=8192,K=8,SH2=256,D=16; % of peak HBM GB/s"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="prod_fp32")
    ap.add_argument("--sets", type=int, default=5, help="distinct input sets rotated per step")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def cpu_baseline(w, target_s):
    import oracle
    from gated_linear_recurrence_history_amd import synth

    def run(n):
        x = synth.make_inputs(w, B=n)
        t0 = time.perf_counter()
        oracle.forward(x["h_history"], x["h_s2"], x["W_A"], x["W_B"], x["W_C"], w.K, w.a_shift)
        oracle.backward(x["h_history"], x["h_s2"], x["W_A"], x["W_B"], x["W_C"], w.K,
                        x["d_context"], w.a_shift)
        return time.perf_counter() - t0

    n = min(w.B, 256)
    t = run(n)
    if t < target_s and n < w.B:
        n = int(min(w.B, max(n, n * target_s / max(t, 1e-6))))
        t = run(n)
    return {"value": n / t, "unit": "samples/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"first {n} of {w.B} samples of {w.name}, forward+backward in fp64, "
                      f"{t:.2f} s"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    from gated_linear_recurrence_history_amd import binding, synth, workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    w = wl.BY_NAME[args.workload]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    sets = []
    for i in range(args.sets):
        x = synth.make_inputs(w, seed=w.seed + 1000 * i)
        sets.append({k: to_dev(v) for k, v in x.items()})
    ctx = torch.empty((w.B, w.D), dtype=torch.float32, device=dev)
    dW = tuple(torch.empty((w.SH2, w.D), dtype=torch.float32, device=dev) for _ in range(3))
    ws = torch.empty(binding.backward_workspace_bytes(w.B, w.K, w.SH2, w.D, w.in_dtype == "bf16"),
                     dtype=torch.uint8, device=dev)
    fwd, bwd, bwd1 = [], [], []
    for t in sets:
        a = (t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"], w.K)
        fwd.append(binding.prepare_forward(*a, ctx, w.a_shift, stream))
        bwd.append(binding.prepare_backward(*a, t["d_context"], dW, ws, w.a_shift, stream))
        bwd1.append(binding.prepare_backward_partials(*a, t["d_context"], ws, w.a_shift, stream))
    red = binding.prepare_backward_reduce(ws, w.B, w.K, w.SH2, w.D, dW, w.in_dtype == "bf16",
                                          stream)
    torch.cuda.synchronize()
    print(f"bench: {w.name} B={w.B} K={w.K} SH2={w.SH2} D={w.D} {w.in_dtype}, "
          f"{args.sets} input sets, warmup {args.warmup}, steps {args.steps}",
          file=sys.stderr, flush=True)

    n = len(sets)
    for i in range(args.warmup):
        fwd[i % n]()
        bwd[i % n]()
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` steps between two events
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        fwd[i % n]()
        bwd[i % n]()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = e0.elapsed_time(e1)
    ms_step = ms_total / args.steps

    # ---- per-kernel durations (events around each launch on the same stream)
    reps = max(20, min(args.steps, 200))
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
    for i in range(reps):
        e = ev[i]
        e[0].record(stream)
        fwd[i % n]()
        e[1].record(stream)
        bwd1[i % n]()
        e[2].record(stream)
        red()
        e[3].record(stream)
    torch.cuda.synchronize()
    k_fwd = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e3
    k_bwd = float(np.mean([e[1].elapsed_time(e[2]) for e in ev])) * 1e3
    k_red = float(np.mean([e[2].elapsed_time(e[3]) for e in ev])) * 1e3

    step_bytes = w.fwd_bytes() + w.bwd_bytes()
    value = w.B / (ms_step * 1e-3)
    hbm_frac = step_bytes / (ms_step * 1e-3) / (HBM_PEAK_GBS * 1e9)

    # dominant kernel against the roof its own arithmetic intensity selects
    if k_bwd >= k_fwd:
        kname, kus, kbytes, kflops = "gscan_bwd_kernel", k_bwd, w.bwd_bytes(), w.bwd_flops()
    else:
        kname, kus, kbytes, kflops = "gscan_fwd_kernel", k_fwd, w.fwd_bytes(), w.fwd_flops()
    t_hbm = kbytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = kflops / (FP32_PEAK_TFLOPS * 1e12)
    if t_hbm >= t_mfma:
        ach = kbytes / (kus * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None}
    else:
        ach = kflops / (kus * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": FP32_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / FP32_PEAK_TFLOPS, 4), "traffic": None}
    roof.update({"kernel": kname, "avg_us": round(kus, 3),
                 "algorithmic_bytes": kbytes, "algorithmic_flops": kflops,
                 "hbm_frac_of_kernel": round(kbytes / (kus * 1e-6) / (HBM_PEAK_GBS * 1e9), 4)})

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "samples/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.in_dtype == "f32" else "bf16-in/f32",
        "data": "synthetic",
        "config": dict(w.describe(), input_sets=args.sets),
        "hbm_frac": round(hbm_frac, 4),
        "hbm_GBs_fwd_bwd": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "wall_ms_per_step": round(wall / args.steps * 1e3, 5),
        "kernels_us": {"gscan_fwd_kernel": round(k_fwd, 3), "gscan_bwd_kernel": round(k_bwd, 3),
                       "gscan_reduce_kernel": round(k_red, 3)},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
