#!/usr/bin/env python3
"""Throughput of the gated temporal scan (forward + backward) on one MI355X.

One step = one forward pass and one backward pass (both phases) over one
batch of the headline workload B=8192, K=8, SH2=256, D=16 (fp32), with all
inputs already resident in HBM.  Steps rotate over several distinct input
sets (together larger than the 256 MB Infinity Cache), so no step finds the
data of an earlier step in that cache.  Within a step the backward reads
the set its forward has just streamed, and part of those reads may be
served by the Infinity Cache (the natural forward-then-backward pattern on
one batch); `no_reuse` times the same work with the backward on a set the
forward did not touch.  Prints one JSON line.

Fields beyond the headline value:
  hbm_frac          algorithmic bytes per step / step time / 8 TB/s
  read_ceiling_GBs  a measured read ceiling: a read-only stream of 1 GiB
                    (two 1 GiB halves read alternately, so no read is served
                    by the Infinity Cache), bytes over time, median of 8
  frac_of_read_ceiling  algorithmic bytes per step / step time / that ceiling
  no_reuse          the step with the backward on input set i+2 while the
                    forward runs on set i (the backward's set was last read
                    six passes, 432 MiB, earlier): time per step, samples/s,
                    fraction of 8 TB/s and of the read ceiling
  graph_ms_per_step the same steps captured once as a HIP graph (one step
                    per input set) and replayed, time per step
  step_us           p10 / p50 / p90 of single-step times (an event pair
                    around each step, measured after the timed region)
  copy_GBs          a streaming figure for context: bytes read plus written
                    by a 512 MiB device-to-device copy over its time (median
                    of 5)
  kernels_us        average duration of each kernel: HIP events on the
                    launch stream around a run of back-to-back launches of
                    that kernel alone (the median of three such runs)
  roofline          the dominant (longest) kernel against the roof that
                    bounds it (the higher of its HBM floor and its MFMA
                    floor): algorithmic bytes per launch over its average
                    duration against 8 TB/s, or the bf16 products it issues
                    (three per fp32 product) against 2.5 PFLOP/s; `traffic`
                    is the HBM bytes per launch that
                    rocprofv3 counters measured for the same kernel source
                    (profiles/traffic_<kernel>_<workload>.txt), else null;
                    where the backward's phase 1 is the split pair (scan
                    pass, then contraction) the two are one phase: their
                    summed time and traffic
  cpu_baseline      the fp64 CPU oracle timed on a bounded sample of the
                    same workload on this host's cores
  configs           every named workload (tiny, headline, long K, bf16 big
                    batch, wide): forward and backward HIP-event time per call
                    (median of three batches) on resident synthetic inputs,
                    samples/s, the fraction
                    of 8 TB/s their algorithmic bytes reach, and the step's
                    floor (per pass the higher of its HBM and MFMA times) as
                    a fraction of its time
  out_of_envelope   the headline shape at SH2 = 240 and 1024, outside the
                    fused kernels (the materialised-projection path): the
                    same figures against the same floor
  bias_grad_reduce  the batch-parallel bias-gradient reduction on the spec's
                    IQN shape [524288 x 3] (fp32, synthetic N(0, 9)): HIP-event
                    time per call, bytes read against 8 TB/s, and the
                    oracle's rate
  enrich            the forward that adds the context into a [B, SH2]
                    h_enriched (gscan_forward_enrich): time per call and
                    over the plain forward
  cifg              the CIFG matrix-memory update in independent mode
                    (gscan_batched_cifg_update) on the page's batch 32,
                    d_model 512 and on batch 256: time per call, bytes (C read
                    and written once) against 8 TB/s, the oracle's time
  input_grads       the backward that also returns the input gradients
                    (gscan_backward_full_ex): HIP-event time per call on the
                    same rotated inputs, its algorithmic bytes (the backward's
                    plus d_h_history and d_h_s2 written) against 8 TB/s, the
                    time over the plain backward, and the oracle's rate for
                    the input gradients on a small sample

The matrix products run on bf16 MFMA with fp32 operands split into a high
and a low bf16 part (three products per fp32 product, fp32 accumulation;
`dtype` says so), so the MFMA time of a pass is at least 3 x its fp32 flops
/ 2.5 PFLOP/s.  At the headline shape that is well under its HBM time; the
long-K and wide workloads are bounded by the matrix cores instead (the
roofline's `bound` says which floor is higher).
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
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
SPLIT_PRODUCTS = 3           # bf16 products per fp32 product
METRIC = "fwd+bwd samples/sec at B=8192,K=8,SH2=256,D=16; % of peak HBM GB/s"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # 500 steps (about 20 ms of GPU work): with 20 the first part of the timed
    # region still ran while the GPU raised its clocks (43.4 against 41.1 us
    # per step on the headline workload; 500 and 2000 give the same)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--workload", default="prod_fp32")
    ap.add_argument("--sets", type=int, default=5, help="distinct input sets rotated per step")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-input-grads", action="store_true",
                    help="skip the timing of the backward with input gradients")
    ap.add_argument("--no-bias-grad", action="store_true",
                    help="skip the timing of the bias-gradient reduction")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload forward/backward timings")
    ap.add_argument("--configs", default="",
                    help="comma-separated workload names to time in configs / out_of_envelope "
                         "(default: all of both)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="finish with 4 untimed device copies of this many MiB (the reference "
                         "for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    return ap.parse_args()


def cpu_baseline(w, target_s):
    """The oracle, as it is, on a bounded sample: the first n samples of the
    workload (all of them if one pass is short), forward + backward, repeated
    until about target_s seconds have passed."""
    import oracle
    from gated_linear_recurrence_history_amd import synth

    n = min(w.B, 1024)
    x = synth.make_inputs(w, B=n)

    def once():
        oracle.forward(x["h_history"], x["h_s2"], x["W_A"], x["W_B"], x["W_C"], w.K, w.a_shift)
        oracle.backward(x["h_history"], x["h_s2"], x["W_A"], x["W_B"], x["W_C"], w.K,
                        x["d_context"], w.a_shift)

    t0 = time.perf_counter()
    once()
    t1 = time.perf_counter() - t0
    if t1 * 4 < target_s and n < w.B:  # a larger sample when one pass is short
        n = int(min(w.B, n * max(1.0, target_s / 4 / max(t1, 1e-6))))
        x = synth.make_inputs(w, B=n)
        t0 = time.perf_counter()
        once()
        t1 = time.perf_counter() - t0
    reps = max(1, int(target_s / max(t1, 1e-6)))
    t0 = time.perf_counter()
    for _ in range(reps):
        once()
    t = time.perf_counter() - t0
    return {"value": n * reps / t, "unit": "samples/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"first {n} of {w.B} samples of {w.name}, fp64 forward+backward, "
                      f"{reps} passes in {t:.1f} s"}


def input_grads(args, w, sets, stream, bwd_us, reps):
    """gscan_backward_full_ex per call (HIP events, rotated inputs) and the
    oracle's input-gradient rate on a small sample."""
    import torch

    import oracle
    from gated_linear_recurrence_history_amd import binding, synth

    dev = sets[0]["h_history"].device
    bf = w.in_dtype == "bf16"
    out = tuple(torch.empty((w.SH2, w.D), device=dev) for _ in range(3)) + (
        torch.empty((w.rows, w.SH2), device=dev), torch.empty((w.B, w.SH2), device=dev))
    ws = torch.empty(binding.backward_full_workspace_bytes(w.B, w.K, w.SH2, w.D, bf),
                     dtype=torch.uint8, device=dev)
    fns = [binding.prepare_backward_full(t["h_history"], t["h_s2"], t["W_A"], t["W_B"],
                                         t["W_C"], w.K, t["d_context"], out, ws, w.a_shift,
                                         stream) for t in sets]
    n = len(fns)
    for i in range(max(args.warmup, n)):
        fns[i % n]()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for i in range(reps):
        fns[i % n]()
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / reps
    nbytes = w.bwd_bytes() + w.dinput_out_bytes()
    gbs = nbytes / (us * 1e-6) / 1e9
    # oracle on the first samples (at most 256), about a second of work
    ns = min(w.B, 256)
    x = synth.make_inputs(w, B=ns)
    t0 = time.perf_counter()
    passes = 0
    while True:
        oracle.backward_inputs(x["h_history"], x["h_s2"], x["W_A"], x["W_B"], x["W_C"], w.K,
                               x["d_context"], w.a_shift)
        passes += 1
        if time.perf_counter() - t0 > 1.0:
            break
    t = time.perf_counter() - t0
    return {"entry": "gscan_backward_full_ex", "us_per_call": round(us, 3),
            "samples_per_s": round(w.B / (us * 1e-6), 1), "algorithmic_bytes": nbytes,
            "GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "over_backward_us": round(us - bwd_us, 3),
            "oracle": {"value": round(ns * passes / t, 1), "unit": "samples/s",
                       "cores": oracle.max_threads(),
                       "sample": f"first {ns} samples, fp64 input gradients, {passes} passes "
                                 f"in {t:.1f} s"}}


def enrich(w, sets, stream, fwd_us, reps):
    """gscan_forward_enrich per call (the context added into a [B, SH2]
    h_enriched at column 0, no separate context output), HIP events, rotated
    inputs; its time over the plain forward."""
    import torch

    from gated_linear_recurrence_history_amd import binding

    dev = sets[0]["h_history"].device
    he = torch.zeros((w.B, w.SH2), dtype=torch.float32, device=dev)
    fns = [binding.prepare_forward_enrich(t["h_history"], t["h_s2"], t["W_A"], t["W_B"],
                                          t["W_C"], w.K, he, 0, w.a_shift, stream) for t in sets]
    n = len(fns)
    for i in range(max(20, n)):
        fns[i % n]()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for i in range(reps):
        fns[i % n]()
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / reps
    # the forward's reads, plus the h_enriched slice read and written
    nbytes = w.fwd_bytes() - w.B * w.D * 4 + 2 * w.B * w.D * 4
    return {"entry": "gscan_forward_enrich", "h_enriched": [w.B, w.SH2], "col_offset": 0,
            "us_per_call": round(us, 3), "over_forward_us": round(us - fwd_us, 3),
            "algorithmic_bytes": nbytes,
            "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def cifg(stream, reps):
    """gscan_batched_cifg_update (independent mode) on the page's shape
    (batch 32, d_model 512, d_input 512) and on a batch of 256: HIP-event time
    per call, rotating over memory sets larger than the Infinity Cache, its
    algorithmic bytes (C read and written once) against 8 TB/s, and the
    oracle's time per call on the page's shape."""
    import numpy as np
    import torch

    import oracle
    from gated_linear_recurrence_history_amd import binding, synth, workloads as wl

    dev = torch.device("cuda:0")
    res = {}
    for w in (wl.CIFG_PAGE, wl.CifgWorkload("cifg_b256", 256, 512, 512)):
        x = synth.make_cifg_inputs(w)
        per = w.B * w.d_model * w.d_model * 4
        nsets = max(2, int(np.ceil(300e6 / per)))
        Cs = [torch.from_numpy(x["C"]).to(dev) for _ in range(nsets)]
        t = {k: torch.from_numpy(v).to(dev) for k, v in x.items() if k != "C"}
        fns = [binding.prepare_batched_cifg_update(C, t["H"], t["X"], t["W_f"], t["b_f"], stream)
               for C in Cs]
        for i in range(2 * nsets):
            fns[i % nsets]()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(reps):
            fns[i % nsets]()
        b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / reps
        nbytes = w.bytes()
        res[w.name] = dict(w.describe(), us_per_call=round(us, 3), algorithmic_bytes=nbytes,
                           GBs=round(nbytes / (us * 1e-6) / 1e9, 1),
                           hbm_frac=round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                           memory_sets=nsets)
        del Cs, t, fns
        torch.cuda.empty_cache()
        if w is wl.CIFG_PAGE:
            t0 = time.perf_counter()
            passes = 0
            while True:
                oracle.cifg_update(x["C"], x["H"], x["X"], x["W_f"], x["b_f"])
                passes += 1
                if time.perf_counter() - t0 > 1.0:
                    break
            el = time.perf_counter() - t0
            res[w.name]["oracle"] = {"us_per_call": round(el / passes * 1e6, 1),
                                     "cores": oracle.max_threads(),
                                     "sample": f"the same shape, {passes} calls in {el:.2f} s"}
    res["entry"] = "gscan_batched_cifg_update"
    return res


def all_configs(stream, workloads=None):
    """Forward and backward per call on every named workload: one input set
    each, the median of three batches of at least 20 calls per figure.  The
    tiny and headline sets fit in the 256 MB Infinity Cache, so their figures
    here are cache-warm (the headline line above rotates input sets); the
    larger sets exceed it."""
    import numpy as np
    import torch

    from gated_linear_recurrence_history_amd import binding, synth, workloads as wl

    dev = torch.device("cuda:0")
    res = {}
    for w in (wl.WORKLOADS if workloads is None else workloads):
        x = synth.make_inputs(w)
        t = {k: (torch.from_numpy(v.view(np.int16)).to(dev).view(torch.bfloat16)
                 if v.dtype == np.uint16 else torch.from_numpy(v).to(dev)) for k, v in x.items()}
        del x
        ctx = torch.empty((w.B, w.D), device=dev)
        dW = tuple(torch.empty((w.SH2, w.D), device=dev) for _ in range(3))
        ws = torch.empty(binding.backward_workspace_bytes(w.B, w.K, w.SH2, w.D,
                                                          w.in_dtype == "bf16"),
                         dtype=torch.uint8, device=dev)
        a = (t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"], w.K)
        f = binding.prepare_forward(*a, ctx, w.a_shift, stream)
        b = binding.prepare_backward(*a, t["d_context"], dW, ws, w.a_shift, stream)
        reps = max(20, min(200, int(2e8 // (w.fwd_bytes() + 1))))
        times = {}
        for name, fn in (("fwd", f), ("bwd", b)):
            for _ in range(3):
                fn()
            # the median of three timed batches, so that one stall of the
            # device (a clock change, another process) does not set the figure
            per = []
            for _ in range(3):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                e0.record(stream)
                for _ in range(reps):
                    fn()
                e1.record(stream)
                torch.cuda.synchronize()
                per.append(e0.elapsed_time(e1) * 1e3 / reps)
            times[name] = sorted(per)[1]
        tot = times["fwd"] + times["bwd"]
        byts = w.fwd_bytes() + w.bwd_bytes()
        # the step's floor: per pass the higher of its HBM time at 8 TB/s and
        # its bf16 MFMA time (three products per fp32 product, two for bf16 rows)
        split = SPLIT_PRODUCTS if w.in_dtype == "f32" else 2
        floor = sum(max(by / (HBM_PEAK_GBS * 1e9), split * fl / (BF16_PEAK_TFLOPS * 1e12)) * 1e6
                    for by, fl in ((w.fwd_bytes(), w.fwd_flops()), (w.bwd_bytes(), w.bwd_flops())))
        res[w.name] = {"B": w.B, "K": w.K, "SH2": w.SH2, "D": w.D, "in_dtype": w.in_dtype,
                       "fwd_us": round(times["fwd"], 2), "bwd_us": round(times["bwd"], 2),
                       "samples_per_s": round(w.B / (tot * 1e-6), 1),
                       "hbm_frac": round(byts / (tot * 1e-6) / (HBM_PEAK_GBS * 1e9), 4),
                       "floor_us": round(floor, 2), "frac_of_floor": round(floor / tot, 4),
                       "reps": reps, "batches": 3}
        del t, ctx, dW, ws
        torch.cuda.empty_cache()
    return res


def bias_grad(args, stream, reps, rows=524288, cols=3):
    """gscan_bias_grad_reduce on the IQN shape: per call (HIP events) over
    several distinct gradients, and the oracle's rate on the same shape."""
    import numpy as np
    import torch

    import oracle
    from gated_linear_recurrence_history_amd import binding

    dev = torch.device("cuda:0")
    rng = np.random.default_rng(5150)
    grads = [(rng.standard_normal((rows, cols)) * 3.0).astype(np.float32) for _ in range(4)]
    dg = [torch.from_numpy(g).to(dev) for g in grads]
    out = torch.empty(cols, dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, binding.lib().gscan_bias_grad_reduce_workspace_bytes(rows, cols)),
                     dtype=torch.uint8, device=dev)
    fns = [binding.prepare_bias_grad_reduce(g, out, ws, stream) for g in dg]
    for i in range(20):
        fns[i % len(fns)]()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for i in range(reps):
        fns[i % len(fns)]()
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / reps
    nbytes = rows * cols * 4 + cols * 4
    gbs = nbytes / (us * 1e-6) / 1e9
    t0 = time.perf_counter()
    passes = 0
    while True:
        oracle.column_sums(grads[passes % len(grads)])
        passes += 1
        if time.perf_counter() - t0 > 0.5:
            break
    t = time.perf_counter() - t0
    return {"entry": "gscan_bias_grad_reduce", "shape": [rows, cols], "us_per_call": round(us, 3),
            "algorithmic_bytes": nbytes, "GBs": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "oracle": {"us_per_call": round(t / passes * 1e6, 1), "cores": oracle.max_threads(),
                       "sample": f"the same shape, {passes} calls in {t:.2f} s"}}


def read_ceiling(stream, nbytes=1 << 30, reps=8):
    """GB/s of a read-only stream over `nbytes` (libgscan_calib.so), two
    buffers of that size read alternately (each exceeds the Infinity Cache,
    so every read comes from HBM); median over `reps` reads."""
    import ctypes

    import numpy as np
    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "gated_linear_recurrence_history_amd",
                                   "libgscan_calib.so"))
    lib.gscan_calib_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                     ctypes.c_void_p]
    lib.gscan_calib_read.restype = ctypes.c_int
    lib.gscan_calib_read_grid.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    bufs = [torch.full((nbytes // 4,), float(i + 1), dtype=torch.float32, device=dev)
            for i in range(2)]
    sink = torch.empty(lib.gscan_calib_read_grid(), dtype=torch.int32, device=dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    times = []
    for i in range(reps + 2):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        rc = lib.gscan_calib_read(bufs[i % 2].data_ptr(), nbytes, sink.data_ptr(), sh)
        b.record(stream)
        if rc != 0:
            raise RuntimeError(f"gscan_calib_read failed: {rc}")
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) * 1e-3)
    del bufs
    torch.cuda.empty_cache()
    return nbytes / float(np.median(times[2:])) / 1e9


def plan_kernels(w):
    """(forward kernel, backward phase-1 kernels) the launch plan picks for
    workload `w`: the library's rule, restated for labelling the bench line."""
    slices = w.D // 16
    groups = -(-w.B // 16)
    perblock = (16 % w.K == 0 or w.K in (32, 64)) and w.SH2 <= 256
    fwd = "gscan_fwd_kernel" if groups <= 512 else "gscan_fwd_persist_kernel"
    if slices == 1 and perblock and groups > 512:
        fwd = "gscan_fwd_rows_kernel"
    if slices >= 2 and (w.K >= 16 or groups <= 512):
        if any(slices % sv == 0 and sv * (w.SH2 // 32) <= 32 for sv in (4, 2)):
            fwd = "gscan_fwd_ms_kernel"
    tiles = w.K in (64, 256) and w.B % (256 // w.K) == 0 and w.D % 32 == 0
    if tiles and w.SH2 == 512:
        fwd = "gscan_fwd_tile_kernel"
    if tiles and w.SH2 == 512 and w.D % 64 == 0:
        return fwd, ("gscan_bwd_scan_kernel", "gscan_bwd_contract_kernel")
    if perblock:
        return fwd, ("gscan_bwd_rows_kernel",)
    return fwd, ("gscan_bwd_kernel",)


def traffic_record(kernel, workload):
    """HBM bytes per launch measured by rocprofv3 for this exact kernel source, or None."""
    from gated_linear_recurrence_history_amd import rocprof_summary as rs
    rec = rs.read_traffic(os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt"))
    if rec is None or rec.get("source_sha256") != rs.kernel_source_sha256():
        return None
    return rec


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

    # ---- the same steps with the backward on a set the forward did not
    # touch: set i + 2 was last read six passes (6 x 72 MiB) earlier
    # (needs five sets or more; with fewer the figure is left out)
    nr_ms = None
    if n >= 5:
        for i in range(2 * n):
            fwd[i % n]()
            bwd[(i + 2) % n]()
        r0 = torch.cuda.Event(enable_timing=True)
        r1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        r0.record(stream)
        for i in range(args.steps):
            fwd[i % n]()
            bwd[(i + 2) % n]()
        r1.record(stream)
        torch.cuda.synchronize()
        nr_ms = r0.elapsed_time(r1) / args.steps

    # ---- the same steps captured once as a HIP graph (one step per input
    # set, the calls prepared on the capture stream) and replayed: what the
    # per-call host work and the launch gaps cost the eager loop
    graph_ms = None
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        cap = torch.cuda.current_stream(dev)
        gsteps = []
        for t in sets:
            a = (t["h_history"], t["h_s2"], t["W_A"], t["W_B"], t["W_C"], w.K)
            gsteps.append((binding.prepare_forward(*a, ctx, w.a_shift, cap),
                           binding.prepare_backward(*a, t["d_context"], dW, ws, w.a_shift, cap)))
        for f_, b_ in gsteps:
            f_()
            b_()
    torch.cuda.synchronize()
    greps = max(1, args.steps // n)
    g.replay()
    torch.cuda.synchronize()
    q0 = torch.cuda.Event(enable_timing=True)
    q1 = torch.cuda.Event(enable_timing=True)
    q0.record(stream)
    for _ in range(greps):
        g.replay()
    q1.record(stream)
    torch.cuda.synchronize()
    graph_ms = q0.elapsed_time(q1) / (greps * n)
    del g

    # ---- per-kernel durations: each kernel launched back to back on the same
    # stream (rotating the input sets), HIP events around the whole run
    reps = max(20, min(args.steps, 200))

    def per_launch_us(fn):
        # the median of three timed runs, so that one stall of the device
        # does not set the figure
        per = []
        for _ in range(3):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for i in range(reps):
                fn(i)
            b.record(stream)
            torch.cuda.synchronize()
            per.append(a.elapsed_time(b) * 1e3 / reps)
        return sorted(per)[1]

    for i in range(n):  # workspace holds partials of set i before each reduce
        bwd1[i]()
    k_fwd = per_launch_us(lambda i: fwd[i % n]())
    k_bwd = per_launch_us(lambda i: bwd1[i % n]())
    k_red = per_launch_us(lambda i: red())

    # ---- spread of single steps (outside the timed region): an event pair
    # around each of `reps` steps, then percentiles of the per-step times
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for i in range(reps):
        ev[i][0].record(stream)
        fwd[i % n]()
        bwd[i % n]()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per_step = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    step_us = {q: round(float(np.percentile(per_step, pq)), 3)
               for q, pq in (("p10", 10), ("p50", 50), ("p90", 90))}

    # ---- a measured streaming ceiling for context: a device-to-device copy
    # of 512 MiB (read + write bytes over its HIP-event time, median of 5)
    cb = 512 << 20
    csrc = torch.empty(cb, dtype=torch.uint8, device=dev)
    cdst = torch.empty_like(csrc)
    ctimes = []
    for _ in range(6):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        cdst.copy_(csrc)
        b.record(stream)
        torch.cuda.synchronize()
        ctimes.append(a.elapsed_time(b) * 1e-3)
    copy_gbs = 2 * cb / float(np.median(ctimes[1:])) / 1e9
    del csrc, cdst

    rd_gbs = read_ceiling(stream)

    step_bytes = w.fwd_bytes() + w.bwd_bytes()
    value = w.B / (ms_step * 1e-3)
    hbm_frac = step_bytes / (ms_step * 1e-3) / (HBM_PEAK_GBS * 1e9)
    step_gbs = step_bytes / (ms_step * 1e-3) / 1e9

    # dominant kernel against HBM (its MFMA time, 3 bf16 products per fp32
    # product at the bf16 peak, is far below its HBM time)
    fname, bnames = plan_kernels(w)
    if k_bwd >= k_fwd:
        # the backward's phase 1: one kernel, or the split pair (scan pass and
        # contraction, timed together as one phase)
        kname, kus, kbytes, kflops = "+".join(bnames), k_bwd, w.bwd_bytes(), w.bwd_flops()
    else:
        bnames = (fname,)
        kname, kus, kbytes, kflops = fname, k_fwd, w.fwd_bytes(), w.fwd_flops()
    t_hbm_us = kbytes / (HBM_PEAK_GBS * 1e9) * 1e6
    # bf16 rows are exact in the high part: two products per fp32 product
    split = SPLIT_PRODUCTS if w.in_dtype == "f32" else 2
    t_mfma_us = split * kflops / (BF16_PEAK_TFLOPS * 1e12) * 1e6
    ach = kbytes / (kus * 1e-6) / 1e9
    recs = [traffic_record(k, w.name) for k in bnames]
    traffic = sum(r["traffic_bytes"] for r in recs) if all(recs) else None
    if t_hbm_us >= t_mfma_us:
        # bound by HBM: algorithmic bytes over time against 8 TB/s
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                "frac_of_read_ceiling": round(ach / rd_gbs, 4)}
    else:
        # bound by the matrix cores: the bf16 products the split arithmetic
        # issues over time against the bf16 peak
        tflops = split * kflops / (kus * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                "achieved_GBs": round(ach, 1)}
    roof.update({"traffic": traffic, "kernel": kname, "avg_us": round(kus, 3),
                 "algorithmic_bytes": kbytes, "algorithmic_flops": kflops,
                 "hbm_floor_us": round(t_hbm_us, 3), "mfma_floor_us": round(t_mfma_us, 3)})

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
        "dtype": ("f32 (bf16x3 split products, fp32 accumulate)" if w.in_dtype == "f32"
                  else "bf16 in, f32 weights (bf16 MFMA products, fp32 accumulate)"),
        "data": "synthetic",
        "config": dict(w.describe(), input_sets=args.sets),
        "hbm_frac": round(hbm_frac, 4),
        "hbm_GBs_fwd_bwd": round(step_gbs, 1),
        "read_ceiling_GBs": round(rd_gbs, 1),
        "frac_of_read_ceiling": round(step_gbs / rd_gbs, 4),
        "no_reuse": None if nr_ms is None else {
            "ms_per_step": round(nr_ms, 5),
            "samples_per_s": round(w.B / (nr_ms * 1e-3), 1),
            "hbm_frac": round(step_bytes / (nr_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "frac_of_read_ceiling": round(step_bytes / (nr_ms * 1e-3) / 1e9 / rd_gbs, 4),
            "backward_set_offset": 2},
        "graph_ms_per_step": None if graph_ms is None else round(graph_ms, 5),
        "step_us": step_us,
        "copy_GBs": round(copy_gbs, 1),
        "wall_ms_per_step": round(wall / args.steps * 1e3, 5),
        "kernels_us": {"forward": round(k_fwd, 3), "backward_phase1": round(k_bwd, 3),
                       "gscan_reduce_kernel": round(k_red, 3)},
        "roofline": roof,
    }
    if not args.no_input_grads:
        out["input_grads"] = input_grads(args, w, sets, stream, k_bwd + k_red, reps)
    out["enrich"] = enrich(w, sets, stream, k_fwd, reps)
    out["cifg"] = cifg(stream, reps)
    if not args.no_bias_grad:
        out["bias_grad_reduce"] = bias_grad(args, stream, reps)
    if not args.no_configs:
        pick = set(args.configs.split(",")) if args.configs else None
        sel = lambda ws: [c for c in ws if pick is None or c.name in pick]  # noqa: E731
        out["configs"] = all_configs(stream, sel(wl.WORKLOADS))
        out["out_of_envelope"] = all_configs(stream, sel(wl.OUT_OF_ENVELOPE))
    if args.copy_calibration_mib > 0:
        nb = args.copy_calibration_mib << 20
        src = torch.ones(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = nb
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
