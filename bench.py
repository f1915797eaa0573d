#!/usr/bin/env python3
"""Benchmark of the hot path on one MI355X.

One step = the weight-gradient step of a Llama-3.1-8B-shaped linear layer at
T = 8192 tokens, the whole hot path:
  1. fused H16 RHT + MX block-32 quantize of dY [8192 x 4096] along T
     (column-wise, uniform E1M2 grid, Philox stochastic rounding, FP6 E2M3
     operand form),
  2. the same for X [8192 x 4096] (E1M2, RTNE),
  3. the block-scaled GEMM dW [4096 x 4096] = dY^T X on the FP6 matrix cores.
Inputs are synthetic (seeded numpy), resident in HBM before timing.  Four
input/output sets rotate so consecutive steps do not hit in the 256 MB
last-level cache.

Timing: W untimed warmup steps; then the timed region, K whole steps back to
back between two HIP events (ms_per_step); then each kernel K times back to
back between two events (after a 50 ms idle gap), which gives its average
launch duration without event records between launches; then, for the batched
quantize and the GEMM, 100 launches with an event recorded after each, whose
intervals give the median, p10 and p90 per launch (`distribution`; each
interval also holds its event's own time, so the median sits above the loop
average).

The JSON line reports the fused quantize bandwidth as `value` (algorithmic
bytes of both operands / the average duration of the one batched launch that
quantizes them), the GEMM
rate under `gemm`, the roofline of the dominant kernel and of each kernel,
and the CPU oracle timed on a bounded sample as `cpu_baseline` (one thread;
under `all_cores`, the same oracle on every host core this process may use, at
most 16, over both whole operands).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = {"fp4": 10100.0, "fp6": 10100.0}   # dense, TFLOP/s

T, N, K = 8192, 4096, 4096     # tokens, out features (dY cols), in features (X cols)


# HBM bytes per launch measured by rocprofv3 FETCH_SIZE / WRITE_SIZE runs of this
# bench, scaled by the factors a 1 GiB device copy gives the same counters
# (fetched = 2 x FETCH_SIZE, written = 1 x WRITE_SIZE; the summaries are
# profiles/wgrad_step_T8192_<variant>_hbm_traffic.md).  Each entry holds only for
# the kernel sources it was measured on: `sha` is sha256[:16] of those files,
# and a kernel whose sources have changed since reports traffic null.
KERNEL_SOURCES = {
    "wgrad_gemm": ["csrc/wgrad_gemm.hip"],
    "quantize_pair_col": ["csrc/quantize_col.hip", "csrc/mxq_device.hpp", "csrc/quant_out.hpp",
                          "csrc/mxq_host.hpp"],
}
MEASURED_TRAFFIC = {
    "e1m2": {
        "quantize_pair_col": {"read": 134663176, "write": 52428817, "sha": "4c5aef178e4e535a"},
        "wgrad_gemm": {"read": 157490367, "write": 67362663, "sha": "9f2a5bb780854909"},
    },
    "e2m1": {
        "quantize_pair_col": {"read": 134705574, "write": 35651600, "sha": "4c5aef178e4e535a"},
        "wgrad_gemm": {"read": 107135314, "write": 67381268, "sha": "9f2a5bb780854909"},
    },
}


def source_sha(kernel: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "fp4_microscaling_quantization_amd", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(variant: str, kernel: str):
    """HBM bytes per launch (read + write) if measured on the current sources."""
    m = MEASURED_TRAFFIC.get(variant, {}).get(kernel)
    if m is None or m["sha"] != source_sha(kernel):
        return None
    return m["read"] + m["write"]


def launch_percentiles(us: list) -> dict:
    """Median, p10 and p90 (linear interpolation between order statistics) of
    per-launch durations in microseconds."""
    xs = sorted(us)
    if not xs:
        raise ValueError("no launches")

    def q(p):
        h = (len(xs) - 1) * p
        lo = int(h)
        hi = min(lo + 1, len(xs) - 1)
        return xs[lo] + (xs[hi] - xs[lo]) * (h - lo)

    return {"median_us": round(q(0.5), 3), "p10_us": round(q(0.1), 3),
            "p90_us": round(q(0.9), 3), "launches": len(xs)}


# Rotating input/output sets of every timed loop span more than the 256 MB
# last-level cache (the MALL), so back-to-back launches cannot be served from it.
ROTATE_BYTES = 640 << 20


def n_sets(set_bytes: float, at_least: int = 4) -> int:
    """Rotating sets needed for set_bytes each to span ROTATE_BYTES."""
    return max(at_least, -(-ROTATE_BYTES // max(int(set_bytes), 1)))


def quant_bytes_per_elem(fmt: int) -> float:
    # read bf16 (2 B) + write codes (0.5 B FP4 / 0.75 B E2M3) + 1 scale byte per 32
    return 2.0 + (0.5 if fmt == 0 else 0.75) + 1.0 / 32


class HipEvent:
    """A HIP event created with hipEventDisableSystemFence: recording it takes a
    timestamp without the system-scope cache writeback / invalidate of a default
    event, so back-to-back kernels are timed without gaps of the event's own
    making.  Recorded on the stream the kernels are launched on."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes as C
        if HipEvent._hip is None:
            import torch  # noqa: F401  (loads the HIP runtime torch was built with)
            h = C.CDLL(HipEvent._loaded_runtime())
            h.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
            h.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
            h.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
            h.hipEventDestroy.argtypes = [C.c_void_p]
            HipEvent._hip = h
        self._C = C
        self.ev = C.c_void_p()
        st = HipEvent._hip.hipEventCreateWithFlags(C.byref(self.ev), self.DISABLE_SYSTEM_FENCE)
        if st != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({st})")

    @staticmethod
    def _loaded_runtime() -> str:
        # the HIP runtime already mapped into this process (the one torch and
        # libmxq use): opening it again by path returns the same instance
        with open("/proc/self/maps") as f:
            for line in f:
                path = line.split()[-1]
                if os.path.basename(path).startswith("libamdhip64.so"):
                    return path
        raise RuntimeError("no HIP runtime loaded in this process")

    def record(self, stream):
        st = HipEvent._hip.hipEventRecord(self.ev, self._C.c_void_p(stream.cuda_stream))
        if st != 0:
            raise RuntimeError(f"hipEventRecord failed ({st})")

    def elapsed_ms(self, end) -> float:
        ms = self._C.c_float()
        st = HipEvent._hip.hipEventElapsedTime(self._C.byref(ms), self.ev, end.ev)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({st})")
        return ms.value

    def __del__(self):
        if HipEvent._hip is not None and self.ev:
            HipEvent._hip.hipEventDestroy(self.ev)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--sets", type=int, default=4, help="rotating input/output sets")
    ap.add_argument("--variant", choices=["e1m2", "e2m1"], default="e1m2",
                    help="e1m2: UFP4 operands as FP6 E2M3; e2m1: MXFP4 operands as FP4")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time budget of the oracle baseline")
    ap.add_argument("--no-quality", action="store_true",
                    help="skip the bias / SQNR diagnostics")
    ap.add_argument("--no-fusion", action="store_true",
                    help="skip the fused / standalone / unfused quantize comparison")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the device-copy rate and the vendor-library GEMM reference")
    ap.add_argument("--no-layer-gemms", action="store_true",
                    help="skip the Fprop / Dgrad GEMM timings")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the timing of each workload's quantize call")
    ap.add_argument("--dist-launches", type=int, default=100,
                    help="launches per kernel for the per-launch duration distribution (0: skip)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--workloads-only", default=None, metavar="NAMES",
                    help="time only these workload quantize calls (comma-separated case "
                         "names, or 'all') and print their JSON object; for counter runs")
    ap.add_argument("--stats-only", action="store_true",
                    help="time only the bias statistics calls and print their JSON object; "
                         "for counter runs")
    ap.add_argument("--no-stats", action="store_true",
                    help="skip the timing of the bias statistics calls")
    ap.add_argument("--no-other-form", action="store_true",
                    help="skip the GEMM timed with the other operand form")
    ap.add_argument("--no-sr8", action="store_true",
                    help="skip the timing of the batched pair with 8-bit SR draws for dY")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from fp4_microscaling_quantization_amd import mxq, synth

    mxq.lib()  # fail loudly if the HIP library is not built
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.workloads_only is not None:
        only = None if args.workloads_only == "all" else set(args.workloads_only.split(","))
        if args.copy_calib:
            copy_calibration(torch, dev)
        rep = workloads_report(torch, mxq, synth, dev, max(args.steps, 10), only)
        print(json.dumps({"workloads": rep}), flush=True)
        return

    if args.stats_only:
        print(json.dumps({"stats": stats_report(torch, mxq, synth, dev, max(args.steps, 10))}),
              flush=True)
        return

    grid = mxq.GRID_E1M2 if args.variant == "e1m2" else mxq.GRID_E2M1
    fmt = mxq.FMT_E2M3 if args.variant == "e1m2" else mxq.FMT_FP4
    signs = synth.sign_mask(synth.SIGNS_WGRAD, 16)
    cfg_dy = mxq.qconfig(grid=grid, round=mxq.SR, hadamard_n=16, sign_mask=signs,
                         sr_seed=synth.SR_SEED_WGRAD)
    cfg_x = mxq.qconfig(grid=grid, round=mxq.RTNE, hadamard_n=16, sign_mask=signs)

    t0 = time.time()
    dy_np = synth.dy_8192x4096()
    x_np = synth.x_wgrad_8192x4096()
    print(f"[bench] inputs generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    def to_dev(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    sets = []
    dy0, x0 = to_dev(dy_np), to_dev(x_np)
    for s in range(args.sets):
        dy = dy0 if s == 0 else dy0.clone()
        xx = x0 if s == 0 else x0.clone()
        qd = mxq.empty_qtensor(N, T, fmt, dev, mxq.LAYOUT_MFMA)
        qx = mxq.empty_qtensor(K, T, fmt, dev, mxq.LAYOUT_MFMA)
        c = torch.empty((N, K), dtype=torch.float32, device=dev)
        sets.append((dy, xx, qd, qx, c))
    torch.cuda.synchronize()

    # the launches of each set, marshalled once so that the host stays ahead
    # of the GPU and the events time the kernels, not the launch path.  A step
    # is one batched quantize launch of both operands (X's RTNE tiles first,
    # then dY's SR tiles: 1-2% faster than the other order) and the GEMM; the
    # two separate quantize launches are timed as well, for comparison.
    calls = []
    for dy, xx, qd, qx, c in sets:
        col_dy = (qd[0], qd[1], fmt, mxq.LAYOUT_MFMA)
        col_x = (qx[0], qx[1], fmt, mxq.LAYOUT_MFMA)
        calls.append((
            mxq.prepare_quantize_batch([(cfg_x, xx, None, col_x), (cfg_dy, dy, None, col_dy)]),
            mxq.prepare_wgrad_gemm(qd[0], qd[1], fmt, grid, qx[0], qx[1], fmt, grid, c,
                                   mxq.LAYOUT_MFMA, N, K, T),
            mxq.prepare_quantize(cfg_dy, dy, col=col_dy),
            mxq.prepare_quantize(cfg_x, xx, col=col_x)))

    stream = torch.cuda.current_stream()

    def step(i):
        q_pair, gemm = calls[i % len(calls)][:2]
        q_pair()
        gemm()

    def timed(fn, n):
        """GPU time of n calls of fn(i), bracketed by two events (seconds)."""
        e0, e1 = HipEvent(), HipEvent()
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_ms(e1) * 1e-3

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # the timed region: K whole steps back to back
    w0 = time.perf_counter()
    t_steps = timed(step, args.steps)
    wall = time.perf_counter() - w0
    # each kernel's average launch duration: K launches of it back to back over
    # the same rotating sets (no event between launches); every loop starts
    # after the same short idle gap, so none inherits the power state the
    # loop before it left
    def own_loop(j):
        time.sleep(0.05)
        return timed(lambda i: calls[i % len(calls)][j](), args.steps) / args.steps
    t_qp, t_gm, t_qdy, t_qx = (own_loop(j) for j in range(4))

    # the same batched pair with 8-bit draws for dY's stochastic rounding
    # (half the Philox work per element), and dY alone that way
    if not args.no_sr8:
        cfg_dy8 = mxq.qconfig(grid=grid, round=mxq.SR, hadamard_n=16, sign_mask=signs,
                              sr_seed=synth.SR_SEED_WGRAD, sr_bits=8)
        calls8 = []
        for dy, xx, qd, qx, c in sets:
            col_dy = (qd[0], qd[1], fmt, mxq.LAYOUT_MFMA)
            col_x = (qx[0], qx[1], fmt, mxq.LAYOUT_MFMA)
            calls8.append((mxq.prepare_quantize_batch([(cfg_x, xx, None, col_x),
                                                       (cfg_dy8, dy, None, col_dy)]),
                           mxq.prepare_quantize(cfg_dy8, dy, col=col_dy)))

        def own_loop8(j):
            time.sleep(0.05)
            return timed(lambda i: calls8[i % len(calls8)][j](), args.steps) / args.steps
        t8_pair, t8_dy = own_loop8(0), own_loop8(1)

    # per-launch durations: n launches of one kernel back to back over the
    # rotating sets, an event recorded after each (events that take no system
    # fence, so the launches stay back to back); duration i = event i to i + 1
    def per_launch(j, n):
        evs = [HipEvent() for _ in range(n + 1)]
        time.sleep(0.05)
        torch.cuda.synchronize()
        evs[0].record(stream)
        for i in range(n):
            calls[i % len(calls)][j]()
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        return launch_percentiles([evs[i].elapsed_ms(evs[i + 1]) * 1e3 for i in range(n)])

    elems = T * N
    qbytes = elems * quant_bytes_per_elem(fmt)                           # per operand
    flops = 2.0 * N * K * T
    q_gbs = 2 * qbytes / t_qp / 1e9
    g_tflops = flops / t_gm / 1e12
    mfma_peak = MFMA_PEAK_TFLOPS["fp6" if fmt == mxq.FMT_E2M3 else "fp4"]

    kernels = {
        "quantize_pair_col": {"bound": "hbm", "avg_us": t_qp * 1e6,
                              "achieved": 2 * qbytes / t_qp / 1e9, "peak": HBM_PEAK_GBS,
                              "unit": "GB/s"},
        "wgrad_gemm": {"bound": "mfma", "avg_us": t_gm * 1e6,
                       "achieved": flops / t_gm / 1e12, "peak": mfma_peak, "unit": "TFLOP/s"},
    }
    for name_, k_ in kernels.items():
        k_["frac"] = k_["achieved"] / k_["peak"]
        for f in ("avg_us", "achieved", "frac"):
            k_[f] = round(k_[f], 4)
        k_["traffic"] = measured_traffic(args.variant, name_)
    dom_name = max(kernels, key=lambda n: kernels[n]["avg_us"])
    dom = dict(kernels[dom_name])
    dom["kernel"] = dom_name
    dom.pop("avg_us")

    rec = {
        "metric": "fused RHT+MXFP4 quantize GB/s (% HBM peak); MXFP4 Wgrad GEMM TFLOPS",
        "value": round(q_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_steps / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"wgrad step T={T}: dY[{T}x{N}] and X[{T}x{K}] bf16 -> H16 RHT + "
                        f"column-wise MX block-32 {args.variant.upper()} "
                        f"({'FP6 E2M3' if fmt == mxq.FMT_E2M3 else 'FP4'} operands in the matrix-core "
                        f"layout; dY SR, X RTNE)"
                        f" -> dW[{N}x{K}] fp32 block-scaled GEMM",
            "global_batch": T,
            "seq_len": T,
            "parallelism": "none (1 GPU)",
            "quantize_frac_hbm": round(q_gbs / HBM_PEAK_GBS, 4),
        },
        "step": {"gpu_ms": round(t_steps / args.steps * 1e3, 4),
                 "wall_ms": round(wall / args.steps * 1e3, 4),
                 "kernels_ms": round((t_qp + t_gm) * 1e3, 4)},
        "quantize_separate": {
            "dy_col_sr_us": round(t_qdy * 1e6, 3), "x_col_rtne_us": round(t_qx * 1e6, 3),
            "both_gbs": round(2 * qbytes / (t_qdy + t_qx) / 1e9, 2),
            "batched_speedup": round((t_qdy + t_qx) / t_qp, 4)},
        "quantize_sr8": None if args.no_sr8 else {
            "pair_us": round(t8_pair * 1e6, 3), "pair_gbs": round(2 * qbytes / t8_pair / 1e9, 2),
            "dy_col_sr8_us": round(t8_dy * 1e6, 3), "dy_gbs": round(qbytes / t8_dy / 1e9, 2)},
        "gemm": {"value": round(g_tflops, 2), "unit": "TFLOP/s", "peak": mfma_peak,
                 "frac": round(g_tflops / mfma_peak, 4)},
        "roofline": dom,
        "kernels": kernels,
    }

    if args.dist_launches > 0:
        rec["distribution"] = {"quantize_pair_col": per_launch(0, args.dist_launches),
                               "wgrad_gemm": per_launch(1, args.dist_launches),
                               "note": "event-to-event interval per launch, an event recorded "
                                       "after each; includes the event's own time"}

    if not args.no_other_form:
        rec["gemm_other_form"] = other_form_gemm_report(torch, mxq, synth, dev, dy0, x0,
                                                        args.variant, args.steps)

    if not args.no_quality:
        rec["quality"] = quality_report(torch, mxq, synth, dev)

    if not args.no_fusion:
        rec["fusion"] = fusion_ratios(torch, mxq, synth, dev, max(args.steps, 10))

    if not args.no_context:
        rec["context"] = context_report(torch, dev, kernels)

    if not args.no_workloads:
        rec["workloads"] = workloads_report(torch, mxq, synth, dev, max(args.steps, 10))

    if not args.no_stats:
        rec["stats"] = stats_report(torch, mxq, synth, dev, max(args.steps, 10))
    if not args.no_layer_gemms:
        rec["layer_gemms"] = layer_gemms_report(torch, mxq, synth, dev, grid, fmt,
                                                max(args.steps, 10), mfma_peak)

    if args.copy_calib:
        rec["copy_calib_bytes"] = copy_calibration(torch, dev)

    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(dy_np, x_np, cfg_dy, cfg_x, fmt, grid, args.cpu_seconds)

    print(json.dumps(rec), flush=True)


def other_form_gemm_report(torch, mxq, synth, dev, dy, x, variant, reps):
    """The step's GEMM with the other operand form, quantized from the same dY
    and X: FP4 codes on the E2M1 grid when the step runs E1M2 (FP6 operands),
    and FP6 codes on the E1M2 grid the other way round.  Timed as the step's
    own GEMM loop: `reps` launches back to back over rotating operand and
    output sets that span more than the last-level cache."""
    other = "e2m1" if variant == "e1m2" else "e1m2"
    grid = mxq.GRID_E2M1 if other == "e2m1" else mxq.GRID_E1M2
    fmt = mxq.FMT_FP4 if other == "e2m1" else mxq.FMT_E2M3
    signs = synth.sign_mask(synth.SIGNS_WGRAD, 16)
    cfg_dy = mxq.qconfig(grid=grid, round=mxq.SR, hadamard_n=16, sign_mask=signs,
                         sr_seed=synth.SR_SEED_WGRAD)
    cfg_x = mxq.qconfig(grid=grid, round=mxq.RTNE, hadamard_n=16, sign_mask=signs)
    qbytes = sum(mxq.qtensor_sizes(L, T, fmt, mxq.LAYOUT_MFMA)[0] for L in (N, K))
    calls, keep = [], []
    for i in range(n_sets(qbytes + 4 * N * K)):
        qd = mxq.empty_qtensor(N, T, fmt, dev, mxq.LAYOUT_MFMA)
        qx = mxq.empty_qtensor(K, T, fmt, dev, mxq.LAYOUT_MFMA)
        c = torch.empty((N, K), dtype=torch.float32, device=dev)
        mxq.quantize_batch([(cfg_x, x, None, (qx[0], qx[1], fmt, mxq.LAYOUT_MFMA)),
                            (cfg_dy, dy, None, (qd[0], qd[1], fmt, mxq.LAYOUT_MFMA))])
        keep.append((qd, qx, c))
        calls.append(mxq.prepare_wgrad_gemm(qd[0], qd[1], fmt, grid, qx[0], qx[1], fmt, grid, c,
                                            mxq.LAYOUT_MFMA, N, K, T))
    for c in calls:
        c()
    torch.cuda.synchronize()
    time.sleep(0.05)
    s = torch.cuda.current_stream()
    e0, e1 = HipEvent(), HipEvent()
    e0.record(s)
    for i in range(reps):
        calls[i % len(calls)]()
    e1.record(s)
    torch.cuda.synchronize()
    t = e0.elapsed_ms(e1) * 1e-3 / reps
    tf = 2.0 * N * K * T / t / 1e12
    peak = MFMA_PEAK_TFLOPS["fp4" if fmt == mxq.FMT_FP4 else "fp6"]
    del keep, calls
    torch.cuda.empty_cache()
    return {"variant": other, "operands": "FP4" if fmt == mxq.FMT_FP4 else "FP6 E2M3",
            "sets": n_sets(qbytes + 4 * N * K), "avg_us": round(t * 1e6, 2),
            "TFLOP_s": round(tf, 1), "frac": round(tf / peak, 4)}


def copy_calibration(torch, dev) -> int:
    """Three plain 1 GiB device-to-device copies: the kernel whose known byte
    count scales rocprofv3's FETCH_SIZE / WRITE_SIZE counters to bytes."""
    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    return 1 << 30


def context_report(torch, dev, kernels):
    """What this GPU delivers outside this library, measured after the timed
    region: a plain 1 GiB device-to-device copy (the practical HBM rate; each
    quantizer's rate is also given as a fraction of it), and the vendor's own
    block-scaled FP4 GEMM (hipBLASLt through torch._scaled_mm, E2M1 operands
    with E8M0 scales per 32, bf16 output) at the weight-gradient shape, for
    comparison with this library's GEMM (fp32 output)."""
    ctx = {}
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * n * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    ctx["device_copy_GBps"] = round(copy_gbs, 1)
    ctx["quantize_frac_of_copy"] = {k: round(v["achieved"] / copy_gbs, 4)
                                    for k, v in kernels.items() if v["unit"] == "GB/s"}
    del a, b
    try:
        g = torch.Generator(device=dev)
        g.manual_seed(5)
        qa = torch.randint(0, 256, (N, T // 2), dtype=torch.uint8, device=dev, generator=g)
        qb = torch.randint(0, 256, (K, T // 2), dtype=torch.uint8, device=dev, generator=g)
        sa = torch.randint(124, 131, (N, T // 32), dtype=torch.uint8, device=dev, generator=g)
        sb = torch.randint(124, 131, (K, T // 32), dtype=torch.uint8, device=dev, generator=g)
        fa, fb = qa.view(torch.float4_e2m1fn_x2), qb.view(torch.float4_e2m1fn_x2)
        ea, eb = sa.view(torch.float8_e8m0fnu), sb.view(torch.float8_e8m0fnu)

        def mm():
            return torch._scaled_mm(fa, fb.t(), ea, eb, out_dtype=torch.bfloat16)
        for _ in range(3):
            mm()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(20):
            mm()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / 20
        ctx["vendor_fp4_gemm"] = {"library": "hipBLASLt via torch._scaled_mm", "out_dtype": "bf16",
                                  "m": N, "n": K, "k": T, "avg_us": round(us, 2),
                                  "TFLOP_s": round(2.0 * N * K * T / (us * 1e-6) / 1e12, 1)}
    except Exception as ex:  # not every torch build has block-scaled FP4 products
        ctx["vendor_fp4_gemm"] = {"unavailable": f"{type(ex).__name__}: {str(ex)[:160]}"}
    torch.cuda.empty_cache()
    return ctx


def quality_report(torch, mxq, synth, dev):
    """What the method does to the numbers, computed by the library's own
    kernels (mxq_quantize, mxq_bias_stats, mxq_gemm_abt) on the GPU after the
    timed region:
      * shrinkage bias and SQNR per workload and grid (RTNE): delta_rel =
        sum sign(y)(yhat - y) / sum |y| (magnitude-weighted signed error),
        delta_norm = mean (|yhat| - |y|) / 2^e, SQNR in dB, the saturated
        fraction, and per grid level the count and mean normalized error;
      * the SQNR change the H16 rotation brings on the activation workload;
      * stochastic rounding on the gradient workload over 64 seeds: mean
        normalized error of the unsaturated elements (expected 0, with its
        5-sigma bound) and of the saturated ones (clamped, not unbiased);
      * the weight-gradient output against the fp64 product of the bf16
        inputs: SQNR and alpha = <C_hat, C> / <C, C> (1 = no shrinkage)."""
    import math
    import numpy as np

    def to_dev(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    def summarize(st, grid):
        n, ns = st["n"], st["n_saturated"]
        lc = [int(v) for v in st["level_count"]]
        return {"delta_rel": st["sum_signed_err"] / st["sum_abs_y"],
                "bucket_ratio": mxq.bucket_ratio(lc, grid),
                "delta_norm": st["sum_err_norm"] / n,
                "sqnr_db": 10.0 * math.log10(st["sum_y2"] / st["sum_err2"]),
                "saturated_frac": ns / n,
                "level_count": lc,
                "level_mean_norm_err": [round(e / c, 5) if c else None
                                        for e, c in zip(st["level_err_norm"], lc)]}

    def stats(x, axis, **kn):
        q = mxq.quantize(x, row=axis == 0, col=axis == 1, row_fmt=0, col_fmt=0, **kn)
        key = "row" if axis == 0 else "col"
        return mxq.bias_stats(x, axis, q[key][0], q[key][1], 0, **kn)

    grids = {"e2m1": mxq.GRID_E2M1, "e1m2": mxq.GRID_E1M2, "e2m1_max4": mxq.GRID_E2M1_MAX4,
             "e2m1_max3": mxq.GRID_E2M1_MAX3}
    rep = {}
    x1 = to_dev(synth.x_1024())
    rep["x_1024_row_n0"] = {g: summarize(stats(x1, 0, grid=v), v) for g, v in grids.items()}
    x2 = to_dev(synth.x_8192x4096())
    r2 = {}
    for g, v in grids.items():
        a = summarize(stats(x2, 0, grid=v), v)
        b = summarize(stats(x2, 0, grid=v, hadamard_n=16), v)
        r2[g] = {"n0": a, "h16": b, "delta_sqnr_db": b["sqnr_db"] - a["sqnr_db"],
                 "delta_bucket_ratio": b["bucket_ratio"] - a["bucket_ratio"]}
    rep["x_8192x4096_row"] = r2
    del x1, x2
    w = to_dev(synth.w_14336x4096())
    ws = synth.sign_mask(synth.SIGNS_W, 32)
    rep["w_14336x4096_h32_signs"] = {
        g: {"row": summarize(stats(w, 0, grid=v, hadamard_n=32, sign_mask=ws), v),
            "col": summarize(stats(w, 1, grid=v, hadamard_n=32, sign_mask=ws), v),
            "row_per_block_signs": summarize(stats(w, 0, grid=v, hadamard_n=32,
                                                   sign_mode=mxq.SIGNS_PER_BLOCK,
                                                   sign_seed=synth.SIGNS_W), v)}
        for g, v in grids.items()}
    del w
    dy = to_dev(synth.dy_16384x4096())
    ds = synth.sign_mask(synth.SIGNS_DY, 16)
    r4 = {g: summarize(stats(dy, 1, grid=v, hadamard_n=16, sign_mask=ds), v) for g, v in grids.items()}
    tot = tot_sat = 0.0
    n_unsat = n_sat = 0
    for seed in range(64):
        st = stats(dy, 1, grid=mxq.GRID_E1M2, round=mxq.SR, hadamard_n=16, sign_mask=ds,
                   sr_seed=seed)
        tot += st["sum_err_norm"] - st["sum_err_norm_sat"]
        tot_sat += st["sum_err_norm_sat"]
        n_unsat += st["n"] - st["n_saturated"]
        n_sat += st["n_saturated"]
    r4["e1m2_sr_64_seeds"] = {"unsaturated_mean_norm_err": tot / n_unsat,
                              "five_sigma_bound": 5 * 0.25 / math.sqrt(n_unsat),
                              "saturated_mean_norm_err": tot_sat / n_sat if n_sat else None,
                              "saturated_frac": n_sat / (n_sat + n_unsat)}
    rep["dy_16384x4096_col_h16_signs"] = r4
    del dy
    # weight-gradient output quality, both operand variants
    dyw, xw = to_dev(synth.dy_8192x4096()), to_dev(synth.x_wgrad_8192x4096())
    ref = dyw.double().t().contiguous() @ xw.double()
    sg = synth.sign_mask(synth.SIGNS_WGRAD, 16)
    r5 = {}
    for name, g, f in (("e1m2_e2m3", mxq.GRID_E1M2, mxq.FMT_E2M3), ("e2m1_fp4", mxq.GRID_E2M1, mxq.FMT_FP4),
                       ("e2m1_max4_fp4", mxq.GRID_E2M1_MAX4, mxq.FMT_FP4),
                       ("e2m1_max3_fp4", mxq.GRID_E2M1_MAX3, mxq.FMT_FP4)):
        qd = mxq.quantize(dyw, grid=g, round=mxq.SR, hadamard_n=16, sign_mask=sg,
                          sr_seed=synth.SR_SEED_WGRAD, row=False, col=True, col_fmt=f,
                          col_layout=mxq.LAYOUT_MFMA)["col"]
        qx = mxq.quantize(xw, grid=g, hadamard_n=16, sign_mask=sg, row=False, col=True,
                          col_fmt=f, col_layout=mxq.LAYOUT_MFMA)["col"]
        c = mxq.gemm_abt(qd[0], qd[1], f, g, qx[0], qx[1], f, g, layout=mxq.LAYOUT_MFMA,
                         m=4096, n=4096, k=8192).double()
        err = c - ref
        r5[name] = {"sqnr_db": 10.0 * math.log10(float((ref * ref).sum()) / float((err * err).sum())),
                    "alpha": float((c * ref).sum() / (ref * ref).sum())}
    rep["wgrad_8192_dW_vs_fp64"] = r5
    del dyw, xw, ref
    torch.cuda.empty_cache()

    def rnd(o):
        if isinstance(o, float):
            return float(f"{o:.6g}")
        if isinstance(o, dict):
            return {k: rnd(v) for k, v in o.items()}
        if isinstance(o, list):
            return [rnd(v) for v in o]
        return o
    return rnd(rep)


def fusion_ratios(torch, mxq, synth, dev, reps):
    """The rotation fused into the quantizer against the plain quantizer (no
    rotation) and against the unfused pair (a rotation kernel writing bf16,
    then the plain quantizer reading it back), on the activation workload
    (X 8192 x 4096, row-wise, H16) and the weight workload (W 14336 x 4096,
    row- and column-wise outputs, H32 + random signs).  Each variant is timed
    as `reps` back-to-back launches over rotating input/output sets whose
    quantizer bytes span more than the last-level cache (n_sets), twice in
    turn with the others; the faster of its two passes is reported."""
    import numpy as np

    def timed(calls):
        torch.cuda.synchronize()
        s = torch.cuda.current_stream()
        e0, e1 = HipEvent(), HipEvent()
        for c in calls[0]:
            c()
        torch.cuda.synchronize()
        e0.record(s)
        for i in range(reps):
            for c in calls[i % len(calls)]:
                c()
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_ms(e1) * 1e3 / reps          # us per repetition

    def to_dev(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    out = {}
    workloads = [
        ("activation_8192x4096_row_h16", synth.x_8192x4096(), 16, 0, True, False),
        ("weight_14336x4096_dual_h32", synth.w_14336x4096(), 32,
         synth.sign_mask(synth.SIGNS_W, 32), True, True),
    ]
    for name, x_np, hn, mask, row, col in workloads:
        rows, cols = x_np.shape
        sets = []
        x0 = to_dev(x_np)
        touched = rows * cols * (2.0 + (int(row) + int(col)) * (0.5 + 1.0 / 32))
        for i in range(n_sets(touched)):
            x = x0 if i == 0 else x0.clone()
            r = mxq.empty_qtensor(rows, cols, mxq.FMT_FP4, dev) if row else None
            c = mxq.empty_qtensor(cols, rows, mxq.FMT_FP4, dev) if col else None
            rot_r = torch.empty_like(x) if row else None
            rot_c = torch.empty_like(x) if col else None
            sets.append((x, r, c, rot_r, rot_c))
        fused, plain, unfused = [], [], []
        cf = mxq.qconfig(grid=mxq.GRID_E2M1, round=mxq.RTNE, hadamard_n=hn, sign_mask=mask)
        c0 = mxq.qconfig(grid=mxq.GRID_E2M1, round=mxq.RTNE)
        for x, r, c, rot_r, rot_c in sets:
            ro = (r[0], r[1], mxq.FMT_FP4) if row else None
            co = (c[0], c[1], mxq.FMT_FP4) if col else None
            fused.append([mxq.prepare_quantize(cf, x, row=ro, col=co)])
            plain.append([mxq.prepare_quantize(c0, x, row=ro, col=co)])
            u = []
            if row:
                u.append(mxq.prepare_rotate(x, mxq.AXIS_ROW, hn, mask, mxq.OUT_BF16, rot_r))
                u.append(mxq.prepare_quantize(c0, rot_r, row=ro))
            if col:
                u.append(mxq.prepare_rotate(x, mxq.AXIS_COL, hn, mask, mxq.OUT_BF16, rot_c))
                u.append(mxq.prepare_quantize(c0, rot_c, col=co))
            unfused.append(u)
        # two passes over the three pipelines, each after a short idle gap; the
        # faster pass of each counts (the first loop after setup runs while the
        # clocks are still ramping)
        tf = tp = tu = float("inf")
        for _ in range(2):
            for which in ("f", "p", "u"):
                time.sleep(0.05)
                if which == "f":
                    tf = min(tf, timed(fused))
                elif which == "p":
                    tp = min(tp, timed(plain))
                else:
                    tu = min(tu, timed(unfused))
        out[name] = {"sets": len(sets), "fused_us": round(tf, 2), "standalone_us": round(tp, 2),
                     "unfused_us": round(tu, 2),
                     "fused_over_standalone": round(tf / tp, 3),
                     "unfused_over_fused": round(tu / tf, 3)}
        del sets, fused, plain, unfused
        torch.cuda.empty_cache()
    return out


def workloads_report(torch, mxq, synth, dev, reps, only=None):
    """Every full-size quantize call of the five workloads (the parity tests'
    cases: the 1024 x 1024 activation, the 8192 x 4096 activation with both
    grids, the 14336 x 4096 weight with both outputs and both grids, the
    16384 x 4096 gradient with SR, and the two Wgrad operands) in its own
    back-to-back loop over rotating input/output sets that span more than
    the last-level cache (n_sets): average launch time and algorithmic
    bandwidth (2 B read per element; per output 0.5 or 0.75 B of codes plus
    1/32 B of scale per element).  `only`: the case names to run (all if
    None)."""
    import numpy as np
    out = {}
    s = torch.cuda.current_stream()
    for case in synth.workload_cases():
        if only is not None and case.name not in only:
            continue
        x_np = case.make()
        rows, cols = x_np.shape
        cfg = mxq.qconfig(**case.knobs())
        nout = int(case.row_out) + int(case.col_out)
        out_bytes = quant_bytes_per_elem(case.fmt) - 2.0     # codes + scale per element
        nbytes = rows * cols * (2.0 + nout * out_bytes)
        calls = []
        x0 = torch.from_numpy(x_np.view(np.int16)).to(dev).view(torch.bfloat16)
        for i in range(n_sets(nbytes)):
            x = x0 if i == 0 else x0.clone()
            lay = case.layout
            r = mxq.empty_qtensor(rows, cols, case.fmt, dev, lay) if case.row_out else None
            c = mxq.empty_qtensor(cols, rows, case.fmt, dev, lay) if case.col_out else None
            calls.append(mxq.prepare_quantize(cfg, x, row=(r[0], r[1], case.fmt, lay) if r else None,
                                              col=(c[0], c[1], case.fmt, lay) if c else None))
        for c in calls:
            c()
        torch.cuda.synchronize()
        time.sleep(0.05)
        e0, e1 = HipEvent(), HipEvent()
        e0.record(s)
        for i in range(reps):
            calls[i % len(calls)]()
        e1.record(s)
        torch.cuda.synchronize()
        t = e0.elapsed_ms(e1) * 1e-3 / reps
        out[case.name] = {"sets": len(calls), "avg_us": round(t * 1e6, 2),
                          "GBps": round(nbytes / t / 1e9, 1),
                          "frac_hbm": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4)}
        del calls
        torch.cuda.empty_cache()
    return out


def stats_report(torch, mxq, synth, dev, reps):
    """The bias statistics (mxq_bias_stats: rotate, dequantize and the fp64
    sums against the codes of one quantize) of the 8192 x 4096 activation, H16,
    E2M1, FP4 codes, along rows and along columns: `reps` back-to-back calls
    over rotating sets (input, codes, scales) that span more than the
    last-level cache.  Algorithmic bytes per call: 2 B read per element plus
    the 0.5 B of codes and 1/32 B of scale read back."""
    import numpy as np
    rows, cols = 8192, 4096
    kn = dict(grid=mxq.GRID_E2M1, hadamard_n=16)
    x0 = torch.from_numpy(synth.x_8192x4096().view(np.int16)).to(dev).view(torch.bfloat16)
    nbytes = rows * cols * (2.0 + 0.5 + 1.0 / 32)
    out = {}
    s = torch.cuda.current_stream()
    for axis, name in ((0, "x8192_h16_e2m1_row"), (1, "x8192_h16_e2m1_col")):
        key = "row" if axis == 0 else "col"
        wsb = mxq.lib().mxq_bias_stats_workspace_size(rows, cols, axis)
        calls = []
        for i in range(n_sets(nbytes)):
            x = x0 if i == 0 else x0.clone()
            q = mxq.quantize(x, row=axis == 0, col=axis == 1, **kn)[key]
            st = torch.zeros(256, dtype=torch.uint8, device=dev)
            ws = torch.empty(max(wsb, 8), dtype=torch.uint8, device=dev)
            calls.append(mxq.prepare_bias_stats(x, axis, q[0], q[1], mxq.FMT_FP4, st, ws, **kn))
        for c in calls:
            c()
        torch.cuda.synchronize()
        time.sleep(0.05)
        e0, e1 = HipEvent(), HipEvent()
        e0.record(s)
        for i in range(reps):
            calls[i % len(calls)]()
        e1.record(s)
        torch.cuda.synchronize()
        t = e0.elapsed_ms(e1) * 1e-3 / reps
        out[name] = {"sets": len(calls), "avg_us": round(t * 1e6, 2),
                     "GBps": round(nbytes / t / 1e9, 1),
                     "frac_hbm": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4)}
        del calls
        torch.cuda.empty_cache()
    return out


def layer_gemms_report(torch, mxq, synth, dev, grid, fmt, reps, peak):
    """The other two GEMMs of the MLP up-projection (8192 tokens, K = 4096,
    N = 14336) through mxq_gemm_abt, with operands in the matrix-core layout
    as the layer GEMM parity tests build them: Fprop Y = X W^T (m = 8192,
    n = 14336, k = 4096) and Dgrad dX = dY W (m = 8192, n = 4096, k = 14336).
    Each product runs `reps` times back to back over rotating operand and
    output sets that span more than the last-level cache."""
    import numpy as np
    T_, K_, N_ = 8192, 4096, 14336
    lay = mxq.LAYOUT_MFMA

    def to_dev(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    signs = synth.sign_mask(synth.SIGNS_W, 32)
    kw = dict(grid=grid, round=mxq.RTNE, hadamard_n=32, sign_mask=signs)
    kd = dict(grid=grid, round=mxq.SR, hadamard_n=32, sign_mask=signs, sr_seed=11)
    qx = mxq.quantize(to_dev(synth.x_8192x4096()), row=True, col=False, row_fmt=fmt,
                      row_layout=lay, **kw)["row"]
    qw = mxq.quantize(to_dev(synth.w_14336x4096()), row=True, col=True, row_fmt=fmt,
                      col_fmt=fmt, row_layout=lay, col_layout=lay, **kw)
    qd = mxq.quantize(to_dev(synth.dy_8192x14336()), row=True, col=False, row_fmt=fmt,
                      row_layout=lay, **kd)["row"]
    out = {}
    s = torch.cuda.current_stream()
    for name, a, b, m, n, k in (("fprop", qx, qw["row"], T_, N_, K_),
                                ("dgrad", qd, qw["col"], T_, K_, N_)):
        # rotating sets: operand copies and outputs spanning the last-level cache
        set_bytes = sum(t.numel() for t in (a[0], a[1], b[0], b[1])) + 4 * m * n
        calls, keep = [], []
        for i in range(n_sets(set_bytes)):
            ai = a if i == 0 else (a[0].clone(), a[1].clone())
            bi = b if i == 0 else (b[0].clone(), b[1].clone())
            c = torch.empty((m, n), dtype=torch.float32, device=dev)
            keep.append((ai, bi, c))
            calls.append(mxq.prepare_wgrad_gemm(ai[0], ai[1], fmt, grid, bi[0], bi[1], fmt, grid,
                                                c, lay, m, n, k, entry="mxq_gemm_abt"))
        for c in calls:
            c()
        torch.cuda.synchronize()
        time.sleep(0.05)
        e0, e1 = HipEvent(), HipEvent()
        e0.record(s)
        for i in range(reps):
            calls[i % len(calls)]()
        e1.record(s)
        torch.cuda.synchronize()
        t = e0.elapsed_ms(e1) * 1e-3 / reps
        tf = 2.0 * m * n * k / t / 1e12
        out[name] = {"m": m, "n": n, "k": k, "sets": len(calls), "avg_us": round(t * 1e6, 2),
                     "TFLOP_s": round(tf, 1), "frac": round(tf / peak, 4)}
        del keep, calls
        torch.cuda.empty_cache()
    return out


def cpu_baseline(dy_np, x_np, cfg_dy, cfg_x, fmt, grid, budget_s):
    """The CPU oracle, as it stands, on a bounded sample of the same step:
    column-wise quantization of the first c columns of dY and of X (all 8192
    tokens each), then the fp64 product of the first g x g outputs, g sized
    (from a 32 x 32 run) to the rest of the time budget."""
    import numpy as np

    from oracle import oracle as orc

    pd = orc.qparams(grid=cfg_dy.grid, round=cfg_dy.round, hadamard_n=cfg_dy.hadamard_n,
                     sign_mask=cfg_dy.sign_mask, sr_seed=cfg_dy.sr_seed)
    px = orc.qparams(grid=cfg_x.grid, round=cfg_x.round, hadamard_n=cfg_x.hadamard_n,
                     sign_mask=cfg_x.sign_mask)
    # calibrate on 8 columns, then size the sample to the budget
    t0 = time.perf_counter()
    orc.quantize_lines(dy_np, orc.AXIS_COL, pd, 0, 8, fmt)
    orc.quantize_lines(x_np, orc.AXIS_COL, px, 0, 8, fmt)
    per_col = (time.perf_counter() - t0) / 8
    ncol = int(max(8, min(N, budget_s / max(per_col, 1e-9))))
    t0 = time.perf_counter()
    cd, sd = orc.quantize_lines(dy_np, orc.AXIS_COL, pd, 0, ncol, fmt)
    cx, sx = orc.quantize_lines(x_np, orc.AXIS_COL, px, 0, ncol, fmt)
    tq = time.perf_counter() - t0
    qbytes = 2 * ncol * T * quant_bytes_per_elem(fmt)
    def gemm(g):
        a = orc.dequantize(cd[:g], sd[:g], grid, fmt)
        b = orc.dequantize(cx[:g], sx[:g], grid, fmt)
        t1 = time.perf_counter()
        orc.gemm_abt_f64(a, b)
        return time.perf_counter() - t1
    g, tg = 32, gemm(32)
    rest = budget_s - tq - tg
    if rest > 0 and ncol >= 64:
        g2 = int(32 * (rest / max(tg, 1e-9)) ** 0.5) // 32 * 32
        g2 = min(g2, ncol)
        if g2 > 32:
            g, tg = g2, gemm(g2)
    rec = {
        "value": round(qbytes / tq / 1e9, 5),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"column-wise quantize of {ncol} of {N} columns of dY and of X (T={T}) "
                  f"in {tq:.1f}s; fp64 GEMM of {g}x{g} outputs over K={T} in {tg:.1f}s",
        "gemm_tflops": round(2.0 * g * g * T / tg / 1e12, 6),
        "cpu": _cpu_model(),
    }
    rec["all_cores"] = cpu_baseline_threads(dy_np, x_np, pd, px, fmt, grid, tg / (2.0 * g * g * T))
    return rec


def oracle_threads() -> int:
    """Host threads for the all-core oracle run: the CPUs this process may use,
    at most 16 (one GPU's share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def split_range(n: int, parts: int) -> list:
    """[start, stop) bounds of `parts` near-equal consecutive pieces of range(n)."""
    parts = max(1, min(parts, n)) if n > 0 else 1
    q, r = divmod(n, parts)
    out, a = [], 0
    for i in range(parts):
        b = a + q + (1 if i < r else 0)
        out.append((a, b))
        a = b
    return out


def cpu_baseline_threads(dy_np, x_np, pd, px, fmt, grid, s_per_flop):
    """The same oracle on every core it may use: the column-wise quantization of
    both whole operands, columns split over threads (each oracle call is one C
    call, which releases the interpreter lock), and an fp64 GEMM sample split
    over output rows, sized to about 3 s."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    from oracle import oracle as orc

    nt = oracle_threads()
    pieces = split_range(N, nt)
    with ThreadPoolExecutor(max_workers=nt) as ex:
        t0 = time.perf_counter()
        res = list(ex.map(lambda ab: (orc.quantize_lines(dy_np, orc.AXIS_COL, pd, ab[0], ab[1] - ab[0], fmt),
                                      orc.quantize_lines(x_np, orc.AXIS_COL, px, ab[0], ab[1] - ab[0], fmt)),
                          pieces))
        tq = time.perf_counter() - t0
        cd = np.concatenate([r[0][0] for r in res])
        sd = np.concatenate([r[0][1] for r in res])
        cx = np.concatenate([r[1][0] for r in res])
        sx = np.concatenate([r[1][1] for r in res])
        # the GEMM sample: g x g outputs, g sized from the one-thread rate to ~3 s
        g = int((3.0 * nt / max(s_per_flop, 1e-15) / (2.0 * T)) ** 0.5) // 32 * 32
        g = max(32, min(g, N))
        # the GEMM's operands, dequantized outside the timed region (also split)
        rows = split_range(g, nt)
        a = np.concatenate(list(ex.map(lambda ab: orc.dequantize(cd[ab[0]:ab[1]], sd[ab[0]:ab[1]], grid, fmt), rows)))
        b = np.concatenate(list(ex.map(lambda ab: orc.dequantize(cx[ab[0]:ab[1]], sx[ab[0]:ab[1]], grid, fmt), rows)))
        t1 = time.perf_counter()
        list(ex.map(lambda ab: orc.gemm_abt_f64(a[ab[0]:ab[1]], b), rows))
        tg = time.perf_counter() - t1
    qbytes = 2 * N * T * quant_bytes_per_elem(fmt)
    return {
        "value": round(qbytes / tq / 1e9, 5),
        "unit": "GB/s",
        "cores": nt,
        "sample": f"column-wise quantize of all {N} columns of dY and of X (T={T}) over {nt} "
                  f"threads in {tq:.2f}s; fp64 GEMM of {g}x{g} outputs over K={T} in {tg:.1f}s",
        "gemm_tflops": round(2.0 * g * g * T / tg / 1e12, 6),
    }


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
