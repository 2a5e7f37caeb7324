#!/usr/bin/env python3
"""Benchmark of the fused FP16 MLP inference kernel on one MI355X.

One step = one complete inference pass (every layer, every row) over one batch that is already
resident in HBM: one mlp_infer call on the page-shaped workload, 65,536 fixed inputs each evaluated
16 times = 1,048,576 evaluations of the 8-layer 32->64x7->4 network ("Profiling neural material
inference", section "Experiment setup").  Prints one JSON line:

  value        M evals/s over exactly --steps steps (wall clock, synchronised on both sides)
  roofline     algorithmic FLOPs per launch / mean launch time (HIP events on the launch stream)
               against the FP16 dense MFMA peak; traffic from committed rocprofv3 counters
  variants     the page's two A/B comparisons: row-major vs packed weights, scalarised vs vector
               activation (per-dispatch event medians, interleaved per layout)
  cpu_baseline the CPU oracle on a bounded sample of the same rows, one host thread
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import statistics
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

METRIC = "M MLP evals/s (8-layer FP16, 1M evals); % of FP16 MFMA peak"
PEAK_FP16_TFLOPS = 2516.6  # MI355X dense FP16 MFMA: 256 CUs x 4,096 FLOP/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = ROOT / "profiles" / "traffic.json"
KERNEL_SOURCES = ["mlp_kernels.hip", "mlp_layout.h"]


def throughput_m_evals(evals: int, ms: float) -> float:
    """M evals/s for `evals` evaluations in `ms` milliseconds."""
    return evals / (ms * 1e-3) / 1e6


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        h.update((ROOT / "mlp_neural_shading_amd" / "csrc" / name).read_bytes())
    return h.hexdigest()[:16]


def load_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed counter runs, if they were taken on this source."""
    try:
        data = json.loads(TRAFFIC_FILE.read_text())
    except (OSError, ValueError):
        return None
    rec = data.get(workload, {}).get(kernel)
    if not rec or rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def time_dispatches(torch, fn, n: int):
    """Per-dispatch times (ms) from HIP events recorded on the launch stream around each call."""
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def measure_ceiling(torch):
    """FP16 MFMA throughput the device sustains on random operands (v_mfma_f32_32x32x16_f16 loop,
    4 waves per SIMD), alone and with 6 packed-FP16 VALU instructions per MFMA, and on all-zero
    operands (which switch little and so let the clock stay high); see mlp_ceiling.h."""
    import ctypes

    lib = ctypes.CDLL(str(ROOT / "mlp_neural_shading_amd" / "libmlp_ceiling.so"))
    lib.mlp_ceiling_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_int, ctypes.c_void_p]
    props = torch.cuda.get_device_properties(0)
    grid = props.multi_processor_count * 4
    gen = torch.Generator(device="cuda").manual_seed(1)
    random_ops = (torch.rand(16384, device="cuda", generator=gen) * 2 - 1).to(torch.float16)
    zero_ops = torch.zeros(16384, dtype=torch.float16, device="cuda")
    out = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
    clk = torch.zeros(2, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()
    res = {}
    for name, operands, k in (("valu_per_mfma_0", random_ops, 0), ("valu_per_mfma_6", random_ops, 6),
                              ("zero_operands", zero_ops, 0)):
        iters = 20000

        def run():
            rc = lib.mlp_ceiling_launch(k, grid, operands.data_ptr(), out.data_ptr(), clk.data_ptr(), iters,
                                        stream.cuda_stream)
            if rc != 0:
                raise RuntimeError("ceiling probe launch failed (%d)" % rc)

        run()
        ms = statistics.median(time_dispatches(torch, run, 3))
        cyc, ticks = clk.cpu().tolist()
        flops = grid * 4 * iters * 8 * 32768
        res[name] = {"tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                     "clock_mhz": round(cyc / (ticks / 100.0)) if ticks else None}
    return res


def cpu_baseline(wl, Ws, bs, x_dev, rows: int):
    import numpy as np
    import torch

    from oracle import oracle

    xb = x_dev[:rows].cpu().view(torch.int16).numpy().view(np.uint16)
    o = oracle.default()
    o.mlp_forward(Ws, bs, xb[:64])  # load and warm the library
    t0 = time.perf_counter()
    o.mlp_forward(Ws, bs, xb, threads=1)
    dt = time.perf_counter() - t0
    return {"value": round(throughput_m_evals(rows, dt * 1e3), 6), "unit": "M evals/s", "cores": 1,
            "kind": "oracle",
            "sample": "first %d of the %d rows, single-threaded C oracle (gcc -O2), %.1f s on %s"
                      % (rows, wl.batch, dt, platform.processor() or platform.machine())}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="page", help="workload name or alias (default: page)")
    ap.add_argument("--no-variants", action="store_true", help="skip the row-major / scalarised A/B")
    ap.add_argument("--cpu-rows", type=int, default=16384, help="rows of the CPU-oracle sample (0: skip)")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the random-operand MFMA ceiling probe")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy five times (scales HBM counters)")
    args = ap.parse_args()

    if args.copy_probe:
        import torch

        src = torch.randn(64 * 1024 * 1024, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read_per_launch": src.numel() * 4,
                          "copy_probe_bytes_written_per_launch": src.numel() * 4}))
        return 0

    if args.gpus != 1:
        print("bench.py measures one GPU: the workload's rows are independent, so N GPUs would each run "
              "the same kernel on 1/N of the rows; only --gpus 1 is supported.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from mlp_neural_shading_amd import binding as B
    from mlp_neural_shading_amd import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = workloads.get(args.workload)
    Ws, bs = wl.weights()
    x = wl.inputs(device=dev)
    y = torch.empty((wl.batch, wl.widths[-1]), dtype=torch.float16, device=dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    flops_per_launch = wl.flops_per_eval * wl.batch

    # One-time conversion (timed separately, as on the page): host pack + upload + sync.
    t0 = time.perf_counter()
    B.mlp_pack_weights(Ws, bs, B.MLP_LAYOUT_PACKED, sh)
    pack_ms = (time.perf_counter() - t0) * 1e3
    kernel = B.mlp_kernel_name(B.MLP_ACT_VECTOR)

    def step():
        B.mlp_infer_ex(wl.batch, x.data_ptr(), y.data_ptr(), sh, B.MLP_ACT_VECTOR)

    for _ in range(args.warmup):
        step()
    # The timed region: exactly --steps back-to-back steps, synchronised on both sides.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    # The same steps again, each bracketed by HIP events on the launch stream: kernel durations.
    launch_ms = time_dispatches(torch, step, args.steps)
    mean_launch_ms = statistics.fmean(launch_ms)
    achieved_tflops = flops_per_launch / (mean_launch_ms * 1e-3) / 1e12

    traffic = load_traffic(wl.name, kernel)
    roofline = {"bound": "mfma", "achieved": round(achieved_tflops, 2), "peak": PEAK_FP16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved_tflops / PEAK_FP16_TFLOPS, 4), "traffic": traffic,
                "kernel": kernel, "mean_launch_ms": round(mean_launch_ms, 6),
                "median_launch_ms": round(statistics.median(launch_ms), 6),
                "io_gbs": round(wl.io_bytes_per_eval * wl.batch / (mean_launch_ms * 1e-3) / 1e9, 1)}

    variants = {}
    if not args.no_variants:
        for layout, lname in ((B.MLP_LAYOUT_PACKED, "packed"), (B.MLP_LAYOUT_ROW_MAJOR, "rowmajor")):
            B.mlp_pack_weights(Ws, bs, layout, sh)
            times = {0: [], 1: []}
            for rnd in range(3):  # interleave the two activation forms, A B A B A B
                for act in (B.MLP_ACT_VECTOR, B.MLP_ACT_SCALARISED):
                    f = lambda a=act: B.mlp_infer_ex(wl.batch, x.data_ptr(), y.data_ptr(), sh, a)
                    for _ in range(3):
                        f()
                    times[act].append(statistics.median(time_dispatches(torch, f, 10)))
            for act, aname in ((B.MLP_ACT_VECTOR, "vector"), (B.MLP_ACT_SCALARISED, "scalarised")):
                med = statistics.median(times[act])
                variants["%s+%s" % (lname, aname)] = {
                    "median_of_medians_ms": round(med, 6),
                    "m_evals_per_s": round(throughput_m_evals(wl.batch, med), 1),
                    "frac_fp16_peak": round(flops_per_launch / (med * 1e-3) / 1e12 / PEAK_FP16_TFLOPS, 4),
                    "kernel": B.mlp_kernel_name(act)}
        B.mlp_pack_weights(Ws, bs, B.MLP_LAYOUT_PACKED, sh)

    if not args.no_ceiling:
        ceiling = measure_ceiling(torch)
        roofline["measured_ceiling"] = dict(ceiling, kind="v_mfma_f32_32x32x16_f16 loop on random FP16 operands")
        c = ceiling["valu_per_mfma_0"]["tflops"]
        roofline["frac_of_measured_ceiling"] = round(achieved_tflops / c, 4)

    cpu = None
    if args.cpu_rows > 0:
        cpu = cpu_baseline(wl, Ws, bs, x, min(args.cpu_rows, wl.unique_rows))

    out = {
        "metric": METRIC,
        "value": round(throughput_m_evals(wl.batch, ms_per_step), 1),
        "unit": "M evals/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": wl.name, "widths": list(wl.widths), "batch": wl.batch,
                   "unique_inputs": wl.unique_rows, "replicas": wl.replicas, "layout": "packed",
                   "activation": "vector", "flops_per_eval": wl.flops_per_eval},
        "frac_fp16_peak": roofline["frac"],
        "pack_ms": round(pack_ms, 4),
        "roofline": roofline,
        "variants": variants,
        "cpu_baseline": cpu,
        "device": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
