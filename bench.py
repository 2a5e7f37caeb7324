#!/usr/bin/env python3
"""Benchmark of the fused FP16 MLP inference kernel on one MI355X.

One step = one complete inference pass (every layer, every row) over one batch that is already
resident in HBM: one mlp_infer call on the page-shaped workload, 65,536 fixed inputs each evaluated
16 times = 1,048,576 evaluations of the 8-layer 32->64x7->4 network ("Profiling neural material
inference", section "Experiment setup").  Prints one JSON line:

  value        M evals/s over exactly --steps steps (wall clock, synchronised on both sides)
  roofline     algorithmic FLOPs per launch / mean launch time (HIP events on the launch stream)
               against the FP16 dense MFMA peak; traffic from committed rocprofv3 counters
  variants     the page's two A/B comparisons, row-major vs packed weights and scalarised vs vector
               activation: 3 processes, each timing 3 warm-ups + 10 dispatches per variant with HIP
               events (variants interleaved), reported as the median of the 3 process medians with
               min and max
  workloads    every workload (all five network shapes) timed the same way, with the FP16 MFMA and
               the HBM fraction of each
  dispatch     an empty kernel timed the same way, and the wall-clock gap between back-to-back steps
  overlap      mlp_infer on a second stream beside a copy or a GEMM: alone, serial and concurrent times
  layered      networks beyond the eight-layer kernels (widths > 128, more than 8 layers): layer by
               layer, or fused up to 16 layers
  clocks       the GPU clock levels the driver reports before and after the measurements
  cpu_baseline the CPU oracle on a bounded sample of the same rows, one host thread pinned to a core
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


def ceiling_lib():
    import ctypes

    lib = ctypes.CDLL(str(ROOT / "mlp_neural_shading_amd" / "libmlp_ceiling.so"))
    lib.mlp_ceiling_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_int, ctypes.c_void_p]
    lib.mlp_ceiling_empty_launch.argtypes = [ctypes.c_int, ctypes.c_void_p]
    return lib


def roofline_grid(B, wl) -> int:
    """Workgroups of the inference kernel for this workload (one per compute unit when persistent)."""
    import torch

    return torch.cuda.get_device_properties(0).multi_processor_count


def measure_empty_dispatch(torch, grid: int) -> float:
    """Median event-timed duration (ms) of an empty kernel with the inference kernel's grid size."""
    lib = ceiling_lib()
    stream = torch.cuda.current_stream()

    def run():
        if lib.mlp_ceiling_empty_launch(grid, stream.cuda_stream) != 0:
            raise RuntimeError("empty-kernel launch failed")

    for _ in range(3):
        run()
    return statistics.median(time_dispatches(torch, run, 10))


def variant_medians(torch, B, wl, Ws, bs, x, y, order=(0, 1)) -> dict:
    """One process's share of the A/B protocol: per layout (in `order`), pack, then for the vector and
    the scalarised activation in turn 3 warm-up dispatches and 10 event-timed ones; returns the median
    (ms) of each variant's 10."""
    sh = torch.cuda.current_stream().cuda_stream
    names = {B.MLP_LAYOUT_PACKED: "packed", B.MLP_LAYOUT_ROW_MAJOR: "rowmajor"}
    layouts = [B.MLP_LAYOUT_PACKED, B.MLP_LAYOUT_ROW_MAJOR]
    out = {}
    for i in order:
        layout = layouts[i]
        B.mlp_pack_weights(Ws, bs, layout, sh)
        for act, aname in ((B.MLP_ACT_VECTOR, "vector"), (B.MLP_ACT_SCALARISED, "scalarised")):
            f = lambda a=act: B.mlp_infer_ex(wl.batch, x.data_ptr(), y.data_ptr(), sh, a)
            for _ in range(3):
                f()
            out["%s+%s" % (names[layout], aname)] = {"ms": statistics.median(time_dispatches(torch, f, 10)),
                                                      "kernel": B.mlp_kernel_name(act)}
    B.mlp_pack_weights(Ws, bs, B.MLP_LAYOUT_PACKED, sh)
    return out


def summarise_variants(runs, wl) -> dict:
    """Median of the per-process medians, with min and max, for each variant."""
    flops = wl.flops_per_eval * wl.batch
    res = {}
    for name in runs[0]:
        ms = [r[name]["ms"] for r in runs]
        med = statistics.median(ms)
        res[name] = {"median_of_medians_ms": round(med, 6), "min_ms": round(min(ms), 6), "max_ms": round(max(ms), 6),
                     "processes": len(ms), "m_evals_per_s": round(throughput_m_evals(wl.batch, med), 1),
                     "frac_fp16_peak": round(flops / (med * 1e-3) / 1e12 / PEAK_FP16_TFLOPS, 4),
                     "kernel": runs[0][name]["kernel"]}
    return res


def protocol_variants(wl_name: str, processes: int = 3) -> list:
    """Run the A/B protocol in `processes` fresh processes, one after another (alternating which
    layout goes first); returns each process's medians."""
    import subprocess

    runs = []
    for i in range(processes):
        cmd = [sys.executable, str(Path(__file__).resolve()), "--protocol-child", "--workload", wl_name,
               "--layout-order", "01" if i % 2 == 0 else "10"]
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
        if r.returncode != 0:
            raise RuntimeError("A/B child process failed (%d): %s" % (r.returncode, r.stderr[-2000:]))
        runs.append(json.loads(r.stdout.strip().splitlines()[-1]))
    return runs


def measure_workloads(torch, B, workloads, skip: str) -> dict:
    """Every workload with the packed image: median of 20 event-timed dispatches (after 3 warm-ups),
    its M evals/s, its fraction of the FP16 MFMA peak and of the HBM peak, and the four variants
    (3 interleaved rounds in this process, median of the round medians)."""
    res = {}
    dev = torch.device("cuda:0")
    sh = torch.cuda.current_stream().cuda_stream
    for name, wl in workloads.WORKLOADS.items():
        Ws, bs = wl.weights()
        x = wl.inputs(device=dev)
        y = torch.empty((wl.batch, wl.widths[-1]), dtype=torch.float16, device=dev)
        B.mlp_pack_weights(Ws, bs, B.MLP_LAYOUT_PACKED, sh)
        f = lambda: B.mlp_infer(wl.batch, x.data_ptr(), y.data_ptr(), sh)
        for _ in range(3):
            f()
        ms = statistics.median(time_dispatches(torch, f, 20))
        tflops = wl.flops_per_eval * wl.batch / (ms * 1e-3) / 1e12
        gbs = wl.io_bytes_per_eval * wl.batch / (ms * 1e-3) / 1e9
        entry = {"widths": list(wl.widths), "batch": wl.batch, "median_ms": round(ms, 6),
                 "m_evals_per_s": round(throughput_m_evals(wl.batch, ms), 1), "tflops": round(tflops, 1),
                 "frac_fp16_peak": round(tflops / PEAK_FP16_TFLOPS, 4), "io_gbs": round(gbs, 1),
                 "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4), "kernel": B.mlp_kernel_name(B.MLP_ACT_VECTOR)}
        if name != skip:
            rounds = [variant_medians(torch, B, wl, Ws, bs, x, y, (0, 1) if r % 2 == 0 else (1, 0)) for r in range(3)]
            entry["variants"] = summarise_variants(rounds, wl)
        # the FP8 variant (E4M3 weights and activations, FP32 accumulation): same timing
        B.mlp_pack_weights(Ws, bs, B.MLP_LAYOUT_PACKED_FP8, sh)
        for _ in range(3):
            f()
        ms8 = statistics.median(time_dispatches(torch, f, 20))
        entry["fp8"] = {"median_ms": round(ms8, 6), "m_evals_per_s": round(throughput_m_evals(wl.batch, ms8), 1),
                        "speedup_vs_fp16": round(ms / ms8, 3),
                        "equiv_tflops": round(wl.flops_per_eval * wl.batch / (ms8 * 1e-3) / 1e12, 1),
                        "kernel": B.mlp_kernel_name(B.MLP_ACT_VECTOR)}
        res[name] = entry
        del x, y
        torch.cuda.empty_cache()
    return res


def measure_overlap(torch, B, wl, x, y) -> dict:
    """mlp_infer on its own stream beside a background workload on another stream (both at the default
    priority), against each alone and one after the other: the gap-filling of running them together.
    Backgrounds: a 512 MiB device copy (HBM-bound) and a 4096^3 FP16 matrix product (MFMA-bound).
    Times are HIP events: the earliest start to the latest end, median of 5."""
    dev = torch.device("cuda:0")
    s_mlp = torch.cuda.Stream(device=dev)
    s_bg = torch.cuda.Stream(device=dev)
    src = torch.empty(256 * 1024 * 1024, dtype=torch.float16, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    a = torch.randn(4096, 4096, device=dev).to(torch.float16)
    bm = torch.randn(4096, 4096, device=dev).to(torch.float16)
    c = torch.empty(4096, 4096, dtype=torch.float16, device=dev)
    backgrounds = {"copy_512MiB": lambda: dst.copy_(src), "gemm_fp16_4096": lambda: torch.matmul(a, bm, out=c)}
    reps = 4  # back-to-back calls of each side per measurement

    def mlp():
        for _ in range(reps):
            B.mlp_infer(wl.batch, x.data_ptr(), y.data_ptr(), s_mlp.cuda_stream)

    def timed(run_mlp, run_bg, together):
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        ends = []
        start.record(torch.cuda.current_stream())
        for st, fn in ((s_mlp, run_mlp), (s_bg, run_bg)):
            if fn is None:
                continue
            st.wait_stream(torch.cuda.current_stream())
            if not together and ends:
                st.wait_event(ends[-1])
            with torch.cuda.stream(st):
                fn()
            e = torch.cuda.Event(enable_timing=True)
            e.record(st)
            ends.append(e)
        torch.cuda.synchronize()
        return max(start.elapsed_time(e) for e in ends)

    res = {"calls_per_side": reps}
    for name, bg in backgrounds.items():
        def bg_run(bg=bg):
            for _ in range(reps):
                bg()
        for _ in range(2):
            timed(mlp, bg_run, True)
        alone_mlp = statistics.median(timed(mlp, None, False) for _ in range(5))
        alone_bg = statistics.median(timed(None, bg_run, False) for _ in range(5))
        serial = statistics.median(timed(mlp, bg_run, False) for _ in range(5))
        together = statistics.median(timed(mlp, bg_run, True) for _ in range(5))
        res[name] = {"mlp_alone_ms": round(alone_mlp, 4), "background_alone_ms": round(alone_bg, 4),
                     "serial_ms": round(serial, 4), "concurrent_ms": round(together, 4),
                     "saved_frac": round(1 - together / serial, 4)}
    del src, dst, a, bm, c
    torch.cuda.empty_cache()
    return res


def measure_layered(torch, B, workloads) -> dict:
    """Networks beyond the dedicated kernels and the eight-layer limit (layer by layer, or the deep
    generic fused kernel up to 16 layers): median of 10 event-timed dispatches after 40 warm-up calls
    (~40 ms: the first ~10 ms after the GPU has been idle run ~10 % slower while the clock ramps up),
    FLOPs = 2 * sum w_{l-1} w_l per row."""
    res = {}
    dev = torch.device("cuda:0")
    sh = torch.cuda.current_stream().cuda_stream
    for name, wl in workloads.LAYERED.items():
        widths, rows = wl.widths, wl.batch
        Ws, bs = wl.weights()
        x = wl.inputs(device=dev)
        y = torch.empty((rows, widths[-1]), dtype=torch.float16, device=dev)
        B.mlp_pack_weights(Ws, bs, B.MLP_LAYOUT_PACKED, sh)
        f = lambda: B.mlp_infer(rows, x.data_ptr(), y.data_ptr(), sh)
        for _ in range(40):
            f()
        ms = statistics.median(time_dispatches(torch, f, 10))
        tflops = wl.flops_per_eval * rows / (ms * 1e-3) / 1e12
        res[name] = {"median_ms": round(ms, 4), "m_evals_per_s": round(throughput_m_evals(rows, ms), 1),
                     "tflops": round(tflops, 1), "frac_fp16_peak": round(tflops / PEAK_FP16_TFLOPS, 4),
                     "kernel": B.mlp_kernel_name(B.MLP_ACT_VECTOR)}
        del x, y
    torch.cuda.empty_cache()
    return res


def current_dpm_level(text: str):
    """The line the amdgpu driver marks with '*' in a pp_dpm_* table ("1: 2400Mhz *"; the level is a
    number, or "S" for deep sleep), as {"level", "freq"}; None if no line is marked."""
    for line in text.splitlines():
        if line.rstrip().endswith("*") and ":" in line:
            level, freq = line.split(":", 1)
            return {"level": level.strip(), "freq": freq.replace("*", "").strip()}
    return None


def read_clocks() -> dict:
    """Current SCLK / MCLK levels from the amdgpu driver's DPM tables in sysfs, read in this process
    with no helper program; best effort, since the clocks cannot be locked here.  With several cards
    visible, the first one that has the tables is read."""
    import glob

    try:
        for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
            if os.path.exists(dev + "/pp_dpm_sclk"):
                mclk = dev + "/pp_dpm_mclk"
                return {"card": dev.split("/")[-2], "sclk": current_dpm_level(Path(dev + "/pp_dpm_sclk").read_text()),
                        "mclk": current_dpm_level(Path(mclk).read_text()) if os.path.exists(mclk) else None}
        return {"error": "no amdgpu DPM tables under /sys/class/drm"}
    except (OSError, ValueError) as e:
        return {"error": "%s: %s" % (type(e).__name__, str(e)[:200])}


def measure_device_pack(torch, B, wl, Ws, bs) -> float:
    """Median event-timed duration (ms) of the device-side conversion of the network's weights, which
    are copied to the device first; leaves the network packed."""
    import numpy as np

    dev = torch.device("cuda:0")
    dW = [torch.from_numpy(np.ascontiguousarray(W).view(np.int16)).to(dev) for W in Ws]
    db = [torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to(dev) for b in bs]
    sh = torch.cuda.current_stream().cuda_stream
    f = lambda: B.mlp_pack_weights_device([t.data_ptr() for t in dW], [t.data_ptr() for t in db], list(wl.widths),
                                          B.MLP_LAYOUT_PACKED, sh)
    for _ in range(3):
        f()
    # Each call allocates the image on the host side before it enqueues the conversion; a busy kernel
    # (~0.25 ms) queued ahead keeps the GPU occupied meanwhile, so the events bracket the conversion
    # kernel alone rather than the host's allocation time.
    lib = ceiling_lib()
    ops = torch.zeros(16384, dtype=torch.float16, device=dev)
    sink = torch.empty(256, dtype=torch.float32, device=dev)
    clk = torch.zeros(2, dtype=torch.int64, device=dev)
    times = []
    for _ in range(10):
        if lib.mlp_ceiling_launch(0, 1, ops.data_ptr(), sink.data_ptr(), clk.data_ptr(), 2000, sh) != 0:
            raise RuntimeError("busy-kernel launch failed")
        times += time_dispatches(torch, f, 1)
    return statistics.median(times)


def measure_ceiling(torch):
    """FP16 MFMA throughput the device sustains on random operands (v_mfma_f32_32x32x16_f16 loop,
    4 waves per SIMD), alone and with 6 or 7 packed-FP16 VALU instructions per MFMA (the fused kernel
    issues between the two), and on all-zero operands (which switch little and so let the clock stay
    high); see mlp_ceiling.h."""
    lib = ceiling_lib()
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
                              ("valu_per_mfma_7", random_ops, 7), ("zero_operands", zero_ops, 0)):
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
    # For scale: the vendor FP16 GEMM (torch.matmul -> hipBLASLt) on one large shape, random operands.
    m, k, n = 65536, 1024, 1024
    a = (torch.rand((m, k), device="cuda", generator=gen) * 2 - 1).to(torch.float16)
    b = (torch.rand((k, n), device="cuda", generator=gen) * 2 - 1).to(torch.float16)
    for _ in range(5):
        c = a @ b
    ms = statistics.median(time_dispatches(torch, lambda: a @ b, 20))
    res["vendor_gemm"] = {"tflops": round(2 * m * k * n / (ms * 1e-3) / 1e12, 1), "shape": "%dx%dx%d" % (m, k, n),
                          "library": "torch.matmul (hipBLASLt), FP16 in, FP32 accumulate"}
    del a, b, c
    return res


def cpu_model() -> str:
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(wl, Ws, bs, x_dev, rows: int):
    """The C oracle, single-threaded and pinned to one core, on the first `rows` rows."""
    import numpy as np
    import torch

    from oracle import oracle

    xb = x_dev[:rows].cpu().view(torch.int16).numpy().view(np.uint16)
    o = oracle.default()
    o.mlp_forward(Ws, bs, xb[:64])  # load and warm the library
    allowed = os.sched_getaffinity(0)
    core = max(allowed)
    os.sched_setaffinity(0, {core})  # this thread only
    try:
        t0 = time.perf_counter()
        o.mlp_forward(Ws, bs, xb, threads=1)
        dt = time.perf_counter() - t0
    finally:
        os.sched_setaffinity(0, allowed)
    return {"value": round(throughput_m_evals(rows, dt * 1e3), 6), "unit": "M evals/s", "cores": 1,
            "kind": "oracle",
            "sample": "first %d of the %d rows (%d distinct inputs in the batch), single-threaded C oracle (gcc %s) pinned "
                      "to CPU %d of %d visible, %.1f s on %s"
                      % (rows, wl.batch, wl.unique_rows, " ".join(oracle.CFLAGS[:4]), core, len(allowed), dt,
                         cpu_model())}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # After the GPU has been idle its first ~10 ms of work run ~10 % slower while the clock ramps up
    # (measured: ~60 us per step for the first 200 page-net steps, 54.3 us afterwards); the default
    # warm-up (~27 ms of the page net) covers that ramp.
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--workload", default="page", help="workload name or alias (default: page)")
    ap.add_argument("--no-variants", action="store_true", help="skip the row-major / scalarised A/B")
    ap.add_argument("--layout", choices=("packed", "rowmajor"), default="packed",
                    help="weight layout of the headline measurement (default: packed)")
    ap.add_argument("--activation", choices=("vector", "scalarised"), default="vector",
                    help="activation form of the headline measurement (default: vector)")
    ap.add_argument("--cpu-rows", type=int, default=65536, help="rows of the CPU-oracle sample (0: skip)")
    ap.add_argument("--no-workloads", action="store_true", help="skip the per-workload table")
    ap.add_argument("--no-overlap", action="store_true", help="skip the two-stream overlap measurement")
    ap.add_argument("--protocol-child", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--layout-order", default="01", help=argparse.SUPPRESS)
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

    if args.protocol_child:
        import torch

        from mlp_neural_shading_amd import binding as B
        from mlp_neural_shading_amd import workloads

        wl = workloads.get(args.workload)
        Ws, bs = wl.weights()
        x = wl.inputs(device="cuda:0")
        y = torch.empty((wl.batch, wl.widths[-1]), dtype=torch.float16, device="cuda:0")
        order = tuple(int(c) for c in args.layout_order)
        print(json.dumps(variant_medians(torch, B, wl, Ws, bs, x, y, order)), flush=True)
        return 0

    if args.gpus != 1:
        print("bench.py measures one GPU: the workload's rows are independent, so N GPUs would each run "
              "the same kernel on 1/N of the rows; only --gpus 1 is supported.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from mlp_neural_shading_amd import binding as B
    from mlp_neural_shading_amd import workloads

    wl = workloads.get(args.workload)
    layered_net = wl.name in workloads.LAYERED  # runs layer by layer: packed FP16 only, no A/B variants
    if layered_net and (args.layout != "packed" or args.activation != "vector"):
        print("%s runs layer by layer, which only the packed layout and the vector activation serve" % wl.name,
              file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    clocks_before = read_clocks()
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
    pack = {"host_ms": round(pack_ms, 4), "device_kernel_ms": round(measure_device_pack(torch, B, wl, Ws, bs), 6),
            "note": "host_ms: host packing + upload + synchronisation (wall clock); device_kernel_ms: the "
                    "conversion kernel of mlp_pack_weights_device from device-resident weights (HIP events "
                    "with the queue kept busy ahead, median of 10); the page quotes ~0.0086 ms for its conversion on its own GPU"}
    layout = B.MLP_LAYOUT_PACKED if args.layout == "packed" else B.MLP_LAYOUT_ROW_MAJOR
    B.mlp_pack_weights(Ws, bs, layout, sh)
    act = B.MLP_ACT_VECTOR if args.activation == "vector" else B.MLP_ACT_SCALARISED
    kernel = B.mlp_kernel_name(act)

    def step():
        B.mlp_infer_ex(wl.batch, x.data_ptr(), y.data_ptr(), sh, act)

    for _ in range(args.warmup):
        step()
    # The timed region: exactly --steps back-to-back steps, synchronised on both sides.  Two HIP
    # events on the launch stream bracket the same region: their interval over --steps is the
    # average launch duration on the GPU (the kernels run back to back, so it is the kernel time
    # plus the gap between consecutive kernels).
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    mean_launch_ms = ev0.elapsed_time(ev1) / args.steps
    achieved_tflops = flops_per_launch / (mean_launch_ms * 1e-3) / 1e12
    # The same steps again, each alone between its own pair of events (which adds the dispatch
    # latency between the first event and the kernel to every interval): reported for reference.
    launch_ms = time_dispatches(torch, step, args.steps)

    traffic = load_traffic(wl.name, kernel)
    roofline = {"bound": "mfma", "achieved": round(achieved_tflops, 2), "peak": PEAK_FP16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved_tflops / PEAK_FP16_TFLOPS, 4), "traffic": traffic,
                "kernel": kernel, "mean_launch_ms": round(mean_launch_ms, 6),
                "isolated_launch_ms": {"mean": round(statistics.fmean(launch_ms), 6),
                                       "median": round(statistics.median(launch_ms), 6),
                                       "min": round(min(launch_ms), 6)},
                "io_gbs": round(wl.io_bytes_per_eval * wl.batch / (mean_launch_ms * 1e-3) / 1e9, 1)}

    dispatch = {"empty_kernel_ms": round(measure_empty_dispatch(torch, roofline_grid(B, wl)), 6),
                "step_minus_kernel_ms": round(ms_per_step - mean_launch_ms, 6)}

    variants = {}
    if not args.no_variants and not layered_net:
        variants = summarise_variants(protocol_variants(wl.name), wl)

    if not args.no_ceiling:
        ceiling = measure_ceiling(torch)
        roofline["measured_ceiling"] = dict(ceiling, kind="v_mfma_f32_32x32x16_f16 loop on random FP16 operands")
        c = ceiling["valu_per_mfma_0"]["tflops"]
        roofline["frac_of_measured_ceiling"] = round(achieved_tflops / c, 4)

    overlap = None
    if not args.no_overlap:
        overlap = measure_overlap(torch, B, wl, x, y)

    per_workload = {}
    layered = {}
    if not args.no_workloads:
        per_workload = measure_workloads(torch, B, workloads, skip=wl.name)
        if wl.name in per_workload:
            per_workload[wl.name]["variants"] = variants
        layered = measure_layered(torch, B, workloads)
    clocks_after = read_clocks()

    cpu = None
    if args.cpu_rows > 0:
        # A bounded sample: at most --cpu-rows rows and at most the FLOPs of 65,536 rows of the
        # page-shaped network (~3.5 GFLOP, ~20 s for the oracle), so wide networks stay short too.
        rows = min(args.cpu_rows, wl.unique_rows, max(64, 65536 * 53760 // wl.flops_per_eval))
        cpu = cpu_baseline(wl, Ws, bs, x, rows)

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
                   "unique_inputs": wl.unique_rows, "replicas": wl.replicas, "layout": args.layout,
                   "activation": args.activation, "flops_per_eval": wl.flops_per_eval},
        "frac_fp16_peak": roofline["frac"],
        "pack_ms": round(pack_ms, 4),
        "pack": pack,
        "roofline": roofline,
        "variants": variants,
        "dispatch": dispatch,
        "overlap": overlap,
        "workloads": per_workload,
        "layered": layered,
        "clocks": {"before": clocks_before, "after": clocks_after,
                   "note": "clocks are not locked on this machine; the kernel-side clock of the ceiling probe "
                           "is in roofline.measured_ceiling"},
        "cpu_baseline": cpu,
        "device": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
