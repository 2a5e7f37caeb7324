"""Host-side checks of the benchmark and its probe library (no GPU needed): the probe library exports
what include/mlp_ceiling.h declares, the benchmark refuses more than one GPU with a message, and the
throughput arithmetic is right."""
import re
import subprocess
import sys
from pathlib import Path

import bench

ROOT = Path(__file__).resolve().parents[1]


def test_ceiling_library_exports_declared_functions():
    import ctypes

    decls = set(re.findall(r"^\s*int\s+(mlp_ceiling\w+)\s*\(", (ROOT / "include" / "mlp_ceiling.h").read_text(), re.M))
    assert decls == {"mlp_ceiling_launch", "mlp_ceiling_empty_launch"}
    lib = ctypes.CDLL(str(ROOT / "mlp_neural_shading_amd" / "libmlp_ceiling.so"))
    for name in decls:
        assert hasattr(lib, name), name
    # argument checks happen before any HIP call
    lib.mlp_ceiling_empty_launch.argtypes = [ctypes.c_int, ctypes.c_void_p]
    assert lib.mlp_ceiling_empty_launch(0, None) == -1


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_throughput_arithmetic():
    # 1,048,576 evaluations in 0.0524288 ms = 20,000 M evals/s
    assert abs(bench.throughput_m_evals(1 << 20, 0.0524288) - 20000.0) < 1e-6


def test_layered_workloads_are_named_apart():
    from mlp_neural_shading_amd import binding as B
    from mlp_neural_shading_amd import workloads

    wide = workloads.get("layered1024")
    assert wide.widths == (64,) + (1024,) * 7 + (16,) and wide.batch == 65536
    deep = workloads.get("layered256")
    assert deep.widths == (256,) * 17 and deep.batch == 262144
    # the fused workloads' tables (which the FP8 and row-major tests iterate) do not list them
    assert not set(workloads.LAYERED) & set(workloads.WORKLOADS)
    assert not set(workloads.LAYERED_ALIASES) & set(workloads.ALIASES)
    # both run layer by layer: every width padded to the layered tiles
    assert B.mlp_plan_widths(wide.widths) == [64] + [1024] * 7 + [128]
    assert B.mlp_plan_widths(deep.widths) == [256] * 17
    # the deep narrow nets: every output width padded to 128 (64-wide layers keep K = 64)
    narrow = workloads.get("layered64deep")
    assert narrow.widths == (64,) * 17 + (16,) and narrow.batch == 1 << 20
    assert B.mlp_plan_widths(narrow.widths) == [64] + [128] * 17
    narrow128 = workloads.get("layered128deep")
    assert narrow128.widths == (128,) * 13 + (16,) and narrow128.batch == 1 << 20
    assert B.mlp_plan_widths(narrow128.widths) == [128] * 14
    fused = workloads.get("deep64fused")  # 16 layers: the deep generic fused kernel, not layer by layer
    assert fused.widths == (64,) * 16 + (16,) and fused.batch == 1 << 20
    assert B.mlp_testing_plan_kernel(fused.widths) == "mlp_fused<generic64v,L=16>"
    assert B.mlp_testing_plan_kernel(narrow.widths).startswith("mlp_layered")


def test_layered_workload_refuses_the_row_major_layout():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--workload", "layered1024", "--layout", "rowmajor"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "packed layout" in r.stderr


def test_clock_level_parser():
    assert bench.current_dpm_level("0: 500Mhz\n1: 2400Mhz *\n") == {"level": "1", "freq": "2400Mhz"}
    assert bench.current_dpm_level("S: 19Mhz *\n0: 500Mhz\n1: 2400Mhz\n") == {"level": "S", "freq": "19Mhz"}
    assert bench.current_dpm_level("0: 500Mhz\n1: 2400Mhz\n") is None
    assert "error" in bench.read_clocks() or "sclk" in bench.read_clocks()
