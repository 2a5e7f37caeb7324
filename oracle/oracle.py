"""TEST INFRASTRUCTURE ONLY: ctypes wrapper around the plain C CPU oracle (``mlp_oracle.c``).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this module.  The product library under ``mlp_neural_shading_amd/`` shares no code with it.

The oracle evaluates the eight-affine-layer FP16 network of "Profiling neural material inference"
("Experiment setup"): FP16 storage, FP32 accumulation (bias first, inputs in ascending order),
rounding to FP16 after every layer, and the vector leaky ReLU max(v, v * half(0.01)) from "Bad versus
good activation" after every layer but the last.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "mlp_oracle.c"
_LIB = _HERE / "liboracle.so"

# Plain, strict IEEE flags: no fast-math, no contraction, no vectorisation tricks that matter.
CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared"]


def build(force: bool = True, src: Path = _SRC, out: Path = _LIB) -> Path:
    """Compile the oracle source ``src`` with gcc into ``out`` (default ``oracle/liboracle.so``)."""
    out = Path(out)
    if force or not out.exists():
        tmp = out.with_name(out.name + ".tmp%d" % os.getpid())
        subprocess.run(["gcc", *CFLAGS, str(src), "-o", str(tmp), "-lm"], check=True)
        os.replace(tmp, out)
    return out


def _bind(path: Path) -> ctypes.CDLL:
    L = ctypes.CDLL(str(path))
    p = ctypes.c_void_p
    L.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
    L.oracle_f16_to_f32.restype = ctypes.c_float
    L.oracle_f32_to_f16.argtypes = [ctypes.c_float]
    L.oracle_f32_to_f16.restype = ctypes.c_uint16
    L.oracle_leaky_f16.argtypes = [ctypes.c_uint16]
    L.oracle_leaky_f16.restype = ctypes.c_uint16
    L.oracle_mlp_forward.argtypes = [ctypes.c_int, p, p, p, ctypes.c_int64, p, p]
    L.oracle_mlp_forward.restype = ctypes.c_int
    L.oracle_mlp_forward_rows.argtypes = [ctypes.c_int, p, p, p, p, ctypes.c_int64, p, p]
    L.oracle_mlp_forward_rows.restype = ctypes.c_int
    for name in ("oracle_f32_to_f16_array", "oracle_f16_to_f32_array", "oracle_leaky_f16_array",
                 "oracle_f32_to_e4m3_array", "oracle_e4m3_to_f32_array"):
        getattr(L, name).argtypes = [ctypes.c_int64, p, p]
        getattr(L, name).restype = None
    L.oracle_fp8_row_exponent.argtypes = [p, ctypes.c_int]
    L.oracle_fp8_row_exponent.restype = ctypes.c_int
    L.oracle_mlp_forward_fp8.argtypes = [ctypes.c_int, p, p, p, ctypes.c_int64, p, p]
    L.oracle_mlp_forward_fp8.restype = ctypes.c_int
    return L


def _ptr(a: np.ndarray) -> ctypes.c_void_p:
    return ctypes.c_void_p(a.ctypes.data)


class _Net:
    """Holds contiguous copies of the weights so the pointer tables stay valid during a call."""

    def __init__(self, weights, biases):
        if len(weights) != len(biases) or not weights:
            raise ValueError("need one bias vector per weight matrix")
        self.W = [_as_bits(w) for w in weights]
        self.b = [_as_bits(b) for b in biases]
        widths = [self.W[0].shape[1]] + [w.shape[0] for w in self.W]
        for l, w in enumerate(self.W):
            if w.shape != (widths[l + 1], widths[l]) or self.b[l].shape != (widths[l + 1],):
                raise ValueError("layer %d: weight %s / bias %s do not chain" % (l, w.shape, self.b[l].shape))
        self.widths = np.asarray(widths, dtype=np.int32)
        self.n_layers = len(self.W)
        self.wp = (ctypes.c_void_p * self.n_layers)(*[w.ctypes.data for w in self.W])
        self.bp = (ctypes.c_void_p * self.n_layers)(*[b.ctypes.data for b in self.b])


def _as_bits(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.float16:
        x = x.view(np.uint16)
    return np.ascontiguousarray(x, dtype=np.uint16)


class Oracle:
    """The oracle's entry points bound to one built copy of ``mlp_oracle.c``."""

    def __init__(self, path: Path):
        self.path = Path(path)
        self.L = _bind(self.path)

    # ---- codec and activation --------------------------------------------------------------

    def f32_to_f16_bits(self, x) -> np.ndarray:
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape, dtype=np.uint16)
        self.L.oracle_f32_to_f16_array(x.size, _ptr(x), _ptr(out))
        return out

    def f16_bits_to_f32(self, h) -> np.ndarray:
        h = np.ascontiguousarray(h, dtype=np.uint16)
        out = np.empty(h.shape, dtype=np.float32)
        self.L.oracle_f16_to_f32_array(h.size, _ptr(h), _ptr(out))
        return out

    def leaky_f16_bits(self, h) -> np.ndarray:
        h = np.ascontiguousarray(h, dtype=np.uint16)
        out = np.empty(h.shape, dtype=np.uint16)
        self.L.oracle_leaky_f16_array(h.size, _ptr(h), _ptr(out))
        return out

    # ---- FP8 E4M3 codec (the FP8 variant) --------------------------------------------------

    def f32_to_e4m3(self, x) -> np.ndarray:
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape, dtype=np.uint8)
        self.L.oracle_f32_to_e4m3_array(x.size, _ptr(x), _ptr(out))
        return out

    def e4m3_to_f32(self, c) -> np.ndarray:
        c = np.ascontiguousarray(c, dtype=np.uint8)
        out = np.empty(c.shape, dtype=np.float32)
        self.L.oracle_e4m3_to_f32_array(c.size, _ptr(c), _ptr(out))
        return out

    def fp8_row_exponent(self, row_bits) -> int:
        r = _as_bits(row_bits).ravel()
        return int(self.L.oracle_fp8_row_exponent(_ptr(r), r.size))

    # ---- network ---------------------------------------------------------------------------

    def mlp_forward_fp8(self, weights, biases, x, threads: int = 1) -> np.ndarray:
        """The FP8 variant of the network (E4M3 weights with a power-of-two scale per output row,
        E4M3 activations scaled by 16); same conventions as ``mlp_forward``."""
        return self._forward(self.L.oracle_mlp_forward_fp8, weights, biases, x, threads)

    def mlp_forward(self, weights, biases, x, threads: int = 1) -> np.ndarray:
        """Evaluate every row of ``x`` ([rows, widths[0]], fp16 or its uint16 bits).

        Returns the fp16 bit patterns [rows, widths[-1]] as uint16.  ``threads`` > 1 splits the rows
        into contiguous shards and runs the same single-threaded C routine on each shard concurrently
        (ctypes releases the GIL); rows are independent, so the split cannot change a result.
        """
        net = _Net(weights, biases)
        x = _as_bits(x)
        if x.ndim != 2 or x.shape[1] != net.widths[0]:
            raise ValueError("x must be [rows, %d]" % net.widths[0])
        rows = x.shape[0]
        y = np.empty((rows, int(net.widths[-1])), dtype=np.uint16)
        L = self.L

        def run(lo, hi):
            if hi > lo:
                rc = L.oracle_mlp_forward(net.n_layers, _ptr(net.widths), net.wp, net.bp, hi - lo,
                                          ctypes.c_void_p(x.ctypes.data + lo * x.strides[0]),
                                          ctypes.c_void_p(y.ctypes.data + lo * y.strides[0]))
                if rc != 0:
                    raise RuntimeError("oracle_mlp_forward failed (%d)" % rc)

        _sharded(run, rows, threads)
        return y

    def _forward(self, fn, weights, biases, x, threads):
        net = _Net(weights, biases)
        x = _as_bits(x)
        if x.ndim != 2 or x.shape[1] != net.widths[0]:
            raise ValueError("x must be [rows, %d]" % net.widths[0])
        rows = x.shape[0]
        y = np.empty((rows, int(net.widths[-1])), dtype=np.uint16)

        def run(lo, hi):
            if hi > lo:
                rc = fn(net.n_layers, _ptr(net.widths), net.wp, net.bp, hi - lo,
                        ctypes.c_void_p(x.ctypes.data + lo * x.strides[0]),
                        ctypes.c_void_p(y.ctypes.data + lo * y.strides[0]))
                if rc != 0:
                    raise RuntimeError("oracle forward failed (%d)" % rc)

        _sharded(run, rows, threads)
        return y

    def mlp_forward_rows(self, weights, biases, x, row_index, threads: int = 1) -> np.ndarray:
        """Evaluate only the rows ``row_index`` of ``x``; returns [len(row_index), widths[-1]] bits."""
        net = _Net(weights, biases)
        x = _as_bits(x)
        idx = np.ascontiguousarray(row_index, dtype=np.int64)
        if idx.size and (idx.min() < 0 or idx.max() >= x.shape[0]):
            raise IndexError("row index out of range")
        y = np.empty((idx.size, int(net.widths[-1])), dtype=np.uint16)
        L = self.L

        def run(lo, hi):
            if hi > lo:
                rc = L.oracle_mlp_forward_rows(net.n_layers, _ptr(net.widths), net.wp, net.bp, _ptr(x), hi - lo,
                                               ctypes.c_void_p(idx.ctypes.data + lo * 8),
                                               ctypes.c_void_p(y.ctypes.data + lo * y.strides[0]))
                if rc != 0:
                    raise RuntimeError("oracle_mlp_forward_rows failed (%d)" % rc)

        _sharded(run, idx.size, threads)
        return y


_default = None
_default_lock = threading.Lock()


def default() -> Oracle:
    """The oracle built from ``mlp_oracle.c`` in this directory (built with gcc on first use)."""
    global _default
    with _default_lock:
        if _default is None:
            if not _LIB.exists():
                build(force=True)
            _default = Oracle(_LIB)
    return _default


def lib() -> ctypes.CDLL:
    return default().L


def f32_to_f16_bits(x):
    return default().f32_to_f16_bits(x)


def f16_bits_to_f32(h):
    return default().f16_bits_to_f32(h)


def leaky_f16_bits(h):
    return default().leaky_f16_bits(h)


def mlp_forward(weights, biases, x, threads: int = 1):
    return default().mlp_forward(weights, biases, x, threads)


def mlp_forward_rows(weights, biases, x, row_index, threads: int = 1):
    return default().mlp_forward_rows(weights, biases, x, row_index, threads)


def mlp_forward_fp8(weights, biases, x, threads: int = 1):
    return default().mlp_forward_fp8(weights, biases, x, threads)


def _sharded(fn, n: int, threads: int) -> None:
    threads = max(1, min(int(threads), n if n > 0 else 1))
    if threads == 1:
        fn(0, n)
        return
    bounds = [n * t // threads for t in range(threads + 1)]
    errors = []

    def wrap(lo, hi):
        try:
            fn(lo, hi)
        except BaseException as e:  # pragma: no cover - re-raised below
            errors.append(e)

    ts = [threading.Thread(target=wrap, args=(bounds[t], bounds[t + 1])) for t in range(threads)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    if errors:
        raise errors[0]
