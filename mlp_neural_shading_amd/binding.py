"""Thin ctypes binding of the C ABI in ``include/mlp.h`` (argument marshalling only).

Every entry point has the C name.  Weights and biases are numpy FP16 arrays (or their uint16 bit
patterns); device buffers and streams are raw handles, e.g. ``tensor.data_ptr()`` and
``torch.cuda.current_stream().cuda_stream``.  ``infer`` is a convenience wrapper that takes torch
tensors and calls ``mlp_infer_ex`` on the current stream.  Nothing here computes: if the HIP library
is missing, every call raises.
"""
from __future__ import annotations

import ctypes
from pathlib import Path
from typing import Optional, Sequence

import numpy as np

LIB_PATH = Path(__file__).resolve().parent / "libmlp.so"

MLP_OK = 0
MLP_ERR_INVALID_ARGUMENT = -1
MLP_ERR_UNSUPPORTED = -2
MLP_ERR_NOT_PACKED = -3
MLP_ERR_OUT_OF_MEMORY = -4
MLP_ERR_HIP = -5
MLP_LAYOUT_ROW_MAJOR = 0
MLP_LAYOUT_PACKED = 1
MLP_LAYOUT_PACKED_FP8 = 2
MLP_ACT_VECTOR = 0
MLP_ACT_SCALARISED = 1
MLP_MAX_LAYERS = 64
MLP_MAX_WIDTH = 4096
MLP_FUSED_MAX_LAYERS = 8
MLP_FUSED_MAX_WIDTH = 128
MLP_FUSED_DEEP_MAX_LAYERS = 16

EXPORTED = (
    "mlp_packed_size", "mlp_plan_widths", "mlp_pack_host", "mlp_pack_weights", "mlp_pack_weights_device",
    "mlp_infer", "mlp_infer_noalloc",
    "mlp_infer_ex", "mlp_set_activation_mode", "mlp_kernel_name", "mlp_debug_read_packed",
    "mlp_last_error", "mlp_release",
    # include/mlp_testing.h
    "mlp_testing_pack_device_on_host", "mlp_testing_plan_kernel",
)


class MlpError(RuntimeError):
    def __init__(self, code: int, func: str, message: str):
        super().__init__("%s failed (%d): %s" % (func, code, message))
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError("HIP library %s is not built; run `python -m mlp_neural_shading_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(str(LIB_PATH))
        p, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        sig = {
            "mlp_packed_size": ([i32, p, i32, p], i32),
            "mlp_plan_widths": ([i32, p, i32, p], i32),
            "mlp_pack_host": ([i32, p, p, p, i32, p, sz], i32),
            "mlp_pack_weights": ([i32, p, p, p, i32, p], i32),
            "mlp_pack_weights_device": ([i32, p, p, p, i32, p], i32),
            "mlp_infer": ([i64, p, p, p], i32),
            "mlp_infer_noalloc": ([i64, p, p, p], i32),
            "mlp_infer_ex": ([i64, p, p, p, i32], i32),
            "mlp_set_activation_mode": ([i32], i32),
            "mlp_kernel_name": ([i32, p, sz], i32),
            "mlp_debug_read_packed": ([p, sz], i32),
            "mlp_last_error": ([], ctypes.c_char_p),
            "mlp_release": ([], None),
            "mlp_testing_pack_device_on_host": ([i32, p, p, p, i32, p, sz, p], i32),
            "mlp_testing_plan_kernel": ([i32, p, i32, p, sz], i32),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _check(rc: int, func: str) -> None:
    if rc != MLP_OK:
        raise MlpError(rc, func, mlp_last_error())


def _bits(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    return np.ascontiguousarray(a, dtype=np.uint16)


class _Weights:
    """Contiguous uint16 copies plus the pointer tables the C ABI takes."""

    def __init__(self, weights: Sequence, biases: Sequence):
        self.W = [_bits(w) for w in weights]
        self.b = [_bits(b) for b in biases]
        self.n = len(self.W)
        self.wp = (ctypes.c_void_p * max(self.n, 1))(*[w.ctypes.data for w in self.W])
        self.bp = (ctypes.c_void_p * max(self.n, 1))(*[b.ctypes.data for b in self.b])
        if self.n and self.W[0].ndim == 2:
            self.widths = np.asarray([self.W[0].shape[1]] + [w.shape[0] for w in self.W], dtype=np.int32)
        else:
            self.widths = np.zeros(self.n + 1, dtype=np.int32)


def _widths(widths) -> np.ndarray:
    return np.ascontiguousarray(widths, dtype=np.int32)


def _stream(stream) -> ctypes.c_void_p:
    return ctypes.c_void_p(int(stream) if stream else 0)


# ---- the C entry points ---------------------------------------------------------------------

def mlp_last_error() -> str:
    return lib().mlp_last_error().decode()


def mlp_packed_size(widths, layout: int = MLP_LAYOUT_PACKED) -> int:
    w = _widths(widths)
    out = ctypes.c_size_t()
    _check(lib().mlp_packed_size(len(w) - 1, w.ctypes.data, layout, ctypes.byref(out)), "mlp_packed_size")
    return out.value


def mlp_plan_widths(widths, layout: int = MLP_LAYOUT_PACKED) -> list:
    w = _widths(widths)
    out = np.zeros(len(w), dtype=np.int32)
    _check(lib().mlp_plan_widths(len(w) - 1, w.ctypes.data, layout, out.ctypes.data), "mlp_plan_widths")
    return out.tolist()


def mlp_pack_host(weights, biases, layout: int = MLP_LAYOUT_PACKED, widths=None) -> np.ndarray:
    ws = _Weights(weights, biases)
    w = _widths(ws.widths if widths is None else widths)
    n = mlp_packed_size(w, layout)
    dst = np.zeros(n, dtype=np.uint8)
    _check(lib().mlp_pack_host(len(w) - 1, w.ctypes.data, ws.wp, ws.bp, layout, dst.ctypes.data, n), "mlp_pack_host")
    return dst


def mlp_pack_weights(weights, biases, layout: int = MLP_LAYOUT_PACKED, stream=None, widths=None) -> None:
    ws = _Weights(weights, biases)
    w = _widths(ws.widths if widths is None else widths)
    _check(lib().mlp_pack_weights(len(w) - 1, w.ctypes.data, ws.wp, ws.bp, layout, _stream(stream)),
           "mlp_pack_weights")


def mlp_pack_weights_device(weight_ptrs, bias_ptrs, widths, layout: int = MLP_LAYOUT_PACKED, stream=None) -> None:
    """weight_ptrs / bias_ptrs: device addresses (ints, e.g. tensor.data_ptr()) of each layer's FP16
    [out][in] matrix and [out] bias; widths: the n_layers + 1 widths."""
    w = _widths(widths)
    n = len(w) - 1
    wp = (ctypes.c_void_p * max(n, 1))(*[int(a) for a in weight_ptrs])
    bp = (ctypes.c_void_p * max(n, 1))(*[int(a) for a in bias_ptrs])
    _check(lib().mlp_pack_weights_device(n, w.ctypes.data, wp if len(weight_ptrs) else None,
                                         bp if len(bias_ptrs) else None, layout, _stream(stream)),
           "mlp_pack_weights_device")


def mlp_infer(batch: int, in_ptr: int, out_ptr: int, stream=None) -> None:
    _check(lib().mlp_infer(int(batch), ctypes.c_void_p(in_ptr), ctypes.c_void_p(out_ptr), _stream(stream)),
           "mlp_infer")


def mlp_infer_noalloc(batch: int, in_ptr: int, out_ptr: int, stream=None) -> None:
    _check(lib().mlp_infer_noalloc(int(batch), ctypes.c_void_p(in_ptr), ctypes.c_void_p(out_ptr), _stream(stream)),
           "mlp_infer_noalloc")


def mlp_infer_ex(batch: int, in_ptr: int, out_ptr: int, stream=None, act_mode: int = MLP_ACT_VECTOR) -> None:
    _check(lib().mlp_infer_ex(int(batch), ctypes.c_void_p(in_ptr), ctypes.c_void_p(out_ptr), _stream(stream),
                              act_mode), "mlp_infer_ex")


def mlp_set_activation_mode(act_mode: int) -> None:
    _check(lib().mlp_set_activation_mode(act_mode), "mlp_set_activation_mode")


def mlp_kernel_name(act_mode: int = MLP_ACT_VECTOR) -> str:
    buf = ctypes.create_string_buffer(256)
    _check(lib().mlp_kernel_name(act_mode, buf, 256), "mlp_kernel_name")
    return buf.value.decode()


def mlp_debug_read_packed(nbytes: int) -> np.ndarray:
    dst = np.zeros(nbytes, dtype=np.uint8)
    _check(lib().mlp_debug_read_packed(dst.ctypes.data, nbytes), "mlp_debug_read_packed")
    return dst


def mlp_release() -> None:
    lib().mlp_release()


def mlp_testing_pack_device_on_host(weights, biases, layout: int = MLP_LAYOUT_PACKED, widths=None):
    """The device conversion kernel's work items run on the host: (image, exact_cover)."""
    ws = _Weights(weights, biases)
    w = _widths(ws.widths if widths is None else widths)
    n = mlp_packed_size(w, layout)
    dst = np.zeros(n, dtype=np.uint8)
    cover = ctypes.c_int(-1)
    _check(lib().mlp_testing_pack_device_on_host(len(w) - 1, w.ctypes.data, ws.wp, ws.bp, layout, dst.ctypes.data, n,
                                                 ctypes.byref(cover)), "mlp_testing_pack_device_on_host")
    return dst, bool(cover.value)


def mlp_testing_plan_kernel(widths, layout: int = MLP_LAYOUT_PACKED) -> str:
    """The kernel mlp_pack_weights would select for this shape and layout (host only)."""
    w = _widths(widths)
    buf = ctypes.create_string_buffer(256)
    _check(lib().mlp_testing_plan_kernel(len(w) - 1, w.ctypes.data, layout, buf, 256), "mlp_testing_plan_kernel")
    return buf.value.decode()


# ---- torch convenience ------------------------------------------------------------------------

def infer(x, out=None, act_mode: Optional[int] = None, stream=None):
    """Run the current network on a CUDA/HIP float16 tensor ``x`` [batch, w0]; returns ``out``."""
    import torch

    if x.dtype != torch.float16 or not x.is_cuda or not x.is_contiguous() or x.dim() != 2:
        raise ValueError("x must be a contiguous 2-D float16 tensor on the GPU")
    if out is None:
        raise ValueError("pass a preallocated float16 output tensor")
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    if act_mode is None:
        mlp_infer(x.shape[0], x.data_ptr(), out.data_ptr(), stream)
    else:
        mlp_infer_ex(x.shape[0], x.data_ptr(), out.data_ptr(), stream, act_mode)
    return out
