"""Host-side checks of the C ABI (no GPU needed): the library loads and exports every function that
include/mlp.h declares, validation errors come back before any HIP call, and the packer's images
follow the documented layout (checked by an unpacker written here from the layout description, not
from the library's code)."""
import ctypes
import re
from pathlib import Path

import numpy as np
import pytest

from mlp_neural_shading_amd import binding as B
from mlp_neural_shading_amd import workloads

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "mlp.h"


def _have_gpu() -> bool:
    try:
        import torch

        return torch.cuda.device_count() > 0
    except Exception:  # pragma: no cover
        return False


def test_library_exports_every_declared_function():
    text = HEADER.read_text() + (ROOT / "include" / "mlp_testing.h").read_text()
    decls = set(re.findall(r"^\s*(?:int|void|const char \*)\s*(mlp_\w+)\s*\(", text, re.M))
    assert decls == set(B.EXPORTED)
    L = B.lib()
    for name in decls:
        assert hasattr(L, name), name


def _err(fn, *args):
    with pytest.raises(B.MlpError) as e:
        fn(*args)
    return e.value.code


def test_shape_validation():
    assert _err(B.mlp_packed_size, [], 1) == B.MLP_ERR_INVALID_ARGUMENT            # n_layers 0 (one width)
    assert _err(B.mlp_packed_size, [4] * 66, 1) == B.MLP_ERR_INVALID_ARGUMENT      # 65 layers
    assert _err(B.mlp_packed_size, [4, 0, 4], 1) == B.MLP_ERR_INVALID_ARGUMENT
    assert _err(B.mlp_packed_size, [4, 4097, 4], 1) == B.MLP_ERR_INVALID_ARGUMENT
    # beyond the fused limits: the layer-by-layer path (packed layout only)
    assert B.mlp_packed_size([4, 129, 4], 1) > 0
    assert B.mlp_packed_size([4] * 10, 1) > 0
    assert _err(B.mlp_packed_size, [4, 129, 4], B.MLP_LAYOUT_ROW_MAJOR) == B.MLP_ERR_UNSUPPORTED
    assert _err(B.mlp_packed_size, [4, 4], 7) == B.MLP_ERR_INVALID_ARGUMENT        # unknown layout
    assert "widths[1]" in B.mlp_last_error() or "layout" in B.mlp_last_error()
    # row-major is compiled only for the dedicated shapes
    assert _err(B.mlp_packed_size, [5, 7, 3], B.MLP_LAYOUT_ROW_MAJOR) == B.MLP_ERR_UNSUPPORTED
    assert B.mlp_packed_size([5, 7, 3], B.MLP_LAYOUT_PACKED) > 0


def test_null_arguments_are_rejected():
    L = B.lib()
    w = np.array([4, 4], np.int32)
    assert L.mlp_packed_size(1, w.ctypes.data, 1, None) == B.MLP_ERR_INVALID_ARGUMENT
    assert L.mlp_packed_size(1, None, 1, ctypes.byref(ctypes.c_size_t())) == B.MLP_ERR_INVALID_ARGUMENT
    assert L.mlp_pack_host(1, w.ctypes.data, None, None, 1, None, 0) == B.MLP_ERR_INVALID_ARGUMENT
    assert L.mlp_plan_widths(1, w.ctypes.data, 1, None) == B.MLP_ERR_INVALID_ARGUMENT
    assert L.mlp_kernel_name(0, None, 0) == B.MLP_ERR_INVALID_ARGUMENT
    assert L.mlp_set_activation_mode(2) == B.MLP_ERR_INVALID_ARGUMENT
    # a too-small destination buffer
    Ws, bs = workloads.init_weights([4, 4])
    ws = B._Weights(Ws, bs)
    dst = np.zeros(16, np.uint8)
    assert L.mlp_pack_host(1, w.ctypes.data, ws.wp, ws.bp, 1, dst.ctypes.data, 16) == B.MLP_ERR_INVALID_ARGUMENT


def test_device_pack_validation():
    L = B.lib()
    w = np.array([4, 4], np.int32)
    null = (ctypes.c_void_p * 1)(0)
    good = (ctypes.c_void_p * 1)(0x10000)
    odd = (ctypes.c_void_p * 1)(0x10001)
    assert L.mlp_pack_weights_device(1, w.ctypes.data, None, good, 1, None) == B.MLP_ERR_INVALID_ARGUMENT
    assert L.mlp_pack_weights_device(1, w.ctypes.data, null, good, 1, None) == B.MLP_ERR_INVALID_ARGUMENT
    assert L.mlp_pack_weights_device(1, w.ctypes.data, good, odd, 1, None) == B.MLP_ERR_INVALID_ARGUMENT
    assert "aligned" in B.mlp_last_error()
    assert L.mlp_pack_weights_device(0, w.ctypes.data, good, good, 1, None) == B.MLP_ERR_INVALID_ARGUMENT
    # row-major is compiled for the dedicated shapes only
    w3 = np.array([5, 7, 3], np.int32)
    two = (ctypes.c_void_p * 2)(0x10000, 0x20000)
    assert L.mlp_pack_weights_device(2, w3.ctypes.data, two, two, B.MLP_LAYOUT_ROW_MAJOR, None) == B.MLP_ERR_UNSUPPORTED


def test_kernel_selection():
    """Which kernel each shape takes (mlp.h's fused limits): the dedicated instances for the workload
    shapes and layouts, the generic 64- and 128-wide families up to 8 layers (element by element
    without vector I/O), up to 16 layers with vector I/O (at widths above 64 unless one 128-wide chain
    serves the whole network), else the layer-by-layer path."""
    plan = B.mlp_testing_plan_kernel
    assert plan(workloads.get("page").widths) == "mlp_fused<32-64x7-4,packed,vector>"
    assert plan(workloads.get("page").widths, B.MLP_LAYOUT_ROW_MAJOR) == "mlp_fused<32-64x7-4,rowmajor,vector>"
    assert plan(workloads.get("wide").widths, B.MLP_LAYOUT_PACKED_FP8) == "mlp_fused_fp8<64-128x7-4>"
    assert plan([9, 64, 3]) == "mlp_fused<generic64,L=2>"
    assert plan([8, 64, 4]) == "mlp_fused<generic64v,L=2>"
    assert plan([9, 65, 3]) == "mlp_fused<generic128,L=2>"
    assert plan([64] * 9) == "mlp_fused<generic64v,L=8>"
    assert plan([64] * 17) == "mlp_fused<generic64v,L=16>"  # 16 narrow layers
    assert plan([64] * 18).startswith("mlp_layered")  # 17 layers
    assert plan([60] + [64] * 9).startswith("mlp_layered")  # 9 layers without vector I/O
    assert plan([64] + [128] * 9 + [4]) == "mlp_fused<generic128v,L=10>"
    assert plan([128] * 13 + [12]) == "mlp_fused<generic128v,L=13>"
    assert plan([128] * 14).startswith("mlp_layered")  # one 128-wide chain serves all 13 layers
    assert plan([64] + [128] * 12 + [16]).startswith("mlp_layered")  # likewise, a 64-wide input
    assert plan([72] + [128] * 12 + [16]) == "mlp_fused<generic128v,L=13>"  # 72 is not its own padding
    assert plan([64, 256, 16]).startswith("mlp_layered")  # a width above 128
    with pytest.raises(B.MlpError) as e:
        plan([64] * 17, B.MLP_LAYOUT_ROW_MAJOR)
    assert e.value.code == B.MLP_ERR_UNSUPPORTED


DEVICE_PACK_CASES = [(name, layout) for name in ["small", "page", "hetero", "wide", "stream"]
                     for layout in (B.MLP_LAYOUT_PACKED, B.MLP_LAYOUT_ROW_MAJOR, B.MLP_LAYOUT_PACKED_FP8)]
DEVICE_PACK_CASES += [("generic-5-7-3", B.MLP_LAYOUT_PACKED), ("generic-100-30-7", B.MLP_LAYOUT_PACKED),
                      ("layered-100-300-129-7", B.MLP_LAYOUT_PACKED), ("generic-40x11", B.MLP_LAYOUT_PACKED),
                      ("generic-32-64x15-12", B.MLP_LAYOUT_PACKED), ("generic-72x10", B.MLP_LAYOUT_PACKED),
                      ("layered-40x18", B.MLP_LAYOUT_PACKED), ("layered-16x34", B.MLP_LAYOUT_PACKED)]


@pytest.mark.parametrize("name,layout", DEVICE_PACK_CASES)
def test_device_conversion_items_run_on_the_host(name, layout):
    """The device conversion kernel's own per-item code, run on the host over every work item: each
    byte of the image is written exactly once and nothing outside it, and the image equals the host
    packer's (weights with both signs and a wide range of magnitudes, so the FP8 row scales differ)."""
    if name.startswith("generic") or name.startswith("layered"):
        parts = name.split("-")[1:]
        widths = tuple(int(p.split("x")[0]) for p in parts for _ in range(int(p.split("x")[1]) if "x" in p else 1))
    else:
        widths = workloads.get(name).widths
    Ws, bs = workloads.init_weights(widths, seed=13)
    rng = np.random.default_rng(13)
    Ws = [(np.asarray(W, np.float64) * np.exp2(rng.integers(-6, 7, size=(W.shape[0], 1)))).astype(np.float16) for W in Ws]
    image, exact = B.mlp_testing_pack_device_on_host(Ws, bs, layout, widths=widths)
    assert exact, "a work item writes outside the image or over another item's bytes, or a byte stays unwritten"
    assert np.array_equal(image, B.mlp_pack_host(Ws, bs, layout, widths=widths))


@pytest.mark.skipif(_have_gpu(), reason="checks the error path taken when no GPU is visible")
def test_device_pack_without_a_device_reports_hip_error():
    with pytest.raises(B.MlpError) as e:
        B.mlp_pack_weights_device([0x10000], [0x20000], [4, 4])
    assert e.value.code == B.MLP_ERR_HIP


def test_infer_before_pack_and_bad_batch():
    B.mlp_release()
    B.mlp_release()  # idempotent
    assert _err(B.mlp_infer, 16, 0x1000, 0x2000) == B.MLP_ERR_NOT_PACKED
    assert _err(B.mlp_infer, -1, 0x1000, 0x2000) == B.MLP_ERR_INVALID_ARGUMENT
    assert _err(B.mlp_infer_ex, 16, 0x1000, 0x2000, None, 9) == B.MLP_ERR_INVALID_ARGUMENT
    assert _err(B.mlp_kernel_name, 0) == B.MLP_ERR_NOT_PACKED
    assert _err(B.mlp_debug_read_packed, 16) == B.MLP_ERR_NOT_PACKED


@pytest.mark.skipif(_have_gpu(), reason="checks the error path taken when no GPU is visible")
def test_pack_without_a_device_reports_hip_error():
    Ws, bs = workloads.init_weights([4, 4])
    with pytest.raises(B.MlpError) as e:
        B.mlp_pack_weights(Ws, bs)
    assert e.value.code == B.MLP_ERR_HIP
    assert "hip" in str(e.value).lower()


def test_plan_widths():
    # a 4-wide last layer on a dedicated FP16 kernel is computed 4 wide (16x16x32 MFMA)
    assert B.mlp_plan_widths(workloads.get("small").widths) == [16, 32, 32, 32, 32, 32, 32, 32, 4]
    assert B.mlp_plan_widths(workloads.get("page").widths) == [32] + [64] * 7 + [4]
    assert B.mlp_plan_widths(workloads.get("hetero").widths) == [32, 64, 64, 64, 128, 64, 64, 32, 4]
    assert B.mlp_plan_widths(workloads.get("stream").widths) == [64] * 8 + [32]
    assert B.mlp_plan_widths(workloads.get("page").widths, B.MLP_LAYOUT_PACKED_FP8) == [32] + [64] * 7 + [32]
    assert B.mlp_plan_widths([2, 2, 1]) == [64, 64, 64]  # generic kernel, zero-padded to 64
    assert B.mlp_plan_widths([2, 65, 1]) == [128, 128, 128]  # a width above 64: the 128-wide family
    assert B.mlp_plan_widths([100, 300, 129, 7]) == [128, 384, 256, 128]  # layer by layer
    assert B.mlp_plan_widths([16] * 10) == [64] * 10  # 9 narrow layers: the deep generic fused kernel
    assert B.mlp_plan_widths([16] * 17) == [64] * 17  # 16 narrow layers: still fused
    assert B.mlp_plan_widths([16] * 18) == [64] + [128] * 17  # 17 layers: layer by layer
    assert B.mlp_plan_widths([12] + [16] * 9) == [64] + [128] * 9  # input width not a multiple of 8
    assert B.mlp_plan_widths([16] * 9 + [65]) == [64] + [128] * 9  # 9 layers, output not a multiple of 4
    assert B.mlp_plan_widths([64] + [128] * 9 + [4]) == [128] * 11  # 10 layers up to 128 wide: fused
    assert B.mlp_plan_widths([64] * 17) == [64] * 17  # at most 64 wide: fused even where a chain serves


# ---- an independent reading of the layer-by-layer image ------------------------------------------
#
# Per layer: A fragments [MT][KB][lane][8] with MT = ceil(w_out / 128) * 4, KB = ceil(w_in / 64) * 4,
# lane = 32 g + m holding row 32 mt + m and input features 16 kb + 8 g + j (natural order); then the
# bias tiles [MT][g][16] FP32 with entry (mt, g, j) = b[32 mt + 8 (j // 4) + 4 g + j % 4].

def _unpack_layered(image, widths):
    off = 0
    Ws, bs = [], []
    for l in range(len(widths) - 1):
        MT = -(-widths[l + 1] // 128) * 4
        KB = -(-widths[l] // 64) * 4
        A = image[off:off + MT * KB * 1024].view(np.uint16).reshape(MT, KB, 2, 32, 8)
        off += MT * KB * 1024
        bias = image[off:off + MT * 128].view(np.float32).reshape(MT, 2, 16)
        off += MT * 128
        full = np.zeros((MT * 32, KB * 16), np.uint16)
        bfull = np.zeros(MT * 32, np.float32)
        for mt in range(MT):
            for g in range(2):
                for j in range(16):
                    bfull[32 * mt + 8 * (j // 4) + 4 * g + j % 4] = bias[mt, g, j]
                for kb in range(KB):
                    full[32 * mt:32 * mt + 32, 16 * kb + 8 * g:16 * kb + 8 * g + 8] = A[mt, kb, g]
        Ws.append(full)
        bs.append(bfull)
    assert off == image.size
    return Ws, bs


@pytest.mark.parametrize("widths", [(100, 300, 129, 7), (16,) * 18, (256, 32, 200)])
def test_layered_image_layout(widths):
    Ws, bs = workloads.init_weights(widths, seed=5)
    image = B.mlp_pack_host(Ws, bs, B.MLP_LAYOUT_PACKED)
    assert image.size == B.mlp_packed_size(widths)
    UW, Ub = _unpack_layered(image, widths)
    for l in range(len(widths) - 1):
        wout, win = Ws[l].shape
        assert np.array_equal(UW[l][:wout, :win], Ws[l].view(np.uint16)), l
        pad = UW[l].copy()
        pad[:wout, :win] = 0
        assert not pad.any(), "padding must be zero"
        assert np.array_equal(Ub[l][:wout], bs[l].astype(np.float32)), l
        assert not Ub[l][wout:].any()


# ---- an independent reading of the packed layout ---------------------------------------------
#
# Packed image, per layer: A fragments [mt][kb][lane][8] FP16 then bias tiles [mt][g][16] FP32, where
# lane = 32 g + m holds row 32 mt + m; slot j of block kb holds input feature
#   layer 0:  16 kb + 8 g + j
#   layer >0: 16 kb + 8 (j // 4) + 4 g + j % 4
# and the bias tile entry (mt, g, j) is b[32 mt + 8 (j // 4) + 4 g + j % 4].  Anything outside the real
# matrix is 0.  MT = ceil(w_out / 32) output tiles, KB = ceil(w_in / 16) input blocks.
#
# A last layer of at most 4 outputs (a 16x16x32 MFMA over both 16-sample halves of a 32-sample
# fragment) is laid out as [kb][lane][8]: lane = 16 a + i holds output i % 4 when i < 8 and
# i // 4 == a % 2 (else zeros), over the slots of group a // 2; its bias tile starts with
# b[0..3], b[0..3] (the C operand of lane groups a = 0 and 1) and is zero after.

def _unpack_narrow(A, bias, KB):
    full = np.zeros((4, KB * 16), np.uint16)
    seen = np.zeros((4, KB * 16), bool)
    for kb in range(KB):
        for lane in range(64):
            a, i = lane // 16, lane % 16
            g = a // 2
            for j in range(8):
                f = 16 * kb + 8 * (j // 4) + 4 * g + j % 4
                v = A[kb, lane, j]
                if i < 8 and i // 4 == a % 2:
                    r = i % 4
                    # the two sample halves must carry the same weight
                    assert not seen[r, f] or full[r, f] == v
                    full[r, f], seen[r, f] = v, True
                else:
                    assert v == 0, "lane %d of a narrow fragment must be zero" % lane
    assert seen.all()
    assert np.array_equal(bias[0:4], bias[4:8]) and not bias[8:].any()
    return full, bias[0:4].copy()


def _unpack(image, kw, widths):
    L = len(widths) - 1
    off = 0
    Ws, bs = [], []
    for l in range(L):
        MT = -(-kw[l + 1] // 32)
        KB = -(-kw[l] // 16)
        if l == L - 1 and kw[L] <= 4:
            A = image[off:off + KB * 1024].view(np.uint16).reshape(KB, 64, 8)
            off += KB * 1024
            bias = image[off:off + 128].view(np.float32)
            off += 128
            full, b4 = _unpack_narrow(A, bias, KB)
            Ws.append(full)
            bs.append(b4)
            continue
        A = image[off:off + MT * KB * 1024].view(np.uint16).reshape(MT, KB, 2, 32, 8)
        off += MT * KB * 1024
        bias = image[off:off + MT * 128].view(np.float32).reshape(MT, 2, 16)
        off += MT * 128
        full = np.zeros((MT * 32, KB * 16), np.uint16)
        bfull = np.zeros(MT * 32, np.float32)
        for mt in range(MT):
            for g in range(2):
                for j in range(16):
                    bfull[32 * mt + 8 * (j // 4) + 4 * g + j % 4] = bias[mt, g, j]
            for kb in range(KB):
                for g in range(2):
                    for j in range(8):
                        f = 16 * kb + 8 * g + j if l == 0 else 16 * kb + 8 * (j // 4) + 4 * g + j % 4
                        full[32 * mt:32 * mt + 32, f] = A[mt, kb, g, :, j]
        Ws.append(full)
        bs.append(bfull)
    assert off == image.size
    return Ws, bs


@pytest.mark.parametrize("name", list(workloads.WORKLOADS) + ["generic-5-7-3", "generic-100-30-7"])
def test_packed_image_layout(name):
    if name.startswith("generic"):
        widths = tuple(int(w) for w in name.split("-")[1:])
        Ws, bs = workloads.init_weights(widths, seed=3)
    else:
        widths = workloads.WORKLOADS[name].widths
        Ws, bs = workloads.init_weights(widths)
    kw = B.mlp_plan_widths(widths)
    image = B.mlp_pack_host(Ws, bs, B.MLP_LAYOUT_PACKED)
    assert image.size % 16 == 0
    assert image.size == B.mlp_packed_size(widths)
    UW, Ub = _unpack(image, kw, widths)
    for l in range(len(widths) - 1):
        wout, win = Ws[l].shape
        got = UW[l]
        assert np.array_equal(got[:wout, :win], Ws[l].view(np.uint16)), l
        pad = got.copy()
        pad[:wout, :win] = 0
        assert not pad.any(), "padding must be zero"
        assert np.array_equal(Ub[l][:wout], bs[l].astype(np.float32)), l  # exact widening
        assert not Ub[l][wout:].any()


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_row_major_image_is_verbatim(name):
    widths = workloads.WORKLOADS[name].widths
    Ws, bs = workloads.init_weights(widths)
    image = B.mlp_pack_host(Ws, bs, B.MLP_LAYOUT_ROW_MAJOR)
    off = 0
    for W, b in zip(Ws, bs):
        n = W.size * 2
        assert np.array_equal(image[off:off + n].view(np.uint16), W.view(np.uint16).ravel())
        off += -(-n // 16) * 16
        n = b.size * 2
        assert np.array_equal(image[off:off + n].view(np.uint16), b.view(np.uint16))
        off += -(-n // 16) * 16
    assert off == image.size


# ---- the FP8 image, read independently (E4M3 values via PyTorch's float8_e4m3fn) ------------------
#
# Per layer: A fragments [MT][KB][lane][32 bytes] (KB = ceil(w_in / 64)), lane = 32 g + m holding row
# 32 mt + m; slot j of block kb holds feature 64 kb + 32 g + j for layer 0 and
# 32 (2 kb + j // 16) + 8 ((j % 16) // 4) + 4 g + j % 4 after; then scale words
# [ceil(MT / 4)][lane][4 bytes] (byte i: E8M0 code of row 32 (4 q + i) + m); then FP32 bias tiles.

def _torch_e4m3_codes(x):
    import torch

    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_fp8_image_layout(name):
    widths = workloads.WORKLOADS[name].widths
    Ws, bs = workloads.init_weights(widths)
    image = B.mlp_pack_host(Ws, bs, B.MLP_LAYOUT_PACKED_FP8)
    assert image.size == B.mlp_packed_size(widths, B.MLP_LAYOUT_PACKED_FP8)
    off = 0
    for l in range(len(widths) - 1):
        win, wout = widths[l], widths[l + 1]
        MT, KB = -(-wout // 32), -(-win // 64)
        A = image[off:off + MT * KB * 2048].reshape(MT, KB, 2, 32, 32)
        off += MT * KB * 2048
        nq = -(-MT // 4)
        S = image[off:off + nq * 256].reshape(nq, 2, 32, 4)
        off += nq * 256
        bias = image[off:off + MT * 128].view(np.float32).reshape(MT, 2, 16)
        off += MT * 128
        W = Ws[l].astype(np.float64)
        for mt in range(MT):
            for m in range(32):
                r = 32 * mt + m
                code = int(S[mt // 4, 0, m, mt % 4])
                assert code == int(S[mt // 4, 1, m, mt % 4])  # both lane groups carry the row's scale
                if r >= wout:
                    assert code == 127 and not A[mt, :, :, m].any()
                    continue
                E = code - 127
                amax = np.abs(W[r]).max()
                assert amax == 0 or 224 < amax / 2.0 ** E <= 448, (l, r, E, amax)
                # every weight is the E4M3 code nearest to w / 2^E (PyTorch's float8_e4m3fn conversion)
                want = _torch_e4m3_codes((W[r] / 2.0 ** E).astype(np.float32))
                for kb in range(KB):
                    for g in range(2):
                        for j in range(32):
                            f = 64 * kb + 32 * g + j if l == 0 else 32 * (2 * kb + j // 16) + 8 * ((j % 16) // 4) + 4 * g + j % 4
                            got = int(A[mt, kb, g, m, j])
                            assert got == (int(want[f]) if f < win else 0), (l, r, f)
        for mt in range(MT):
            for g in range(2):
                for j in range(16):
                    r = 32 * mt + 8 * (j // 4) + 4 * g + j % 4
                    assert bias[mt, g, j] == (np.float32(bs[l][r]) if r < wout else 0.0)
    assert off == image.size


def test_fp8_is_for_the_dedicated_shapes():
    assert B.mlp_packed_size(workloads.get("page").widths, B.MLP_LAYOUT_PACKED_FP8) > 0
    assert _err(B.mlp_packed_size, [5, 7, 3], B.MLP_LAYOUT_PACKED_FP8) == B.MLP_ERR_UNSUPPORTED
    assert _err(B.mlp_packed_size, [4, 4], 3) == B.MLP_ERR_INVALID_ARGUMENT
