"""GPU tests of the device-side weight conversion (mlp_pack_weights_device, the conversion run as a
kernel in the stream, "Row-major versus InferencingOptimal weights"): its image must equal the host
packer's bit for bit -- the host packer's own layout is pinned on the CPU by test_abi_host.py's
independent unpacker, and the kernel's per-item code is run on the CPU over every work item there
(extents and contents) before it runs here -- for every dedicated shape and layout (packed, row-major
and FP8) and for shapes served by the generic kernels, and it must be stream-ordered."""
import numpy as np
import pytest

from mlp_neural_shading_amd import binding as B
from mlp_neural_shading_amd import workloads

from gpu_util import device, log, run, to_device

pytestmark = pytest.mark.gpu

CASES = [(name, layout) for name in workloads.WORKLOADS
         for layout in (B.MLP_LAYOUT_PACKED, B.MLP_LAYOUT_ROW_MAJOR, B.MLP_LAYOUT_PACKED_FP8)]
GENERIC = [(5, 7, 3), (2, 2, 1), (128,) * 9, (1, 128, 1), (17, 33, 65, 100, 3),
           (32, 48, 64, 40, 64, 64, 8, 64, 56, 64, 64, 24, 64, 64, 64, 64, 12),  # 16 layers, fused
           (16,) * 21]  # 20 layers, layer by layer: two conversion launches


def _device_weights(Ws, bs):
    import torch

    dev = device()
    dW = [torch.from_numpy(np.ascontiguousarray(W).view(np.int16)).to(dev) for W in Ws]
    db = [torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to(dev) for b in bs]
    return dW, db


def _pack_both(widths, Ws, bs, layout):
    import torch

    host = B.mlp_pack_host(Ws, bs, layout, widths=widths)
    dW, db = _device_weights(Ws, bs)
    stream = torch.cuda.current_stream().cuda_stream
    B.mlp_pack_weights_device([t.data_ptr() for t in dW], [t.data_ptr() for t in db], widths, layout, stream)
    torch.cuda.synchronize()
    return host, B.mlp_debug_read_packed(host.size)


@pytest.mark.parametrize("name,layout", CASES)
def test_device_image_equals_host_image(name, layout):
    wl = workloads.WORKLOADS[name]
    Ws, bs = wl.weights()
    log("device pack", name, "layout", layout)
    host, got = _pack_both(list(wl.widths), Ws, bs, layout)
    assert got.dtype == np.uint8 and got.size == host.size
    assert np.array_equal(got, host)


@pytest.mark.parametrize("widths", GENERIC)
def test_device_image_generic_shapes(widths):
    Ws, bs = workloads.init_weights(widths, seed=11)
    log("device pack generic", widths)
    host, got = _pack_both(list(widths), Ws, bs, B.MLP_LAYOUT_PACKED)
    assert np.array_equal(got, host)


def test_inference_after_device_pack_is_stream_ordered():
    """Weights written, converted and used on one side stream with no host synchronisation in
    between give the same bits as the host-packed network."""
    import torch

    wl = workloads.get("page")
    Ws, bs = wl.weights()
    x = wl.inputs(device=device(), rows=4133)
    expect = run(Ws, bs, x)
    side = torch.cuda.Stream()
    dW = [torch.empty(W.shape, dtype=torch.int16, device=device()) for W in Ws]
    db = [torch.empty(b.shape, dtype=torch.int16, device=device()) for b in bs]
    host_W = [torch.from_numpy(np.ascontiguousarray(W).view(np.int16)).pin_memory() for W in Ws]
    host_b = [torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).pin_memory() for b in bs]
    out = torch.full((x.shape[0], wl.widths[-1]), float("nan"), dtype=torch.float16, device=device())
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for d, h in zip(dW + db, host_W + host_b):
            d.copy_(h, non_blocking=True)
        B.mlp_pack_weights_device([t.data_ptr() for t in dW], [t.data_ptr() for t in db], list(wl.widths),
                                  B.MLP_LAYOUT_PACKED, side.cuda_stream)
        B.mlp_infer(x.shape[0], x.data_ptr(), out.data_ptr(), side.cuda_stream)
    side.synchronize()
    got = out.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, expect)


@pytest.mark.parametrize("name", list(workloads.ALIASES))
def test_fp8_inference_after_device_pack(name):
    """FP8 weights converted on the device (row scales of several magnitudes) give the bits of the
    host-packed FP8 network."""
    import torch

    wl = workloads.get(name)
    Ws, bs = wl.weights()
    rng = np.random.default_rng(4)
    Ws = [(np.asarray(W, np.float64) * np.exp2(rng.integers(-3, 2, size=(W.shape[0], 1)))).astype(np.float16) for W in Ws]
    x = wl.inputs(device=device(), rows=2050)
    expect = run(Ws, bs, x, layout=B.MLP_LAYOUT_PACKED_FP8)
    dW, db = _device_weights(Ws, bs)
    B.mlp_pack_weights_device([t.data_ptr() for t in dW], [t.data_ptr() for t in db], list(wl.widths),
                              B.MLP_LAYOUT_PACKED_FP8, torch.cuda.current_stream().cuda_stream)
    log("FP8 inference after device pack", name)
    got = run(Ws, bs, x, layout=B.MLP_LAYOUT_PACKED_FP8, pack=False)
    assert np.array_equal(got, expect)


def test_repack_in_place_is_stream_ordered():
    """A device conversion of a network whose image has the size of the current one rewrites that image
    in place, in stream order: the inference enqueued before it on the same stream still computes the
    first network, the one after it the second, with no host synchronisation in between."""
    import torch

    wl = workloads.get("page")
    Ws1, bs1 = wl.weights()
    Ws2, bs2 = workloads.init_weights(list(wl.widths), seed=77)
    x = wl.inputs(device=device(), rows=4133)
    expect1, expect2 = run(Ws1, bs1, x), run(Ws2, bs2, x)
    assert not np.array_equal(expect1, expect2)
    dW1, db1 = _device_weights(Ws1, bs1)
    dW2, db2 = _device_weights(Ws2, bs2)
    stream = torch.cuda.current_stream().cuda_stream
    outs = [torch.full((x.shape[0], wl.widths[-1]), float("nan"), dtype=torch.float16, device=device())
            for _ in range(3)]
    log("in-place re-pack, page net, 3 conversions and inferences on one stream")
    for (dW, db), out in zip([(dW1, db1), (dW2, db2), (dW1, db1)], outs):
        B.mlp_pack_weights_device([t.data_ptr() for t in dW], [t.data_ptr() for t in db], list(wl.widths),
                                  B.MLP_LAYOUT_PACKED, stream)
        B.mlp_infer(x.shape[0], x.data_ptr(), out.data_ptr(), stream)
    torch.cuda.synchronize()
    got = [o.cpu().view(torch.int16).numpy().view(np.uint16) for o in outs]
    assert np.array_equal(got[0], expect1)
    assert np.array_equal(got[1], expect2)
    assert np.array_equal(got[2], expect1)
