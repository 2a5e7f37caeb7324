"""mlp_infer_noalloc (the entry point that allocates nothing) against mlp_infer, through the C ABI.

The layer-by-layer path is the one that needs scratch memory: mlp_infer takes its two activation
buffers from a stream-ordered pool, mlp_infer_noalloc from a fixed 64 MiB array per GPU, in smaller
row blocks.  Rows are independent and both run the same kernels, so the outputs must be bit-identical.
Two calls in a row, the second on a smaller input (the array then holds the first call's contents),
plus a fused network (no scratch: the same kernel as mlp_infer)."""
import numpy as np
import pytest

from gpu_util import log
from mlp_neural_shading_amd import binding as B
from mlp_neural_shading_amd import workloads

pytestmark = pytest.mark.gpu


def _both(x, wL):
    import torch

    stream = torch.cuda.current_stream().cuda_stream
    y_ref = torch.full((x.shape[0], wL), float("nan"), dtype=torch.float16, device=x.device)
    y_na = torch.full((x.shape[0], wL), float("nan"), dtype=torch.float16, device=x.device)
    B.mlp_infer(x.shape[0], x.data_ptr(), y_ref.data_ptr(), stream)
    B.mlp_infer_noalloc(x.shape[0], x.data_ptr(), y_na.data_ptr(), stream)
    torch.cuda.synchronize()
    a = y_ref.cpu().view(torch.int16).numpy()
    b = y_na.cpu().view(torch.int16).numpy()
    assert np.isfinite(y_ref.cpu().float().numpy()).all()
    return a, b


def test_noalloc_matches_mlp_infer_layered():
    """Widest hidden layer 4096 (padded): the 64 MiB array holds 4,096-row blocks, so 10,000 rows take
    three blocks where mlp_infer takes one; then 2,500 rows (one partial block)."""
    import torch

    widths = (48, 4096, 1000, 10)
    Ws, bs = workloads.init_weights(widths, seed=11)
    B.mlp_pack_weights(Ws, bs, B.MLP_LAYOUT_PACKED)
    assert B.mlp_kernel_name().startswith("mlp_layered")
    for rows in (10000, 2500):
        x = workloads.input_block(rows, widths[0], seed=rows, device="cuda")
        log("no-alloc layered", widths, "rows", rows)
        a, b = _both(x, widths[-1])
        assert np.array_equal(a, b), rows


def test_noalloc_matches_mlp_infer_layered_deep():
    """Seventeen 256-wide layers (the blocks hold 65,536 rows): one call over 70,001 rows (two blocks),
    then 777 rows."""
    widths = (256,) * 17
    Ws, bs = workloads.init_weights(widths, seed=12)
    B.mlp_pack_weights(Ws, bs, B.MLP_LAYOUT_PACKED)
    for rows in (70001, 777):
        x = workloads.input_block(rows, widths[0], seed=rows, device="cuda")
        log("no-alloc deep", "rows", rows)
        a, b = _both(x, widths[-1])
        assert np.array_equal(a, b), rows


def test_noalloc_matches_mlp_infer_fused():
    wl = workloads.get("page")
    Ws, bs = wl.weights()
    B.mlp_pack_weights(Ws, bs, B.MLP_LAYOUT_PACKED)
    for rows in (5000, 333):
        x = wl.inputs(device="cuda", rows=rows)
        log("no-alloc fused page", "rows", rows)
        a, b = _both(x, wl.widths[-1])
        assert np.array_equal(a, b), rows


def test_noalloc_does_not_allocate_in_steady_state():
    """After the first call (which looks up the array's address), further calls leave the device's
    free memory unchanged, where mlp_infer's pool would hold two blocks of activations."""
    import torch

    widths = (64, 2048, 2048, 16)
    Ws, bs = workloads.init_weights(widths, seed=13)
    B.mlp_release()  # returns the pool's cached blocks
    B.mlp_pack_weights(Ws, bs, B.MLP_LAYOUT_PACKED)
    x = workloads.input_block(20000, widths[0], seed=5, device="cuda")
    y = torch.empty((20000, widths[-1]), dtype=torch.float16, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    B.mlp_infer_noalloc(20000, x.data_ptr(), y.data_ptr(), stream)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for _ in range(3):
        B.mlp_infer_noalloc(20000, x.data_ptr(), y.data_ptr(), stream)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    log("free memory before/after three no-alloc calls:", free0, free1)
    assert free1 >= free0 - (2 << 20)  # two blocks of activations would be 2 x 20,000 x 2,048 x 2 = 164 MB
