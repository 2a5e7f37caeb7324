"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark times, on rows
the oracle can compute one by one; plus properties that hold at any size (all outputs finite,
replicated inputs give identical outputs, results do not depend on the batch)."""
import numpy as np
import pytest

from conftest import host_threads
from gpu_util import compare, log
from mlp_neural_shading_amd import binding as B
from mlp_neural_shading_amd import workloads

pytestmark = pytest.mark.gpu


def _run_full(wl, act=B.MLP_ACT_VECTOR, layout=B.MLP_LAYOUT_PACKED):
    import torch

    Ws, bs = wl.weights()
    x = wl.inputs(device="cuda")
    y = torch.empty((wl.batch, wl.widths[-1]), dtype=torch.float16, device="cuda")
    B.mlp_pack_weights(Ws, bs, layout)
    B.mlp_infer_ex(wl.batch, x.data_ptr(), y.data_ptr(), torch.cuda.current_stream().cuda_stream, act)
    torch.cuda.synchronize()
    return Ws, bs, x, y


def _rows_bits(t, idx):
    import torch

    sel = t.index_select(0, torch.as_tensor(idx, device=t.device))
    return sel.cpu().view(torch.int16).numpy().view(np.uint16)


def _sample(wl, n_random, edge, extra=()):
    rng = np.random.default_rng(77)
    idx = np.concatenate([np.arange(edge), np.arange(wl.batch - edge, wl.batch),
                          rng.integers(0, wl.batch, size=n_random), np.asarray(extra, dtype=np.int64)])
    return np.unique(idx[(idx >= 0) & (idx < wl.batch)])


def test_page_workload_full(oracle_mod):
    """1,048,576 evals = 65,536 inputs x 16: every unique row against the oracle, every replica
    bit-identical to the first (each evaluation is independent and deterministic)."""
    import torch

    wl = workloads.get("page")
    log("full", wl.name)
    Ws, bs, x, y = _run_full(wl)
    assert bool(torch.isfinite(y).all())
    u = wl.unique_rows
    first = y[:u]
    for r in range(1, wl.replicas):
        assert torch.equal(y[r * u:(r + 1) * u], first), "replica %d differs" % r
    xb = x[:u].cpu().view(torch.int16).numpy().view(np.uint16)
    ref = oracle_mod.mlp_forward(Ws, bs, xb, threads=host_threads())
    stats = compare(first.cpu().view(torch.int16).numpy().view(np.uint16), ref, what=wl.name)
    log("   ", stats)
    # the other three variants on the full dispatch give the same bits
    for layout, act in [(B.MLP_LAYOUT_PACKED, B.MLP_ACT_SCALARISED), (B.MLP_LAYOUT_ROW_MAJOR, B.MLP_ACT_VECTOR)]:
        _, _, _, y2 = _run_full(wl, act=act, layout=layout)
        assert torch.equal(y2, y), (layout, act)


# small and hetero: every row (4,096 and 1,048,576); wide (4,194,304 rows of 107,008 MACs): the first
# and last 65,536 rows and 1,048,576 seeded random rows (~1.2 M rows of the oracle, about a minute and a
# half on a 16-core host; the whole batch would take over five minutes).
@pytest.mark.parametrize("name,n_random,edge", [("small", 0, 4096), ("hetero", 0, 524288), ("wide", 1048576, 65536)])
def test_full_size_sampled(oracle_mod, name, n_random, edge):
    import torch

    wl = workloads.get(name)
    log("full", wl.name)
    Ws, bs, x, y = _run_full(wl)
    assert bool(torch.isfinite(y).all())
    idx = _sample(wl, n_random, edge)
    ref = oracle_mod.mlp_forward_rows(Ws, bs, _rows_bits(x, idx), np.arange(idx.size), threads=host_threads())
    log("   ", compare(_rows_bits(y, idx), ref, what=wl.name), "rows checked", idx.size)


# The layer-by-layer networks at the sizes the benchmark times (one block of rows each; a GEMM launch
# per layer, or one launch per chain of layers): the first and last row tiles and seeded random rows
# against the oracle (the 1024-wide net costs ~6.4 M multiply-adds per row on the host, the 256-wide
# one ~1 M, the deep narrow ones 0.07 M and 0.2 M).
@pytest.mark.parametrize("name,n_random,edge", [("layered1024", 1024, 256), ("layered256", 4096, 1024),
                                                ("layered64deep", 65536, 4096), ("layered128deep", 16384, 4096),
                                                ("deep64fused", 65536, 4096)])
def test_layered_workload_full_size_sampled(oracle_mod, name, n_random, edge):
    import torch

    wl = workloads.get(name)
    log("full", wl.name, B.mlp_plan_widths(wl.widths))
    Ws, bs, x, y = _run_full(wl)
    assert bool(torch.isfinite(y).all())
    idx = _sample(wl, n_random, edge)
    ref = oracle_mod.mlp_forward_rows(Ws, bs, _rows_bits(x, idx), np.arange(idx.size), threads=host_threads())
    log("   ", compare(_rows_bits(y, idx), ref, what=wl.name), "rows checked", idx.size)


def test_streaming_workload_full(oracle_mod):
    """67,108,864 distinct inputs (8 GiB in, 2 GiB out): the first and last 65,536 rows, the rows whose
    input bytes straddle each 2 GiB boundary (64-bit addressing) and 1,048,576 seeded random rows."""
    import torch

    wl = workloads.get("stream")
    log("full", wl.name, "(8 GiB of input)")
    Ws, bs, x, y = _run_full(wl)
    assert bool(torch.isfinite(y).all())
    row_bytes = 2 * wl.widths[0]
    edges = []
    for k in (1, 2, 3):
        r = (k << 31) // row_bytes
        edges += list(range(r - 64, r + 64))
    idx = _sample(wl, 1048576, 65536, extra=edges)  # first / last 65,536 rows, 2 GiB edges, random rows
    ref = oracle_mod.mlp_forward_rows(Ws, bs, _rows_bits(x, idx), np.arange(idx.size), threads=host_threads())
    log("   ", compare(_rows_bits(y, idx), ref, what=wl.name), "rows checked", idx.size)
    del x, y
    torch.cuda.empty_cache()


def test_batch_independence_and_determinism():
    """Row r's output depends only on input row r: any batch prefix and any repeat give the same
    bits (the grid size changes with the batch)."""
    import torch

    wl = workloads.get("hetero")
    Ws, bs = wl.weights()
    x = wl.inputs(device="cuda", rows=200003)
    B.mlp_pack_weights(Ws, bs)
    s = torch.cuda.current_stream().cuda_stream
    full = torch.empty((x.shape[0], wl.widths[-1]), dtype=torch.float16, device="cuda")
    B.mlp_infer(x.shape[0], x.data_ptr(), full.data_ptr(), s)
    again = torch.empty_like(full)
    B.mlp_infer(x.shape[0], x.data_ptr(), again.data_ptr(), s)
    torch.cuda.synchronize()
    assert torch.equal(full, again)
    for n in (1, 64, 1000, 65537, 131072):
        part = torch.full((n, wl.widths[-1]), float("nan"), dtype=torch.float16, device="cuda")
        B.mlp_infer(n, x.data_ptr(), part.data_ptr(), s)
        torch.cuda.synchronize()
        assert torch.equal(part, full[:n]), n
    # an offset start (rows 1000..) is the same computation on the same rows
    off = 1024
    part = torch.empty((5000, wl.widths[-1]), dtype=torch.float16, device="cuda")
    B.mlp_infer(5000, x[off:].data_ptr(), part.data_ptr(), s)
    torch.cuda.synchronize()
    assert torch.equal(part, full[off:off + 5000])


def test_boundary_errors_on_device():
    import torch

    wl = workloads.get("small")
    Ws, bs = wl.weights()
    B.mlp_pack_weights(Ws, bs)
    x = wl.inputs(device="cuda", rows=64)
    y = torch.empty((64, 4), dtype=torch.float16, device="cuda")
    B.mlp_infer(0, x.data_ptr(), y.data_ptr())  # batch 0: nothing launched
    with pytest.raises(B.MlpError) as e:
        B.mlp_infer(63, x.data_ptr() + 2, y.data_ptr())
    assert e.value.code == B.MLP_ERR_INVALID_ARGUMENT and "aligned" in str(e.value)
    with pytest.raises(B.MlpError) as e:
        B.mlp_infer(64, x.data_ptr(), x.data_ptr() + 16)
    assert e.value.code == B.MLP_ERR_INVALID_ARGUMENT and "overlap" in str(e.value)
    # the device image round-trips to the host image
    n = B.mlp_packed_size(wl.widths)
    assert np.array_equal(B.mlp_debug_read_packed(n), B.mlp_pack_host(Ws, bs))
    assert "16-32x7-4" in B.mlp_kernel_name(B.MLP_ACT_VECTOR)
    # a generic-shape net has no scalarised kernel
    Wg, bg = workloads.init_weights((5, 7, 3))
    B.mlp_pack_weights(Wg, bg)
    with pytest.raises(B.MlpError) as e:
        B.mlp_infer_ex(4, x.data_ptr(), y.data_ptr(), None, B.MLP_ACT_SCALARISED)
    assert e.value.code == B.MLP_ERR_UNSUPPORTED
    B.mlp_release()
    with pytest.raises(B.MlpError) as e:
        B.mlp_infer(4, x.data_ptr(), y.data_ptr())
    assert e.value.code == B.MLP_ERR_NOT_PACKED


# Every kernel family evaluates a small or ragged batch exactly as it evaluates the same rows inside a
# larger one: the tails (rows past the batch, masked loads and stores) must not change a bit.
@pytest.mark.parametrize("widths", [
    (64, 64, 64, 64, 64, 64, 64, 64, 16),   # dedicated (streaming shape)
    (24, 40, 16, 48, 8, 60, 12, 56, 6),     # generic, 64-wide, element by element
    (24, 40, 16, 48, 8, 60, 12, 56, 8),     # generic, 64-wide, vector I/O
    (9, 65, 3),                             # generic, 128-wide, element by element
    (24, 40, 16, 72, 8, 100, 12, 56, 8),    # generic, 128-wide, vector I/O
    (64, 256, 256, 16),                     # layer by layer
    (48,) * 18,                             # layer by layer, unaligned K (a 64-wide chain)
    (48,) * 13,                             # generic, 64-wide, 12 layers
])
def test_batch_prefix_invariance_every_family(widths):
    import torch

    Ws, bs = workloads.init_weights(widths, seed=21)
    rng = np.random.default_rng(22)
    big = 4096 + 77
    x = torch.from_numpy(rng.uniform(-1, 1, size=(big, widths[0])).astype(np.float16)).to("cuda")
    B.mlp_pack_weights(Ws, bs)
    log("prefix invariance", widths, B.mlp_kernel_name(B.MLP_ACT_VECTOR))
    s = torch.cuda.current_stream().cuda_stream
    full = torch.empty((big, widths[-1]), dtype=torch.float16, device="cuda")
    B.mlp_infer(big, x.data_ptr(), full.data_ptr(), s)
    for n in (1, 2, 31, 33, 63, 65, 257, 1000):
        part = torch.full((n, widths[-1]), float("nan"), dtype=torch.float16, device="cuda")
        B.mlp_infer(n, x.data_ptr(), part.data_ptr(), s)
        torch.cuda.synchronize()
        assert torch.equal(part, full[:n]), (widths, n)
