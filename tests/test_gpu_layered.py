"""GPU parity of the layer-by-layer path (networks wider than 128, or deeper than 8 layers, or than 16
when every width is at most 64: one MFMA GEMM with the fused bias / rounding / leaky-ReLU epilogue per
layer, "Profiling neural material inference", "Experiment setup") against the CPU oracle, through
the C ABI.

- order-free nets (every partial sum exact): bit for bit against the oracle and int64 products;
- permutation chains (the leaky slope on negative values through every layer): bit for bit;
- random weights N(0, 1/fan_in): the contract tolerance plus the internal bar, over ragged row
  counts, odd widths (unaligned rows), more than one block of 65,536 rows, and 24 layers;
- the device-side conversion builds the same image; two streams running at once do not interfere.
"""
import numpy as np
import pytest

from conftest import host_threads
from gpu_util import compare, device, log, run, to_device
from mlp_neural_shading_amd import binding as B
from mlp_neural_shading_amd import workloads

pytestmark = pytest.mark.gpu


def f16(a):
    return np.asarray(a, dtype=np.float64).astype(np.float16)


def _x(rows, w, seed):
    rng = np.random.default_rng(seed)
    return f16(rng.uniform(-1, 1, size=(rows, w))).view(np.uint16)


@pytest.mark.parametrize("widths,rows", [
    ((64, 256, 256, 16), 4133),               # wider than 128
    ((48,) * 18, 3000),                        # 17 layers
    ((100, 300, 129, 7), 1000),                # odd widths: unaligned input and output rows
    ((1024, 1024, 8), 700),                    # K = 1024
    ((16, 4096, 4), 257),                      # the widest layer allowed
    ((24,) * 25, 513),                         # 24 layers
])
def test_random_nets(oracle_mod, widths, rows):
    Ws, bs = workloads.init_weights(widths, seed=len(widths) + rows)
    x = _x(rows, widths[0], rows)
    log("layered net", widths, "rows", rows)
    y = run(Ws, bs, x)
    ref = oracle_mod.mlp_forward(Ws, bs, x, threads=host_threads())
    stats = compare(y, ref, what=str(widths))
    log("  max |d| %.3g, bit-identical %.4f" % (stats["max_abs"], stats["bit_identical_frac"]))


def test_more_than_one_block_of_rows(oracle_mod):
    # a 4096-wide hidden layer keeps the pass at its minimum of 65,536 rows: two passes
    widths = (64, 4096, 8)
    rows = 65536 + 777
    Ws, bs = workloads.init_weights(widths, seed=9)
    x = _x(rows, widths[0], 4)
    log("layered net", widths, "rows", rows)
    y = run(Ws, bs, x)
    ref = oracle_mod.mlp_forward(Ws, bs, x, threads=host_threads())
    compare(y, ref, what="two row blocks")


@pytest.mark.parametrize("seed", range(4))
def test_integer_exact_nets(oracle_mod, seed):
    """Small non-negative integers with every intermediate <= 2048: unique results, bit for bit."""
    rng = np.random.default_rng(500 + seed)
    L = int(rng.integers(2, 12))
    widths = [int(w) for w in rng.integers(1, 400, size=L + 1)]
    widths[int(rng.integers(0, L + 1))] = int(rng.integers(129, 600))  # at least one wide layer
    W = [np.zeros((widths[l + 1], widths[l]), np.int64) for l in range(L)]
    for l in range(L):
        for r in range(widths[l + 1]):
            # two ones per row in the first layer, one afterwards: intermediates stay <= 8 + L
            W[l][r, rng.integers(0, widths[l], size=2 if l == 0 else 1)] += 1
    b = [rng.integers(0, 2, size=widths[l + 1]) for l in range(L)]
    x = rng.integers(0, 4, size=(517, widths[0]))
    h = x.copy()
    for l in range(L):
        h = h @ W[l].T + b[l]
    assert h.max() <= 2048
    Wf, bf, xf = [f16(w) for w in W], [f16(v) for v in b], f16(x)
    log("integer-exact layered net widths", widths)
    y = run(Wf, bf, xf.view(np.uint16))
    assert np.array_equal(y, f16(h).view(np.uint16))
    assert np.array_equal(y, oracle_mod.mlp_forward(Wf, bf, xf))


def test_permutation_chain_bit_exact(oracle_mod):
    rng = np.random.default_rng(77)
    widths = (200, 300, 150, 260, 140, 180, 300, 200, 170, 9)
    diag = (1, -64, -1, -64, -1, -64, -1, 1)
    Ws, bs = [], []
    for l in range(len(widths) - 1):
        win, wout = widths[l], widths[l + 1]
        W = np.zeros((wout, win))
        src = rng.permutation(max(win, wout))
        for r in range(wout):
            if src[r] < win:
                W[r, src[r]] = diag[l % len(diag)]
        Ws.append(f16(W))
        bs.append(f16(np.zeros(wout)))
    x = _x(1013, widths[0], 3)
    log("permutation chain (layered)", widths)
    assert np.array_equal(run(Ws, bs, x), oracle_mod.mlp_forward(Ws, bs, x))


def _signed_chain(widths, rng, diag=(1, -64, -1, -64, -1, -64, -1, 1)):
    Ws, bs = [], []
    for l in range(len(widths) - 1):
        win, wout = widths[l], widths[l + 1]
        W = np.zeros((wout, win))
        src = rng.permutation(max(win, wout))
        for r in range(wout):
            W[r, src[r] % win] = diag[l % len(diag)]
        Ws.append(f16(W))
        bs.append(f16(np.zeros(wout)))
    return Ws, bs


@pytest.mark.parametrize("rows", [517, 1000, 2048])
def test_large_tile_layers_bit_exact(oracle_mod, rows):
    """Layers whose padded output width is a multiple of 256 and whose input rows are whole 16-byte
    chunks (input width = its padding to 64) run on the 256 x 256 workgroup tile, K = 64 in its
    two-stage form: 64 -> 512 (K = 64), 512 -> 256, 256 -> 768, 768 -> 1024, 1024 -> 1000 (K of 32
    stages, split around the barrier; 1,024 padded outputs, 1,000 stored), then 1000 -> 16 on the
    128 x 256 tile.  Integer-exact nets (against int64 products) and a signed permutation chain
    (against the oracle), bit for bit, over partial row tiles."""
    widths = (64, 512, 256, 768, 1024, 1000, 16)
    rng = np.random.default_rng(rows)
    L = len(widths) - 1
    W = [np.zeros((widths[l + 1], widths[l]), np.int64) for l in range(L)]
    for l in range(L):
        for r in range(widths[l + 1]):
            W[l][r, rng.integers(0, widths[l], size=2 if l == 0 else 1)] += 1
    b = [rng.integers(0, 2, size=widths[l + 1]) for l in range(L)]
    x = rng.integers(0, 4, size=(rows, widths[0]))
    h = x.astype(np.float64)  # sums of small integers: exact in float64, and BLAS-fast
    for l in range(L):
        h = h @ W[l].T.astype(np.float64) + b[l]
    assert h.max() <= 2048
    Wf, bf, xf = [f16(w) for w in W], [f16(v) for v in b], f16(x).view(np.uint16)
    log("integer-exact large-tile net", widths, "rows", rows)
    assert np.array_equal(run(Wf, bf, xf), f16(h).view(np.uint16))
    Ws, bs = _signed_chain(widths, rng)
    xs = _x(rows, widths[0], rows + 1)
    log("signed permutation chain, large tile", widths, "rows", rows)
    assert np.array_equal(run(Ws, bs, xs), oracle_mod.mlp_forward(Ws, bs, xs))


@pytest.mark.parametrize("rows", [700, 131849])
def test_full_width_tiles_bit_exact(oracle_mod, rows):
    """Layers on the 256 x 256 tile that store every padded output write their rows with range-checked
    buffer stores, the rows past the batch falling outside the tile's range.  K depths of two, four,
    six, eight and 32 stages (64, 128, 192, 256, 1024); 131,849 rows give up to 2,064 tiles and a
    9-row last tile, 700 rows a 188-row one.  The 256 -> 192 layer (256 padded outputs, 192 stored)
    takes the checked store path and 256 -> 128 and 512 -> 16 the 128 x 256 tile in between.
    Integer-exact nets against float64 sums of small integers, and a signed permutation chain against
    the oracle, bit for bit."""
    widths = (64, 256, 1024, 256, 192, 256, 128, 512, 16)
    rng = np.random.default_rng(rows)
    L = len(widths) - 1
    W = [np.zeros((widths[l + 1], widths[l])) for l in range(L)]
    for l in range(L):
        for r in range(widths[l + 1]):
            W[l][r, rng.integers(0, widths[l], size=2 if l == 0 else 1)] += 1
    b = [rng.integers(0, 2, size=widths[l + 1]).astype(np.float64) for l in range(L)]
    x = rng.integers(0, 4, size=(rows, widths[0])).astype(np.float64)
    h = x
    for l in range(L):
        h = h @ W[l].T + b[l]
    assert h.max() <= 2048
    Wf, bf, xf = [f16(w) for w in W], [f16(v) for v in b], f16(x).view(np.uint16)
    log("integer-exact full-width net", widths, "rows", rows)
    assert np.array_equal(run(Wf, bf, xf), f16(h).view(np.uint16))
    Ws, bs = _signed_chain(widths, rng)
    xs = _x(rows, widths[0], rows + 1)
    log("signed permutation chain, full-width tiles", widths, "rows", rows)
    assert np.array_equal(run(Ws, bs, xs), oracle_mod.mlp_forward(Ws, bs, xs, threads=host_threads()))


@pytest.mark.parametrize("widths", [(128, 256, 256, 200, 256, 256), (64, 256, 256, 256, 100), (256,) * 17,
                                    (64,) * 17 + (16,), (128,) * 13 + (16,),
                                    (100, 100, 128, 64, 120, 40, 64, 128, 72, 8), (128, 128, 128, 72, 300, 16)])
@pytest.mark.parametrize("rows", [517, 131849])
def test_chained_layers_bit_exact(oracle_mod, widths, rows):
    """Consecutive layers of one padded output width (256 with K of 128..256, or 128 with K of 64 or
    128) run as one chain, the row tile's activations kept in LDS: a whole net ending in a 256-wide
    chain (K of 128, a 200-wide layer whose padded outputs must be exact zeros for the next K, no
    activation after the last layer), a chain between single layers (its last layer activated), 16
    layers of 256; narrow deep nets as 128-wide chains (17 layers of 64 then 16 outputs, K of 64 in two
    stages; 13 layers of 128; two single layers, then a chain over padded widths 120, 40 and 72 ending
    in 8 outputs; a chain that stores 72 of its 128 outputs for a single layer to read with K padded
    to 128).  Integer-exact nets against float64 sums of small integers, and a signed
    permutation chain against the oracle, bit for bit, over a ragged last tile and many tiles."""
    rng = np.random.default_rng(rows + len(widths))
    L = len(widths) - 1
    W = [np.zeros((widths[l + 1], widths[l])) for l in range(L)]
    for l in range(L):
        for r in range(widths[l + 1]):
            W[l][r, rng.integers(0, widths[l], size=2 if l == 0 else 1)] += 1
    b = [rng.integers(0, 2, size=widths[l + 1]).astype(np.float64) for l in range(L)]
    x = rng.integers(0, 4, size=(rows, widths[0])).astype(np.float64)
    h = x
    for l in range(L):
        h = h @ W[l].T + b[l]
    assert h.max() <= 2048
    Wf, bf, xf = [f16(w) for w in W], [f16(v) for v in b], f16(x).view(np.uint16)
    log("integer-exact chained net", widths[:6], "layers", L, "rows", rows)
    assert np.array_equal(run(Wf, bf, xf), f16(h).view(np.uint16))
    Ws, bs = _signed_chain(widths, rng)
    xs = _x(rows, widths[0], rows + 2)
    log("signed permutation chain, chained layers", widths[:6], "rows", rows)
    assert np.array_equal(run(Ws, bs, xs), oracle_mod.mlp_forward(Ws, bs, xs, threads=host_threads()))


@pytest.mark.parametrize("widths", [(60,) + (64,) * 9 + (12,), (124,) + (128,) * 9 + (60,), (250,) + (256,) * 4 + (100,)])
@pytest.mark.parametrize("rows", [1029, 70001])
def test_chains_between_unaligned_rows(oracle_mod, widths, rows):
    """Chains read and write whole 16-byte rows of exactly their K columns: an input width below its
    padding to 64 (rows of 120, 248 or 500 bytes) puts the first layer on a single GEMM launch, an
    output width that is not a multiple of 8 the last, and the layers between stay one chain (64, 128
    and 256 wide).  A signed permutation chain against the oracle, bit for bit."""
    rng = np.random.default_rng(rows + widths[0])
    Ws, bs = _signed_chain(widths, rng)
    x = _x(rows, widths[0], rows + 5)
    log("chain between unaligned rows", widths[:3], "layers", len(widths) - 1, "rows", rows)
    assert np.array_equal(run(Ws, bs, x), oracle_mod.mlp_forward(Ws, bs, x, threads=host_threads()))


def test_large_tile_random_net(oracle_mod):
    widths = (64, 1024, 1024, 1000, 16)
    Ws, bs = workloads.init_weights(widths, seed=21)
    x = _x(1333, widths[0], 21)
    log("large-tile random net", widths)
    y = run(Ws, bs, x)
    ref = oracle_mod.mlp_forward(Ws, bs, x, threads=host_threads())
    stats = compare(y, ref, what=str(widths))
    log("  max |d| %.3g, bit-identical %.4f" % (stats["max_abs"], stats["bit_identical_frac"]))


def test_device_conversion_of_a_layered_net():
    import torch

    widths = (100, 300, 129, 7) + (40,) * 7  # 10 layers: two launches of the conversion kernel
    Ws, bs = workloads.init_weights(widths, seed=2)
    host = B.mlp_pack_host(Ws, bs)
    dev = device()
    dW = [torch.from_numpy(np.ascontiguousarray(W).view(np.int16)).to(dev) for W in Ws]
    db = [torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to(dev) for b in bs]
    B.mlp_pack_weights_device([t.data_ptr() for t in dW], [t.data_ptr() for t in db], list(widths))
    torch.cuda.synchronize()
    assert np.array_equal(B.mlp_debug_read_packed(host.size), host)


def test_two_streams_at_once(oracle_mod):
    """Each call takes its scratch on its own stream: two streams running the network at once give
    the bits of one stream alone."""
    import torch

    widths = (96, 512, 512, 24)
    Ws, bs = workloads.init_weights(widths, seed=12)
    x = _x(20000, widths[0], 8)
    expect = run(Ws, bs, x)
    dev = device()
    xt = to_device(x)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[torch.full((x.shape[0], widths[-1]), float("nan"), dtype=torch.float16, device=dev) for _ in range(3)]
            for _ in streams]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for k in range(3):
        for s, o in zip(streams, outs):
            B.mlp_infer(x.shape[0], xt.data_ptr(), o[k].data_ptr(), s.cuda_stream)
    torch.cuda.synchronize()
    for o in outs:
        for t in o:
            assert np.array_equal(t.cpu().view(torch.int16).numpy().view(np.uint16), expect)
