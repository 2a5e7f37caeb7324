"""GPU parity of the fused kernel on deep networks: 9 to 16 layers (input width a multiple of 8, output
width a multiple of 4) run as one fused dispatch when every width is at most 64 (all layers' weights
in LDS), and at widths up to 128 unless one 128-wide chain of the layer-by-layer path serves the
whole network; every layer the page's affine layer with the FP16 leaky ReLU between layers
("Profiling neural material inference", "Experiment setup" and "Bad versus good activation").
Against the CPU oracle through the C ABI:

- order-free nets (every partial sum exact): bit for bit, against int64 products and the oracle;
- permutation chains (the leaky slope on negative values through every layer): bit for bit;
- random weights N(0, 1/fan_in): the contract tolerance plus the internal bar, at ragged batches;
- the shapes just beyond the limits (17 layers; an input width that is not a multiple of 8) run
  layer by layer and agree as well.
"""
import numpy as np
import pytest

from conftest import host_threads
from gpu_util import compare, log, run
from mlp_neural_shading_amd import binding as B
from mlp_neural_shading_amd import workloads

pytestmark = pytest.mark.gpu


def f16(a):
    return np.asarray(a, dtype=np.float64).astype(np.float16)


def _x(rows, w, seed):
    rng = np.random.default_rng(seed)
    return f16(rng.uniform(-1, 1, size=(rows, w))).view(np.uint16)


def _widths(rng, L, hi):
    """L + 1 widths of at most hi: the input a multiple of 8, the output a multiple of 4."""
    w = [int(v) for v in rng.integers(1, hi + 1, size=L + 1)]
    w[0] = 8 * int(rng.integers(1, hi // 8 + 1))
    w[-1] = 4 * int(rng.integers(1, hi // 4 + 1))
    if hi > 64:
        w[L // 2] = int(rng.integers(65, hi + 1))  # one width above 64: the 128-wide family
        w[-1] = 4 * (2 * int(rng.integers(0, hi // 8)) + 1)  # not a multiple of 8: no whole-network chain
    return w


@pytest.mark.parametrize("L,hi", [(9, 64), (12, 64), (16, 64), (10, 128), (16, 128)])
def test_integer_exact_deep_nets(oracle_mod, L, hi):
    rng = np.random.default_rng(900 + L + hi)
    widths = _widths(rng, L, hi)
    W = [np.zeros((widths[l + 1], widths[l]), np.int64) for l in range(L)]
    for l in range(L):
        for r in range(widths[l + 1]):
            W[l][r, rng.integers(0, widths[l], size=2 if l == 0 else 1)] += 1
    b = [rng.integers(0, 2, size=widths[l + 1]) for l in range(L)]
    x = rng.integers(0, 4, size=(4133, widths[0]))
    h = x.copy()
    for l in range(L):
        h = h @ W[l].T + b[l]
    assert h.max() <= 2048
    Wf, bf, xf = [f16(w) for w in W], [f16(v) for v in b], f16(x)
    log("integer-exact deep fused net", widths)
    y = run(Wf, bf, xf.view(np.uint16))
    name = B.mlp_kernel_name(B.MLP_ACT_VECTOR)
    assert name == "mlp_fused<generic%dv,L=%d>" % (hi, L), name
    assert np.array_equal(y, f16(h).view(np.uint16))
    assert np.array_equal(y, oracle_mod.mlp_forward(Wf, bf, xf, threads=host_threads()))


@pytest.mark.parametrize("rows", [1013, 65536 * 2 + 77])
def test_permutation_chain_16_layers(oracle_mod, rows):
    widths = (32, 48, 64, 40, 64, 64, 8, 64, 56, 64, 64, 24, 64, 64, 64, 64, 12)
    diag = (1, -64, -1, -64, -1, -64, -1, 1)
    rng = np.random.default_rng(rows)
    Ws, bs = [], []
    for l in range(len(widths) - 1):
        win, wout = widths[l], widths[l + 1]
        W = np.zeros((wout, win))
        src = rng.permutation(max(win, wout))
        for r in range(wout):
            W[r, src[r] % win] = diag[l % len(diag)]
        Ws.append(f16(W))
        bs.append(f16(np.zeros(wout)))
    x = _x(rows, widths[0], rows + 1)
    log("permutation chain, 16 fused layers, rows", rows)
    y = run(Ws, bs, x)
    assert B.mlp_kernel_name(B.MLP_ACT_VECTOR) == "mlp_fused<generic64v,L=16>"
    assert np.array_equal(y, oracle_mod.mlp_forward(Ws, bs, x, threads=host_threads()))


@pytest.mark.parametrize("widths,family", [
    ((64,) * 10 + (16,), "generic64v"), ((32,) + (64,) * 15 + (4,), "generic64v"), ((16,) * 17, "generic64v"),
    ((64,) + (128,) * 9 + (4,), "generic128v"), ((96, 100, 128, 64, 120, 40, 64, 128, 72, 8), "generic128v"),
    ((128,) * 13 + (12,), "generic128v"),     # the output width keeps it off a whole-network chain
    ((128,) * 14, "layered"),                 # one 128-wide chain serves all 13 layers
    ((64,) * 17 + (16,), "layered"),          # 17 layers: one 64-wide chain
    ((60,) + (64,) * 10 + (16,), "layered"),  # input width not a multiple of 8
])
def test_random_weights(oracle_mod, widths, family):
    Ws, bs = workloads.init_weights(widths, seed=len(widths))
    x = _x(4096 + 37, widths[0], len(widths) + 3)
    y = run(Ws, bs, x)
    name = B.mlp_kernel_name(B.MLP_ACT_VECTOR)
    log("deep net", widths[:4], "layers", len(widths) - 1, name)
    assert name.startswith("mlp_layered" if family == "layered" else "mlp_fused<%s," % family), name
    stats = compare(y, oracle_mod.mlp_forward(Ws, bs, x, threads=host_threads()), what=str(widths))
    log("  max |d| %.3g, bit-identical %.4f" % (stats["max_abs"], stats["bit_identical_frac"]))
