"""GPU parity: the HIP library, called through its C ABI, against the CPU oracle on the same inputs.

- order-free nets (every partial sum exact): bit for bit, on the generic and the dedicated kernels;
- random-weight workloads: the contract tolerance plus the internal bar, at sizes spanning several
  tiles with ragged tails, and at the workloads' full sizes on sampled rows;
- the two A/B variants of the page (row-major weights, scalarised activation) give the same bits as
  the production kernel ("Row-major versus InferencingOptimal weights": the layout "does not change
  the network"; "Bad versus good activation": the two forms compute the same function).
"""
import numpy as np
import pytest

from conftest import host_threads
from gpu_util import compare, log, run, to_device
from mlp_neural_shading_amd import binding as B
from mlp_neural_shading_amd import workloads

pytestmark = pytest.mark.gpu

DEDICATED = list(workloads.ALIASES)  # small, page, hetero, wide, stream
VARIANTS = [(B.MLP_LAYOUT_PACKED, B.MLP_ACT_VECTOR), (B.MLP_LAYOUT_PACKED, B.MLP_ACT_SCALARISED),
            (B.MLP_LAYOUT_ROW_MAJOR, B.MLP_ACT_VECTOR), (B.MLP_LAYOUT_ROW_MAJOR, B.MLP_ACT_SCALARISED)]
VNAME = {v: ("packed" if v[0] else "rowmajor") + "-" + ("scalarised" if v[1] else "vector") for v in VARIANTS}


def f16(a):
    return np.asarray(a, dtype=np.float64).astype(np.float16)


# ---- order-free nets: bit for bit -----------------------------------------------------------

def test_hand_worked_two_layer_net(oracle_mod):
    import json
    from pathlib import Path

    g = json.loads((Path(__file__).parent / "golden" / "hand_2layer.json").read_text())
    W = [f16(w) for w in g["weights"]]
    b = [f16(v) for v in g["biases"]]
    x = f16(g["x"]).view(np.uint16)
    log("hand-worked 2-layer net (generic kernel)")
    y = run(W, b, x)
    assert [hex(int(v)) for v in y.ravel()] == g["y_bits"][0]


def test_sign_alternating_diagonal_net():
    import json
    from pathlib import Path

    g = json.loads((Path(__file__).parent / "golden" / "sign_alternating_diag.json").read_text())
    W = [f16(d * np.eye(4)) for d in g["diag"]]
    b = [f16(np.zeros(4)) for _ in g["diag"]]
    x = f16(np.repeat(np.asarray(g["x"])[:, None], 4, axis=1)).view(np.uint16)
    y = run(W, b, x)
    want = np.array([int(h, 16) for h in g["y_bits"]], dtype=np.uint16)
    assert np.array_equal(y, np.repeat(want[:, None], 4, axis=1))


@pytest.mark.parametrize("seed,hi", [(s, 129) for s in range(8)] + [(s, 65) for s in range(8, 12)])
def test_integer_exact_nets_generic(oracle_mod, seed, hi):
    """Random non-square shapes (generic kernels; widths below `hi`, so the last seeds run the
    64-wide family): small non-negative integers, every intermediate <= 2048, so the GPU must equal
    the oracle and the int64 product bit for bit."""
    rng = np.random.default_rng(200 + seed)
    L = int(rng.integers(1, 9))
    widths = [int(w) for w in rng.integers(1, hi, size=L + 1)]
    W = [np.zeros((widths[l + 1], widths[l]), np.int64) for l in range(L)]
    for l in range(L):
        for r in range(widths[l + 1]):
            W[l][r, rng.integers(0, widths[l], size=2)] += 1  # <= 2 ones per row: values at most double
    b = [rng.integers(0, 2, size=widths[l + 1]) for l in range(L)]
    x = rng.integers(0, 4, size=(333, widths[0]))
    h = x.copy()
    for l in range(L):
        h = h @ W[l].T + b[l]
    assert h.max() <= 2048
    Wf, bf, xf = [f16(w) for w in W], [f16(v) for v in b], f16(x)
    log("integer-exact generic net widths", widths)
    y = run(Wf, bf, xf.view(np.uint16))
    assert np.array_equal(y, f16(h).view(np.uint16))
    assert np.array_equal(y, oracle_mod.mlp_forward(Wf, bf, xf))


def _permutation_chain(widths, rng, diag=(1, -64, -1, -64, -1, -64, -1, 1)):
    """W_l = d_l * (random partial permutation): every output is d_l times one input, so every
    binary32 sum is exact and the only roundings are the per-layer binary16 ones -- the result is
    unique, and it exercises the leaky slope on negative values through every layer."""
    L = len(widths) - 1
    Ws, bs = [], []
    for l in range(L):
        win, wout = widths[l], widths[l + 1]
        W = np.zeros((wout, win))
        src = rng.permutation(max(win, wout))
        for r in range(wout):
            if src[r] < win:
                W[r, src[r]] = diag[l % len(diag)]
        Ws.append(f16(W))
        bs.append(f16(np.zeros(wout)))
    return Ws, bs


GENERIC_SHAPES = {"generic": (24, 40, 16, 72, 8, 100, 12, 56, 6), "generic64": (24, 40, 16, 48, 8, 60, 12, 56, 6),
                  "generic64v": (24, 40, 16, 48, 8, 60, 12, 56, 8), "generic128v": (24, 40, 16, 72, 8, 100, 12, 56, 8)}


@pytest.mark.parametrize("name", DEDICATED + ["generic", "generic64", "generic64v", "generic128v"])
def test_permutation_chain_bit_exact(oracle_mod, name):
    rng = np.random.default_rng(31)
    widths = GENERIC_SHAPES[name] if name in GENERIC_SHAPES else workloads.get(name).widths
    Ws, bs = _permutation_chain(widths, rng)
    x = f16(rng.uniform(-1, 1, size=(1000 + 13, widths[0]))).view(np.uint16)
    ref = oracle_mod.mlp_forward(Ws, bs, x)
    variants = VARIANTS[:1] if name in GENERIC_SHAPES else VARIANTS
    for v in variants:
        log("permutation chain", name, VNAME[v])
        y = run(Ws, bs, x, *v)
        assert np.array_equal(y, ref), VNAME[v]


@pytest.mark.parametrize("name", DEDICATED)
def test_integer_exact_nets_dedicated(oracle_mod, name):
    rng = np.random.default_rng(41)
    widths = workloads.get(name).widths
    L = len(widths) - 1
    W = [np.zeros((widths[l + 1], widths[l]), np.int64) for l in range(L)]
    for l in range(L):
        for r in range(widths[l + 1]):
            W[l][r, rng.integers(0, widths[l], size=2)] += 1
    b = [rng.integers(0, 2, size=widths[l + 1]) for l in range(L)]
    x = rng.integers(0, 4, size=(2048 + 5, widths[0]))
    h = x.copy()
    for l in range(L):
        h = h @ W[l].T + b[l]
    assert h.max() <= 2048
    Wf, bf, xf = [f16(w) for w in W], [f16(v) for v in b], f16(x).view(np.uint16)
    want = f16(h).view(np.uint16)
    for v in VARIANTS:
        log("integer-exact", name, VNAME[v])
        assert np.array_equal(run(Wf, bf, xf, *v), want), VNAME[v]


def test_subnormal_results_bit_exact(oracle_mod):
    """Values that pass through the binary16 subnormal range (gradual underflow must not flush)."""
    widths = (16, 32, 32, 32, 32, 32, 32, 32, 4)
    rng = np.random.default_rng(5)
    Ws, bs = _permutation_chain(widths, rng, diag=(1, -1, 1, -1, 1, -1, 1, 1))
    x = f16(-rng.uniform(2.0**-12, 2.0**-4, size=(777, 16))).view(np.uint16)
    ref = oracle_mod.mlp_forward(Ws, bs, x)
    a = np.abs(ref.view(np.float16).astype(np.float64))
    assert ((a > 0) & (a < 2.0**-14)).any(), "the case must reach subnormals"
    for v in VARIANTS:
        assert np.array_equal(run(Ws, bs, x, *v), ref), VNAME[v]
    # the generic kernel too (a 9-wide first layer forces it)
    Wg = [f16(np.pad(Ws[0].astype(np.float64), ((0, 0), (0, 1))))] + Ws[1:]
    xg = np.pad(x, ((0, 0), (0, 1)))
    assert np.array_equal(run(Wg, bs, xg), oracle_mod.mlp_forward(Wg, bs, xg))


@pytest.mark.parametrize("widths,family", [
    (GENERIC_SHAPES["generic64"], "generic64"), (GENERIC_SHAPES["generic64v"], "generic64v"),
    (GENERIC_SHAPES["generic"], "generic128"), ((9, 64, 3), "generic64"), ((9, 65, 3), "generic128"),
    ((64,) * 9, "generic64v"), ((8, 64, 4), "generic64v"), ((48, 64, 64, 64, 64, 64, 8), "generic64v"),
    ((40, 64, 6), "generic64"), ((24, 40, 16, 72, 8, 100, 12, 56, 8), "generic128v"), ((64, 128, 4), "generic128v"),
    ((128,) * 9, "generic128v"), ((72, 96, 6), "generic128")])
def test_generic_families_random_weights(oracle_mod, widths, family):
    """A shape with no dedicated kernel runs on the first generic family that serves it (every width
    padded to 64, else to 128; each with vector I/O when the input width is a multiple of 8 and the
    output width a multiple of 4, else element by element); random weights against the oracle at a
    ragged batch."""
    rng = np.random.default_rng(len(widths) * 100 + widths[1])
    Ws, bs = workloads.init_weights(widths, seed=5)
    x = f16(rng.uniform(-1, 1, size=(4096 + 37, widths[0]))).view(np.uint16)
    y = run(Ws, bs, x)
    name = B.mlp_kernel_name(B.MLP_ACT_VECTOR)
    log("generic shape", widths, name)
    assert "<%s," % family in name, name
    compare(y, oracle_mod.mlp_forward(Ws, bs, x, threads=host_threads()), what=str(widths))


# ---- random-weight workloads at test sizes ---------------------------------------------------

@pytest.mark.parametrize("name", DEDICATED)
def test_random_weights_ragged_batches(oracle_mod, name):
    wl = workloads.get(name)
    Ws, bs = wl.weights()
    rows = 4096 + 37
    x = wl.inputs(device="cuda", rows=rows)
    xb = x.cpu().view(__import__("torch").int16).numpy().view(np.uint16)
    ref = oracle_mod.mlp_forward(Ws, bs, xb, threads=host_threads())
    first = None
    for v in VARIANTS:
        log("random weights", name, VNAME[v], "rows", rows)
        y = run(Ws, bs, x, *v)
        stats = compare(y, ref, what="%s %s" % (name, VNAME[v]))
        log("   ", stats)
        if first is None:
            first = y
        else:  # same MFMA order and the same roundings: identical bits
            assert np.array_equal(y, first), VNAME[v]
        for n in (1, 15, 17, 63, 65, 1000):
            yn = run(Ws, bs, x[:n], *v, pack=False)
            assert np.array_equal(yn, first[:n]), (VNAME[v], n)
