"""Pins that tie the oracle's network evaluation to facts outside itself.

Each pin is chosen so that a plausible mistake in the oracle fails at least one of them:

- hand-worked two-layer net (golden fixture): catches a transposed weight operand, a dropped bias,
  a wrong slope, and a missing rounding (see ``golden/hand_2layer.json``);
- sign-alternating diagonal net (golden fixture): catches ReLU-for-leaky, an activation after the
  output layer, a missing FP16 rounding between layers, and a wrong slope constant;
- identity passthrough and all-positive affine nets: the layer plumbing and indexing against closed
  forms computed in float64;
- integer-exact nets: every value and partial sum is an exact small integer, so the oracle must
  equal an int64 brute force bit for bit, whatever the shapes (non-square layers catch index and
  orientation mistakes);
- zero nets and the padded output row: bias routing;
- positive homogeneity with zero biases.

The network is the eight-affine-layer FP16 MLP of "Profiling neural material inference"
("Experiment setup"); the activation is the vector leaky ReLU of "Bad versus good activation".
"""
import json
from pathlib import Path

import numpy as np
import pytest

GOLDEN = Path(__file__).resolve().parent / "golden"
SLOPE = 0.01000213623046875  # half(0.01)


def f16(a):
    return np.asarray(a, dtype=np.float64).astype(np.float16)


def bits(a):
    return np.asarray(a, dtype=np.float16).view(np.uint16)


def test_hand_worked_two_layer_net(oracle_mod):
    g = json.loads((GOLDEN / "hand_2layer.json").read_text())
    W = [f16(w) for w in g["weights"]]
    b = [f16(v) for v in g["biases"]]
    x = f16(g["x"])
    y = oracle_mod.mlp_forward(W, b, x)
    assert [hex(int(v)) for v in y.ravel()] == g["y_bits"][0]
    # the hidden layer alone (one-layer net: no activation) then the oracle's leaky
    h = oracle_mod.mlp_forward(W[:1], b[:1], x)
    h = oracle_mod.leaky_f16_bits(h)
    assert [hex(int(v)) for v in h.ravel()] == g["hidden_bits"][0]


def test_sign_alternating_diagonal_net(oracle_mod):
    g = json.loads((GOLDEN / "sign_alternating_diag.json").read_text())
    W = [f16(d * np.eye(4)) for d in g["diag"]]
    b = [f16(np.zeros(4)) for _ in g["diag"]]
    x = f16(np.repeat(np.asarray(g["x"])[:, None], 4, axis=1))
    y = oracle_mod.mlp_forward(W, b, x)
    want = np.array([int(h, 16) for h in g["y_bits"]], dtype=np.uint16)
    assert np.array_equal(y, np.repeat(want[:, None], 4, axis=1))
    assert np.allclose(y.view(np.float16)[:, 0].astype(np.float64), g["y_values"], rtol=0, atol=0)


@pytest.mark.parametrize("width", [4, 32])
def test_identity_passthrough(oracle_mod, width):
    """W = I, b = 0 at every layer: x >= 0 passes through bit-exactly; x < 0 leaves seven
    successive single roundings of x * half(0.01) (seven hidden activations, none after layer 8).
    A zero result is +0: the binary32 sum starts from the +0 bias, and +0 + (-0) = +0."""
    rng = np.random.default_rng(11)
    W = [f16(np.eye(width)) for _ in range(8)]
    b = [f16(np.zeros(width)) for _ in range(8)]
    x = f16(rng.uniform(-4, 4, size=(257, width)))
    x[0, :] = 0.0
    x[1, 0] = -0.0
    y = oracle_mod.mlp_forward(W, b, x)
    ref = x.astype(np.float64)
    for _ in range(7):
        ref = np.where(ref < 0, (ref * SLOPE).astype(np.float16).astype(np.float64), ref)
        ref = np.where(ref == 0, 0.0, ref)
    assert np.array_equal(y, bits(ref))


def _forward_bound(widths, n_layers):
    # Non-negative data: each layer adds at most (w_in + 1) binary32 roundings (relative u32) and one
    # binary16 rounding (relative u16) to a sum of non-negative terms, so relative errors compound as
    # prod_l (1 + u16) * (1 + u32)^(w_in + 1) - 1.
    u16, u32 = 2.0**-11, 2.0**-24
    rel = 1.0
    for l in range(n_layers):
        rel *= (1 + u16) * (1 + u32) ** (widths[l] + 1)
    return rel - 1.0


@pytest.mark.parametrize("widths", [(16, 32, 32, 32, 32, 32, 32, 32, 4),
                                    (32, 64, 64, 64, 128, 64, 64, 32, 4),
                                    (5, 7, 3, 9)])
def test_all_positive_net_is_one_affine_map(oracle_mod, widths):
    """With W, b, x >= 0 every pre-activation is >= 0, the leaky ReLU is the identity, and the net
    is the single affine map x -> W8(...(W1 x + b1)...) + b8, computed here exactly in float64."""
    rng = np.random.default_rng(5)
    L = len(widths) - 1
    W = [f16(rng.uniform(0, 2.0 / widths[l], size=(widths[l + 1], widths[l]))) for l in range(L)]
    b = [f16(rng.uniform(0, 0.1, size=widths[l + 1])) for l in range(L)]
    x = f16(rng.uniform(0, 1, size=(300, widths[0])))
    y = oracle_mod.mlp_forward(W, b, x).view(np.float16).astype(np.float64)
    ref = x.astype(np.float64)
    for l in range(L):
        ref = ref @ W[l].astype(np.float64).T + b[l].astype(np.float64)
    bound = _forward_bound(widths, L)
    assert np.all(np.abs(y - ref) <= bound * np.abs(ref) + 1e-12)
    # The bound is tight enough to see a single dropped term or bias:
    assert bound < 5e-3


@pytest.mark.parametrize("seed", range(6))
def test_integer_exact_nets_match_int64_brute_force(oracle_mod, seed):
    """Small non-negative integers with every intermediate <= 2048: all binary16 values and all
    binary32 partial sums are exact, so the oracle must equal the int64 matrix product bit for bit.
    Shapes are random and non-square, so a transposed or mis-indexed operand cannot pass."""
    rng = np.random.default_rng(100 + seed)
    L = int(rng.integers(1, 9))
    widths = [int(w) for w in rng.integers(1, 40, size=L + 1)]
    for _ in range(200):
        W = [rng.integers(0, 3, size=(widths[l + 1], widths[l])) * (rng.random((widths[l + 1], widths[l])) < 0.15)
             for l in range(L)]
        b = [rng.integers(0, 4, size=widths[l + 1]) for l in range(L)]
        x = rng.integers(0, 4, size=(64, widths[0]))
        h, ok = x.astype(np.int64), True
        for l in range(L):
            h = h @ W[l].T.astype(np.int64) + b[l]
            ok &= bool(np.abs(h).max() <= 2048)
        if ok:
            break
    else:  # pragma: no cover
        pytest.skip("no in-range integer net found")
    y = oracle_mod.mlp_forward([f16(w) for w in W], [f16(v) for v in b], f16(x))
    assert np.array_equal(y, bits(h.astype(np.float64)))


def test_zero_last_layer_gives_its_bias(oracle_mod):
    rng = np.random.default_rng(3)
    widths = (16, 32, 32, 32, 32, 32, 32, 32, 4)
    W = [f16(rng.standard_normal((widths[l + 1], widths[l])) / np.sqrt(widths[l])) for l in range(8)]
    b = [f16(rng.uniform(-0.1, 0.1, widths[l + 1])) for l in range(8)]
    W[7][:] = 0
    x = f16(rng.uniform(-1, 1, (100, 16)))
    y = oracle_mod.mlp_forward(W, b, x)
    assert np.array_equal(y, np.repeat(bits(b[7])[None, :], 100, axis=0))


def test_zeroed_output_row_gives_exact_zero(oracle_mod):
    """A 'pad' output (a row of W8 and its bias set to zero) is exactly +0."""
    rng = np.random.default_rng(4)
    widths = (32, 64, 64, 64, 64, 64, 64, 64, 4)
    W = [f16(rng.standard_normal((widths[l + 1], widths[l])) / np.sqrt(widths[l])) for l in range(8)]
    b = [f16(rng.uniform(-0.1, 0.1, widths[l + 1])) for l in range(8)]
    W[7][3, :] = 0
    b[7][3] = 0
    y = oracle_mod.mlp_forward(W, b, f16(rng.uniform(-1, 1, (200, 32))))
    assert np.all(y[:, 3] == 0)
    assert np.any(y[:, :3] != 0)


def _intermediates(oracle_mod, W, b, x):
    """Every hidden activation, obtained from the oracle on prefix nets plus its own leaky."""
    out = []
    for l in range(1, len(W)):
        h = oracle_mod.mlp_forward(W[:l], b[:l], x)
        out.append(oracle_mod.leaky_f16_bits(h))
    return out


@pytest.mark.parametrize("k", [1, 3, -2])
def test_positive_homogeneity_without_bias(oracle_mod, k):
    """With b = 0, scaling the input by 2^k scales every output by 2^k bit-exactly as long as no
    value is subnormal or overflows (RNE commutes with power-of-two scaling and the leaky ReLU is
    positively homogeneous).  Rows with a subnormal intermediate in either run are excluded."""
    rng = np.random.default_rng(7)
    widths = (32, 64, 64, 64, 64, 64, 64, 64, 4)
    W = [f16(rng.standard_normal((widths[l + 1], widths[l])) / np.sqrt(widths[l])) for l in range(8)]
    b = [f16(np.zeros(widths[l + 1])) for l in range(8)]
    # Inputs of magnitude ~256 keep the hidden values far from the binary16 subnormal range
    # (|v| < 2^-14, reached after the slope when |v| < ~6e-3) and far from overflow (65504).
    x = f16(rng.uniform(-256, 256, (400, 32)))
    xs = f16(x.astype(np.float64) * 2.0**k)
    y = oracle_mod.mlp_forward(W, b, x).view(np.float16).astype(np.float64)
    ys = oracle_mod.mlp_forward(W, b, xs).view(np.float16).astype(np.float64)

    def clean(inp, outp):
        m = np.ones(inp.shape[0], bool)
        for h in _intermediates(oracle_mod, W, b, inp) + [bits(outp)]:
            a = np.abs(h.view(np.float16).astype(np.float64))
            m &= ~np.any((a > 0) & (a < 2.0**-14), axis=1)
        return m

    keep = clean(x, y) & clean(xs, ys)
    assert keep.sum() > 300
    assert np.array_equal(ys[keep], y[keep] * 2.0**k)


def test_rows_are_independent_and_row_subset_matches(oracle_mod):
    rng = np.random.default_rng(9)
    widths = (16, 32, 32, 4)
    W = [f16(rng.standard_normal((widths[l + 1], widths[l]))) for l in range(3)]
    b = [f16(rng.uniform(-0.1, 0.1, widths[l + 1])) for l in range(3)]
    x = f16(rng.uniform(-1, 1, (97, 16)))
    full = oracle_mod.mlp_forward(W, b, x)
    idx = np.array([96, 0, 5, 5, 50])
    assert np.array_equal(oracle_mod.mlp_forward_rows(W, b, x, idx), full[idx])
    assert np.array_equal(oracle_mod.mlp_forward(W, b, x[:13]), full[:13])
    assert np.array_equal(oracle_mod.mlp_forward(W, b, x, threads=4), full)


def test_accumulation_is_binary32(oracle_mod):
    """2048 + 1 + 1 is 2050 (0x6801) when the sum is carried in binary32 and rounded once; a binary16
    running sum would stick at 2048 (2049 ties to even).  FP16 inputs with an FP32 accumulator are
    the mixed-precision convention of "Working with Cooperative Matrices" ("Hardware Constraints and
    Capabilities")."""
    W = [f16([[1.0, 1.0, 1.0]])]
    b = [f16([0.0])]
    y = oracle_mod.mlp_forward(W, b, f16([[2048.0, 1.0, 1.0]]))
    assert int(y[0, 0]) == 0x6801
