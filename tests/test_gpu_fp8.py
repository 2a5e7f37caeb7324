"""GPU parity of the FP8 kernels (MLP_LAYOUT_PACKED_FP8) against the oracle's FP8 network, through the
C ABI, on the dedicated shapes.

- order-free nets, bit for bit against the FP8 oracle:
  - integer-exact nets (every weight, every 16 h and every partial sum exact in E4M3 / binary32);
  - signed permutation chains: one nonzero weight per row, a power of two of either sign (so its E4M3
    code is exact), zero or random biases (bias plus one product is a single binary32 rounding in
    any order); every layer's input goes through E4M3(16 h) of both signs and every negative
    pre-activation through the binary16 leaky slope;
  - the eight-layer sign-alternating diagonal golden (tests/golden/fp8_sign_alternating_diag.json),
    embedded in the small shape;
- random weights at the workloads' initialisations, ragged row counts, and at full size on sampled rows
  in the benchmark's launch configuration: the contract tolerance on every element and the FP8 bar
  below.

The FP8 bar (its own tolerance: the contract's 1e-2 is stated for the FP16 network).  The kernel and
the oracle quantise identically (the same E4M3 codes for the weights, the same scale per row, the same
conversion of 16 h).  Every product of two E4M3 values has at most 8 significant bits, so at these
initialisations the binary32 sums are exact in any order: the test checks that the network evaluated
with exact sums (rounded once to binary32) gives the oracle's bits, so summation order alone explains
no difference.  What remains is the FP8 MFMA's own accumulator, which need not be an IEEE binary32
adder.  The bar models an accumulator accurate to half a binary16 ulp of each dot product (the
precision of the layer's own FP16 result): the test evaluates the network with every layer's sums
perturbed by a random relative error of up to 2^-11 before the binary16 rounding (two seeded draws)
and takes the larger statistics of the two.  Such an error flips some binary16 roundings by one ulp,
and a flip that takes the next layer's 16 h across an E4M3 rounding boundary moves that activation by
a whole E4M3 step (2^-4 .. 2^-3 of its size): at these initialisations the outputs then move by up to
~0.02-0.04, ~1e-3 on average.  The GPU passes if max |d| <= 1.5 x the model's max, mean |d| <= 1.25 x
its mean and the count beyond the contract's 1e-2 <= 1.25 x its count + 2 (the factors cover the
draw-to-draw spread of these statistics: the max varies by ~1.4x between draws, the mean and the count
by ~10 %).  Sign, slope and indexing slips fail the bit-exact nets above.
"""
import json
from pathlib import Path

import numpy as np
import pytest

from conftest import host_threads
from gpu_util import CONTRACT_TOL, log, run
from mlp_neural_shading_amd import binding as B
from mlp_neural_shading_amd import workloads

pytestmark = pytest.mark.gpu

FP8 = B.MLP_LAYOUT_PACKED_FP8
GOLDEN = Path(__file__).parent / "golden" / "fp8_sign_alternating_diag.json"


def f16(a):
    return np.asarray(a, dtype=np.float64).astype(np.float16)


def _e4m3(x):
    """E4M3 value nearest to x (nearest even), via PyTorch's float8_e4m3fn cast."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e4m3fn).to(torch.float32).numpy()


def _fp8_net(Ws, bs, x_bits, rng=None, rel=0.0):
    """The FP8 network (the oracle's readings) with exact sums rounded once to binary32; with rel > 0
    every sum is first scaled by (1 + u rel), u ~ U(-1, 1) per element (an accumulator error model)."""
    s = np.uint16(0x211F).view(np.float16)  # half(0.01)
    h = np.asarray(x_bits).view(np.float16).astype(np.float32)
    L = len(Ws)
    for l in range(L):
        W = np.asarray(Ws[l]).view(np.float16).astype(np.float64)
        amax = np.abs(W).max(axis=1)
        E = np.zeros(W.shape[0])
        nz = amax > 0
        E[nz] = np.ceil(np.log2(amax[nz] / 448.0))
        E[nz] += amax[nz] > 448.0 * 2.0 ** E[nz]  # guard the log2 rounding: smallest E with amax <= 448 2^E
        E[nz] -= amax[nz] <= 448.0 * 2.0 ** (E[nz] - 1)
        Wq = _e4m3((W / 2.0 ** E[:, None]).astype(np.float32)).astype(np.float64) * 2.0 ** E[:, None]
        xq = _e4m3(np.float32(16) * h).astype(np.float64) / 16.0
        acc = xq @ Wq.T + np.asarray(bs[l]).view(np.float16).astype(np.float64)[None, :]
        if rel:
            acc = acc * (1.0 + rel * rng.uniform(-1.0, 1.0, size=acc.shape))
        v = acc.astype(np.float32).astype(np.float16)
        if l + 1 < L:
            v = np.maximum(v, (v * s).astype(np.float16))
        h = v.astype(np.float32)
    return h.astype(np.float16).view(np.uint16)


def _stats(a_bits, o_bits):
    a = np.asarray(a_bits).view(np.float16).astype(np.float64)
    o = np.asarray(o_bits).view(np.float16).astype(np.float64)
    d = np.abs(a - o)
    beyond = ~((d <= CONTRACT_TOL) | (d <= CONTRACT_TOL * np.abs(o)))
    return d, beyond


def _compare_fp8(g_bits, o_bits, Ws, bs, x_bits, what, order_free=True):
    """GPU vs oracle against the bar of the accumulator error model (module docstring).  order_free:
    require every sum to be exact in binary32 (then the exact-sum network gives the oracle's bits); over
    many rows a few sums of products spanning more than 24 bits are not, and their binary32 summation
    order matters by ~2^-24 relative, far inside the model's 2^-11 perturbation: with order_free=False
    those outputs are counted and bounded instead."""
    g = np.asarray(g_bits).view(np.float16).astype(np.float64)
    assert np.isfinite(g).all(), what
    exact = _fp8_net(Ws, bs, x_bits)
    if order_free:
        assert np.array_equal(exact, o_bits), "%s: the sums are not order-free here" % what
    else:
        differ = int((exact != np.asarray(o_bits)).sum())
        log("  %s: %d of %d outputs where binary32 summation order matters" % (what, differ, exact.size))
        assert differ <= 1e-3 * exact.size, what
    model = [_stats(_fp8_net(Ws, bs, x_bits, np.random.default_rng(100 + k), 2.0 ** -11), o_bits) for k in range(2)]
    m_max = max(d.max() for d, _ in model)
    m_mean = max(d.mean() for d, _ in model)
    m_beyond = max(int(b.sum()) for _, b in model)
    d, beyond = _stats(g_bits, o_bits)
    same = float((np.asarray(g_bits) == np.asarray(o_bits)).mean())
    log("  %s: GPU max |d| %.3g, mean %.3g, beyond 1e-2 %d of %d, bit-identical %.4f; half-ulp model: max %.3g, "
        "mean %.3g, beyond %d" % (what, d.max(), d.mean(), int(beyond.sum()), d.size, same, m_max, m_mean, m_beyond))
    assert d.max() <= 1.5 * m_max, what
    assert d.mean() <= 1.25 * m_mean, what
    assert beyond.sum() <= 1.25 * m_beyond + 2, what
    return same


def _signed_chain(widths, rng, diag=(1, -64, -1, -64, -1, -64, -1, 1), random_bias=False):
    """One nonzero weight per row, diag[l] (a power of two, exact in E4M3 under its row scale), from a
    random partial permutation; zero biases or random binary16 ones in [-0.1, 0.1]."""
    L = len(widths) - 1
    Ws, bs = [], []
    for l in range(L):
        win, wout = widths[l], widths[l + 1]
        W = np.zeros((wout, win))
        src = rng.permutation(max(win, wout))
        for r in range(wout):
            W[r, src[r] % win] = diag[l % len(diag)]
        Ws.append(f16(W))
        bs.append(f16(rng.uniform(-0.1, 0.1, size=wout) if random_bias else np.zeros(wout)))
    return Ws, bs


@pytest.mark.parametrize("random_bias", [False, True], ids=["zero-bias", "random-bias"])
@pytest.mark.parametrize("name", list(workloads.ALIASES))
def test_signed_permutation_chain_bit_exact(oracle_mod, name, random_bias):
    rng = np.random.default_rng(57)
    widths = workloads.get(name).widths
    Ws, bs = _signed_chain(widths, rng, random_bias=random_bias)
    x = f16(rng.uniform(-1, 1, size=(1000 + 13, widths[0]))).view(np.uint16)
    ref = oracle_mod.mlp_forward_fp8(Ws, bs, x)
    assert (ref.view(np.float16) < 0).any() and (ref.view(np.float16) > 0).any()
    log("FP8 signed permutation chain", name, "random bias" if random_bias else "zero bias")
    y = run(Ws, bs, x, layout=FP8)
    assert np.array_equal(y, ref)


def test_sign_alternating_golden_on_the_small_shape(oracle_mod):
    """The golden's four-wide diagonal chain as the first four features of the small shape
    (16 -> 32 x 7 -> 4, diagonal weights d_l on rows that have a same-index input, zero elsewhere)."""
    g = json.loads(GOLDEN.read_text())
    widths = workloads.get("small").widths
    Ws = [f16(np.eye(widths[l + 1], widths[l]) * g["diag"][l]) for l in range(8)]
    bs = [f16(np.zeros(widths[l + 1])) for l in range(8)]
    rng = np.random.default_rng(3)
    x = rng.uniform(-1, 1, size=(300, widths[0]))
    x[:, :4] = np.array(g["x"])[None, :]
    x = f16(x).view(np.uint16)
    y = run(Ws, bs, x, layout=FP8)
    want = np.array([int(v, 16) for v in g["y_bits"]], np.uint16)
    assert (y == want[None, :]).all()
    assert np.array_equal(y, oracle_mod.mlp_forward_fp8(Ws, bs, x))


@pytest.mark.parametrize("name", list(workloads.ALIASES))
def test_integer_exact_nets_bit_exact(oracle_mod, name):
    widths = workloads.get(name).widths
    rng = np.random.default_rng(90)
    L = len(widths) - 1
    W = [np.zeros((widths[l + 1], widths[l]), np.int64) for l in range(L)]
    for l in range(L):
        for r in range(widths[l + 1]):
            W[l][r, rng.integers(0, widths[l])] = 1  # one one per row
    b = [rng.integers(0, 2, size=widths[l + 1]) for l in range(L)]
    x = rng.integers(0, 4, size=(2000 + 37, widths[0]))
    h = x.copy()
    for l in range(L):
        h = h @ W[l].T + b[l]
    assert h.max() <= 16  # 16 h <= 256 is an E4M3 value for every integer h <= 16
    Wf, bf, xf = [f16(w) for w in W], [f16(v) for v in b], f16(x)
    log("FP8 integer-exact", name)
    y = run(Wf, bf, xf.view(np.uint16), layout=FP8)
    assert np.array_equal(y, f16(h).view(np.uint16))
    assert np.array_equal(y, oracle_mod.mlp_forward_fp8(Wf, bf, xf))


@pytest.mark.parametrize("name", list(workloads.ALIASES))
def test_random_weights(oracle_mod, name):
    wl = workloads.get(name)
    Ws, bs = wl.weights()
    rows = 4133 if name != "wide" else 1037
    import torch

    xt = wl.inputs(device="cuda", rows=rows)
    xb = xt.cpu().view(torch.int16).numpy().view(np.uint16)
    log("FP8 random weights", name, "rows", rows)
    y = run(Ws, bs, xt, layout=FP8)
    ref = oracle_mod.mlp_forward_fp8(Ws, bs, xb, threads=host_threads())
    _compare_fp8(y, ref, Ws, bs, xb, name)
    # and the FP8 network stays close to the FP16 one
    y16 = oracle_mod.mlp_forward(Ws, bs, xb, threads=host_threads())
    d = np.abs(y.view(np.float16).astype(np.float64) - y16.view(np.float16).astype(np.float64))
    log("  FP8 vs FP16 network: mean |d| %.3g, max %.3g" % (d.mean(), d.max()))
    assert d.mean() < 0.015 and d.max() < 0.1


def test_prefixes_and_determinism(oracle_mod):
    """Every batch prefix gives the leading rows of the full batch, and reruns give the same bits."""
    import torch

    wl = workloads.get("page")
    Ws, bs = wl.weights()
    xt = wl.inputs(device="cuda", rows=3000)
    full = run(Ws, bs, xt, layout=FP8)
    for n in (1, 31, 33, 65, 1000):
        assert np.array_equal(run(Ws, bs, xt[:n], layout=FP8, pack=False), full[:n]), n
    assert np.array_equal(run(Ws, bs, xt, layout=FP8, pack=False), full)


def _rows_bits(t, idx):
    import torch

    sel = t.index_select(0, torch.as_tensor(idx, device=t.device))
    return sel.cpu().view(torch.int16).numpy().view(np.uint16)


# Full size, one dispatch over the whole batch (the launch configuration bench.py times): every row of
# the small net, the page net's 65,536 distinct inputs (and its 16 replicas bit-identical), and for the
# larger nets the first and last rows plus seeded random rows (for the streaming net also the rows whose
# inputs straddle each 2 GiB boundary), against the FP8 oracle with the bar above.
@pytest.mark.parametrize("name,edge,n_random", [("small", 4096, 0), ("page", 65536, 0), ("hetero", 16384, 32768),
                                                ("wide", 8192, 16384), ("stream", 8192, 16384)])
def test_full_size_sampled(oracle_mod, name, edge, n_random):
    import torch

    wl = workloads.get(name)
    Ws, bs = wl.weights()
    x = wl.inputs(device="cuda")
    y = torch.empty((wl.batch, wl.widths[-1]), dtype=torch.float16, device="cuda")
    log("FP8 full size", wl.name)
    B.mlp_pack_weights(Ws, bs, FP8)
    B.mlp_infer(wl.batch, x.data_ptr(), y.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all())
    if wl.replicas > 1:
        u = wl.unique_rows
        for r in range(1, wl.replicas):
            assert torch.equal(y[r * u:(r + 1) * u], y[:u]), "replica %d differs" % r
    rng = np.random.default_rng(78)
    extra = []
    if name == "stream":
        row_bytes = 2 * wl.widths[0]
        for k in (1, 2, 3):
            r = (k << 31) // row_bytes
            extra += list(range(r - 64, r + 64))
    idx = np.concatenate([np.arange(edge), np.arange(wl.batch - edge, wl.batch),
                          rng.integers(0, wl.batch, size=n_random), np.asarray(extra, dtype=np.int64)])
    idx = np.unique(idx[(idx >= 0) & (idx < wl.batch)])
    xb, yb = _rows_bits(x, idx), _rows_bits(y, idx)
    del x, y
    torch.cuda.empty_cache()
    ref = oracle_mod.mlp_forward_fp8(Ws, bs, xb, threads=host_threads())
    _compare_fp8(yb, ref, Ws, bs, xb, "%s full size (%d rows checked)" % (name, idx.size), order_free=False)
