"""Helpers for the GPU parity tests: run the HIP library through its C ABI and compare with the
oracle at the contract tolerance and at the internal bar."""
from __future__ import annotations

import sys

import numpy as np

from mlp_neural_shading_amd import binding as B

# An element passes if |g - o| <= 1e-2 or |g - o| <= 1e-2 * |o|; NaN/Inf never pass.
CONTRACT_TOL = 1e-2
# Legitimate differences come only from the MFMA's summation order inside an FP32 accumulator
# (~1e-7 relative per sum) turned into at most one or two binary16 ulps per layer; at these
# initialisations outputs are below ~1 in magnitude (ulp <= 2^-11 ~ 4.9e-4), so 2e-3 bounds four
# ulps of accumulated disagreement.  A leaky-slope or bias bug moves outputs by >= 7e-3.
INTERNAL_TOL = 2e-3


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def device():
    import torch

    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible GPU")
    B.lib()  # raises if the HIP library is not built
    return torch.device("cuda:0")


def to_device(x_bits: np.ndarray):
    import torch

    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    return torch.from_numpy(x_bits.view(np.int16)).view(torch.float16).to(device())


def run(Ws, bs, x, layout=B.MLP_LAYOUT_PACKED, act=B.MLP_ACT_VECTOR, pack=True):
    """Pack (unless pack=False), run one mlp_infer_ex over all rows of x, return output bits."""
    import torch

    dev = device()
    if pack:
        B.mlp_pack_weights(Ws, bs, layout)
    xt = x if isinstance(x, torch.Tensor) else to_device(x)
    wL = int(np.asarray(bs[-1]).shape[0])
    out = torch.full((xt.shape[0], wL), float("nan"), dtype=torch.float16, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    B.mlp_infer_ex(xt.shape[0], xt.data_ptr(), out.data_ptr(), stream, act)
    torch.cuda.synchronize()
    return out.cpu().view(torch.int16).numpy().view(np.uint16)


def compare(g_bits, o_bits, internal=INTERNAL_TOL, what=""):
    g = np.asarray(g_bits).view(np.float16).astype(np.float64)
    o = np.asarray(o_bits).view(np.float16).astype(np.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    assert np.isfinite(g).all(), "%s: non-finite GPU output" % what
    d = np.abs(g - o)
    ok = (d <= CONTRACT_TOL) | (d <= CONTRACT_TOL * np.abs(o))
    assert ok.all(), "%s: %d elements outside the contract tolerance, max |d| %.3g" % (what, (~ok).sum(), d.max())
    assert d.max() <= internal, "%s: max |d| %.3g above the internal bar %.3g" % (what, d.max(), internal)
    same = float((np.asarray(g_bits) == np.asarray(o_bits)).mean())
    return {"max_abs": float(d.max()), "bit_identical_frac": same}
