"""GPU test: mlp_infer recorded into a HIP graph (stream capture) and replayed.  The fused path
allocates nothing and clears nothing per call, so a captured call is just the kernel launch; every
replay, with the program's own eager work and synchronisations in between, must give the eager
result bit for bit."""
import numpy as np
import pytest

from mlp_neural_shading_amd import binding as B
from mlp_neural_shading_amd import workloads

from gpu_util import device, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("layout", [B.MLP_LAYOUT_PACKED, B.MLP_LAYOUT_PACKED_FP8])
def test_graph_replays_match_eager(layout):
    import torch

    dev = device()
    wl = workloads.get("page")
    Ws, bs = wl.weights()
    x = wl.inputs(device=dev, rows=20000)
    y = torch.empty((x.shape[0], wl.widths[-1]), dtype=torch.float16, device=dev)
    B.mlp_pack_weights(Ws, bs, layout)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        B.mlp_infer(x.shape[0], x.data_ptr(), y.data_ptr(), s.cuda_stream)
    torch.cuda.synchronize()
    eager = y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(3):
            B.mlp_infer(x.shape[0], x.data_ptr(), y.data_ptr(), s.cuda_stream)
    for i in range(5):
        y.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager), i
    log("graph replays identical to eager, layout", layout)
