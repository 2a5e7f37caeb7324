"""GPU test: mlp_infer on its own stream while other work runs on another stream (the async-compute
situation of "Optimization Techniques", "Async Compute": the network shares the GPU with other
work) gives the same bits as when it runs alone, and the other work is undisturbed."""
import numpy as np
import pytest

from mlp_neural_shading_amd import binding as B
from mlp_neural_shading_amd import workloads

from gpu_util import device, log, run

pytestmark = pytest.mark.gpu


def test_concurrent_streams_give_identical_results():
    import torch

    dev = device()
    wl = workloads.get("page")
    Ws, bs = wl.weights()
    x = wl.inputs(device=dev, rows=65536)
    expect = run(Ws, bs, x)  # packs the network and runs it alone
    src = torch.arange(64 * 1024 * 1024, device=dev, dtype=torch.int32)
    dst = torch.zeros_like(src)
    a = torch.randn(2048, 2048, device=dev)
    c_expect = a @ a
    s_mlp, s_bg = torch.cuda.Stream(), torch.cuda.Stream()
    outs = [torch.full((x.shape[0], wl.widths[-1]), float("nan"), dtype=torch.float16, device=dev) for _ in range(4)]
    s_mlp.wait_stream(torch.cuda.current_stream())
    s_bg.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s_bg):
        for _ in range(3):
            dst.copy_(src)
            c = a @ a
    for o in outs:
        B.mlp_infer(x.shape[0], x.data_ptr(), o.data_ptr(), s_mlp.cuda_stream)
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        got = o.cpu().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got, expect), i
    assert torch.equal(dst, src)
    assert torch.allclose(c, c_expect, rtol=1e-4, atol=1e-3)
    log("concurrent streams: %d inferences identical" % len(outs))
