"""The run call under HIP graph capture: it allocates nothing, synchronises
nothing and issues no memset, so a captured layer replays on the device.  Each
replay (with the program's own eager work and synchronisations between
replays) must give the eager result bit for bit."""
import numpy as np
import pytest

import moe_inputs as MI
from tests.harness import Problem

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape", [(16, 8, 2, 256, 512, "mxfp4", "fp8"),      # single-block routing
                                   (300, 5, 2, 256, 384, "mxfp4", "mxfp8"),   # chunked routing
                                   (64, 32, 4, 512, 256, "mxfp4", "bf16")])
def test_captured_layer_replays_match_eager(shape):
    import torch

    import mixed_precision_moe_topk_amd as M

    T, E, k, H, I, wf, af = shape
    wl = MI.small_workload(T, E, k, H, I, wf, af, 71, 1.0)
    p = Problem(wl, experts_for_oracle=[])
    eager = p.run_gpu()["out"]
    lay = M.workspace_layout(p.dims, T, k)
    ws = torch.empty(lay.total, dtype=torch.uint8, device="cuda")
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream
        M.run_ws(p.dims, p.h_dev, p.l_dev, p.weights, p.scales, k, out, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        M.run_ws(p.dims, p.h_dev, p.l_dev, p.weights, p.scales, k, out, ws)
    for _ in range(3):
        out.zero_()
        ws.fill_(0xAB)  # stale intermediates must not matter
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint16), eager)
        p.run_gpu()  # eager work between replays
    del graph
