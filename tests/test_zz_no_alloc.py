"""moe_run_noalloc (the run call for callers that cannot allocate: its
workspace is the library's static device array) against moe_run_ws with a
caller workspace, through the C ABI on the GPU: the same kernels, so the
outputs must be bit-identical, on two calls in a row (the second with fewer
tokens, over the array the first call left behind), for every activation
format; and a layer whose workspace exceeds the array is refused before any
launch."""
import numpy as np
import pytest

import moe_inputs as MI
from tests.harness import Problem, check_output

pytestmark = pytest.mark.gpu

CASES = [  # (wfmt, afmt, seed): T = 96 then 40 tokens, E = 12, top-4, H 1024, I 512
    ("mxfp4", "fp8", 61), ("mxfp4", "bf16", 62), ("int4", "fp8", 63),
    ("mxfp4", "mxfp8", 64), ("mxfp4", "mxfp4", 65),
]


def _run_both(p, T):
    import torch

    import mixed_precision_moe_topk_amd as M

    wl = p.wl
    h, lg = p.h_dev[:T].contiguous(), p.l_dev[:T].contiguous()
    out_ws = torch.empty((T, wl.hidden), dtype=torch.int16, device="cuda")
    out_na = torch.full((T, wl.hidden), 0x7FC0, dtype=torch.int16, device="cuda")
    ws = torch.empty(M.workspace_query(p.dims, T, wl.top_k), dtype=torch.uint8, device="cuda")
    M.run_ws(p.dims, h, lg, p.weights, p.scales, wl.top_k, out_ws, ws)
    M.run_noalloc(p.dims, h, lg, p.weights, p.scales, wl.top_k, out_na)
    torch.cuda.synchronize()
    return out_ws.cpu().numpy().view(np.uint16), out_na.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("wf,af,seed", CASES, ids=[f"{c[0]}x{c[1]}" for c in CASES])
def test_noalloc_matches_caller_workspace(wf, af, seed):
    import mixed_precision_moe_topk_amd as M

    wl = MI.small_workload(96, 12, 4, 1024, 512, wf, af, seed, 1.0)
    assert M.workspace_query(M.LayerDims(12, 1024, 512, wf, af), 96, 4) <= M.NOALLOC_SCRATCH_BYTES
    p = Problem(wl, experts_for_oracle=range(12))
    for T in (96, 40):  # the second call smaller than the first
        ref, got = _run_both(p, T)
        assert np.array_equal(got, ref), (T, np.count_nonzero(got != ref))
    # and within the output contract of the oracle (40-token batch)
    r = p.run_oracle(tokens=np.arange(40))
    check_output(got, r["out"])


def test_noalloc_refuses_a_workspace_beyond_the_array():
    import torch

    import mixed_precision_moe_topk_amd as M

    d = M.LayerDims(256, 7168, 2048, "mxfp4", "fp8")
    T = 4096
    assert M.workspace_query(d, T, 8) > M.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, 7168), dtype=torch.int16, device="cuda")
    lg = torch.zeros((T, 256), dtype=torch.float32, device="cuda")
    w = torch.zeros(16, dtype=torch.uint8, device="cuda")
    out = torch.zeros((T, 7168), dtype=torch.int16, device="cuda")
    with pytest.raises(M.MoeError) as ei:
        M.run_noalloc(d, x, lg, w, w, 8, out)
    assert ei.value.status == 3 and "static scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert int(out.abs().sum()) == 0  # nothing ran
