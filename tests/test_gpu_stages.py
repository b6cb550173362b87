"""The stage entry points moe_route and moe_quantize_tokens, called through
the C ABI on the GPU, against the CPU oracle on the same seeded inputs:
routing ids, expert offsets, row maps and the GEMM work map bit-exact,
routing weights within 1e-6; token codes, token scales and E8M0 block scales
bit-exact."""
import numpy as np
import pytest

import moe_inputs as MI
import oracle as O
from oracle import formats as F
from oracle import quant as Q
from tests.harness import expected_work_map, mx_scale_row_bytes, mx_scales_canonical

pytestmark = pytest.mark.gpu


def _route_outputs(torch, T, E, k):
    dev = "cuda"
    return (torch.empty((T, k), dtype=torch.int32, device=dev),
            torch.empty((T, k), dtype=torch.float32, device=dev),
            torch.empty(E + 1, dtype=torch.int32, device=dev),
            torch.empty(T * k, dtype=torch.int32, device=dev),
            torch.empty((T, k), dtype=torch.int32, device=dev))


ROUTE_CASES = [
    # (tokens, experts, top_k, logit bias sigma, tie grid (0: continuous), seed)
    (1, 8, 2, 0.0, 0.0, 101),       # single token
    (37, 8, 2, 0.0, 0.0, 102),      # one partial 64-token chunk
    (64, 256, 8, 0.0, 0.0, 103),    # the decode batch shape (single-block routing)
    (65, 256, 8, 0.0, 0.0, 104),    # first batch past the single-block path
    (300, 384, 6, 2.0, 0.0, 105),   # skewed loads, empty experts
    (257, 16, 4, 0.0, 0.5, 106),    # logits on a 0.5 grid: many exact ties
    (130, 1024, 16, 0.0, 0.25, 107),  # the most experts and the largest top-k, with ties
    (5, 3, 3, 0.0, 0.0, 108),       # k = E
    (1024, 256, 8, 0.0, 0.0, 109),  # the INT4 batch (16 chunks)
    (1025, 256, 8, 0.0, 0.0, 110),  # a last chunk of one token
    (700, 1024, 2, 0.0, 0.25, 111),  # 11 chunks x 1024 experts, ties
    (500, 128, 4, 2.0, 0.5, 112),   # 8 chunks, skewed, ties
]


@pytest.mark.parametrize("T,E,k,bias,grid,seed", ROUTE_CASES)
def test_route_matches_oracle(T, E, k, bias, grid, seed):
    import torch

    import mixed_precision_moe_topk_amd as M

    logits = MI.router_logits(seed, T, E, bias)
    if grid:
        logits = (np.round(logits / grid) * grid).astype(np.float32)
    d = M.LayerDims(E, 256, 256, "mxfp4", "fp8")
    ws = torch.full((M.workspace_query(d, T, k),), 0xA5, dtype=torch.uint8, device="cuda")
    ids, w, off, rt, sr = _route_outputs(torch, T, E, k)
    M.route(d, torch.from_numpy(logits).cuda(), k, ids, w, off, rt, sr, ws)
    torch.cuda.synchronize()

    rid, rw = O.route(logits, k)
    roff, rrt, _, rsr = O.expand(rid, E)
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert np.max(np.abs(w.cpu().numpy() - rw)) <= 1e-6
    assert np.array_equal(off.cpu().numpy(), roff.astype(np.int32))
    assert np.array_equal(rt.cpu().numpy(), rrt.astype(np.int32))
    assert np.array_equal(sr.cpu().numpy(), rsr.astype(np.int32))
    # the GEMM work map lands in the workspace regions the layout names
    lay = M.workspace_layout(d, T, k)
    wsn = ws.cpu().numpy()
    n = int(wsn[lay.num_tiles:lay.num_tiles + 4].view(np.int32)[0])
    tiles = wsn[lay.tiles:lay.tiles + 16 * n].view(np.int32).reshape(n, 4)[:, :3]
    assert np.array_equal(tiles, expected_work_map(roff, lay.tile_m))


def test_route_nan_logits_rank_as_minus_infinity():
    """Regression: NaN logits (a whole row, and scattered entries) rank as
    -inf on the GPU as in the oracle; every id is a valid expert index and
    the row maps stay a permutation; finite weights match, NaN weights sit
    where the oracle's do."""
    import torch

    import mixed_precision_moe_topk_amd as M

    T, E, k = 70, 256, 8
    logits = MI.router_logits(110, T, E)
    logits[3, :] = np.nan
    logits[5, ::3] = np.nan
    logits[9, 10] = np.nan
    logits[11, :] = -np.inf
    d = M.LayerDims(E, 256, 256, "mxfp4", "fp8")
    ws = torch.full((M.workspace_query(d, T, k),), 0xA5, dtype=torch.uint8, device="cuda")
    ids, w, off, rt, sr = _route_outputs(torch, T, E, k)
    M.route(d, torch.from_numpy(logits).cuda(), k, ids, w, off, rt, sr, ws)
    torch.cuda.synchronize()
    rid, rw = O.route(logits, k)
    roff, rrt, _, rsr = O.expand(rid, E)
    g_ids, g_w = ids.cpu().numpy(), w.cpu().numpy()
    assert np.array_equal(g_ids, rid)
    assert g_ids.min() >= 0 and g_ids.max() < E
    assert np.array_equal(np.isnan(g_w), np.isnan(rw))
    fin = ~np.isnan(rw)
    assert np.max(np.abs(g_w[fin] - rw[fin])) <= 1e-6
    assert np.array_equal(off.cpu().numpy(), roff.astype(np.int32))
    assert np.array_equal(rt.cpu().numpy(), rrt.astype(np.int32))
    assert np.array_equal(sr.cpu().numpy(), rsr.astype(np.int32))


def test_route_into_workspace_regions():
    """Outputs placed at the workspace offsets moe_run_ws uses give the same
    bits as separate buffers."""
    import torch

    import mixed_precision_moe_topk_amd as M

    T, E, k = 200, 64, 6
    logits = torch.from_numpy(MI.router_logits(109, T, E, 1.0)).cuda()
    d = M.LayerDims(E, 512, 256, "mxfp4", "fp8")
    lay = M.workspace_layout(d, T, k)
    ws = torch.zeros(lay.total, dtype=torch.uint8, device="cuda")

    def region(off, count, dtype):
        return ws[off:off + 4 * count].view(dtype)

    inside = (region(lay.ids, T * k, torch.int32), region(lay.topk_w, T * k, torch.float32),
              region(lay.offsets, E + 1, torch.int32), region(lay.row_token, T * k, torch.int32),
              region(lay.slot_row, T * k, torch.int32))
    M.route(d, logits, k, *inside, ws)
    sep = _route_outputs(torch, T, E, k)
    ws2 = torch.zeros_like(ws)
    M.route(d, logits, k, *sep, ws2)
    torch.cuda.synchronize()
    for a, b in zip(inside, sep):
        assert torch.equal(a.reshape(-1).view(torch.int32), b.reshape(-1).view(torch.int32))


def _tokens(seed, T, H):
    """bf16 bits of N(0,1) tokens; token 0 all zero, token 1 scaled by 2^20,
    token 2 by 2^-20 (exact in bf16), when there are that many."""
    bits = MI.hidden_bf16(seed, T, H).copy()
    x = F.bf16_to_f32(bits)
    if T > 0:
        bits[0] = 0
    for t, e in ((1, 20), (2, -20)):
        if t < T:
            bits[t] = ((x[t] * np.float32(2.0 ** e)).astype(np.float32).view(np.uint32) >> 16)
    return bits


@pytest.mark.parametrize("afmt", ["fp8", "mxfp8", "mxfp4"])
@pytest.mark.parametrize("T,H,seed", [(1, 128, 201), (33, 7168, 202), (200, 384, 203),
                                      (3, 8320, 204)])
def test_quantize_tokens_matches_oracle(afmt, T, H, seed):
    import torch

    import mixed_precision_moe_topk_amd as M

    bits = _tokens(seed, T, H)
    x = F.bf16_to_f32(bits)
    d = M.LayerDims(8, H, 256, "mxfp4", afmt)
    cols = H // 2 if afmt == "mxfp4" else H
    codes = torch.empty((T, cols), dtype=torch.uint8, device="cuda")
    scales = torch.empty(T, dtype=torch.float32, device="cuda")
    mx = afmt != "fp8"
    bsc = torch.empty((T, mx_scale_row_bytes(H)), dtype=torch.uint8, device="cuda") if mx else None
    M.quantize_tokens(d, torch.from_numpy(bits.view(np.int16)).cuda(), codes, scales, bsc)
    torch.cuda.synchronize()
    gc, gs = codes.cpu().numpy(), scales.cpu().numpy()
    if afmt == "fp8":
        rc, rs = Q.e4m3_rows(x)
        assert np.array_equal(gc, rc)
        assert np.array_equal(gs.view(np.uint32), rs.view(np.uint32))
        return
    rc, rsc = Q.mxfp8_rows(x) if afmt == "mxfp8" else Q.mxfp4_quantize(x)
    assert np.array_equal(gc, rc)
    assert np.array_equal(mx_scales_canonical(bsc.cpu().numpy(), H), rsc)
    assert np.all(gs == 1.0)


@pytest.mark.parametrize("afmt", ["fp8", "mxfp8", "mxfp4"])
def test_quantize_tokens_tiny_and_huge_rows(afmt):
    """Token rows scaled by 2^-100 ... 2^-131 (amax / 448 subnormal, 1 / s
    beyond the float32 range, bf16 subnormal elements) and by 2^100, rounded
    to bf16: codes and scales bit-exact against the oracle's quantiser."""
    import torch

    import mixed_precision_moe_topk_amd as M

    H = 512
    exps = [-100, -115, -119, -120, -122, -124, -126, -128, -131, 100, 0]
    x0 = F.bf16_to_f32(MI.hidden_bf16(211, len(exps), H))
    x = np.stack([x0[i] * np.float32(2.0 ** e) for i, e in enumerate(exps)]).astype(np.float32)
    bits = F.bf16_rne(x)
    x = F.bf16_to_f32(bits)
    T = len(exps)
    d = M.LayerDims(8, H, 256, "mxfp4", afmt)
    cols = H // 2 if afmt == "mxfp4" else H
    codes = torch.empty((T, cols), dtype=torch.uint8, device="cuda")
    scales = torch.empty(T, dtype=torch.float32, device="cuda")
    mx = afmt != "fp8"
    bsc = torch.empty((T, mx_scale_row_bytes(H)), dtype=torch.uint8, device="cuda") if mx else None
    M.quantize_tokens(d, torch.from_numpy(bits.view(np.int16)).cuda(), codes, scales, bsc)
    torch.cuda.synchronize()
    gc, gs = codes.cpu().numpy(), scales.cpu().numpy()
    if afmt == "fp8":
        rc, rs = Q.e4m3_rows(x)
        assert np.array_equal(gs.view(np.uint32), rs.view(np.uint32)), (gs, rs)
        for t in range(T):
            assert np.array_equal(gc[t], rc[t]), (exps[t], np.count_nonzero(gc[t] != rc[t]))
        return
    rc, rsc = Q.mxfp8_rows(x) if afmt == "mxfp8" else Q.mxfp4_quantize(x)
    for t in range(T):
        assert np.array_equal(gc[t], rc[t]), exps[t]
    assert np.array_equal(mx_scales_canonical(bsc.cpu().numpy(), H), rsc)


def test_quantize_tokens_bf16_unsupported():
    import torch

    import mixed_precision_moe_topk_amd as M

    d = M.LayerDims(8, 256, 256, "mxfp4", "bf16")
    h = torch.zeros((4, 256), dtype=torch.int16, device="cuda")
    c = torch.empty((4, 256), dtype=torch.uint8, device="cuda")
    s = torch.empty(4, dtype=torch.float32, device="cuda")
    with pytest.raises(M.MoeError) as ei:
        M.quantize_tokens(d, h, c, s)
    assert ei.value.status == 2
