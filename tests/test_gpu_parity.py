"""GPU parity of the HIP path against the CPU oracle, stage by stage, on seeded
inputs at sizes the oracle finishes in seconds (several tiles, ragged tails,
every GEMM tile configuration and every format combination)."""
import numpy as np
import pytest

import moe_inputs as MI
from tests.harness import Problem, check_output, compare_all

pytestmark = pytest.mark.gpu

SMALL = [
    # (tokens, experts, top_k, hidden, inter, wfmt, afmt, seed, bias)  GEMM cfg by rows/expert
    (70, 6, 3, 384, 256, "mxfp4", "fp8", 11, 0.0),    # 35 rows/expert -> 48-row tiles
    (70, 6, 3, 384, 256, "mxfp4", "bf16", 12, 0.0),
    (70, 6, 3, 384, 256, "int4", "fp8", 13, 0.0),
    (300, 5, 2, 256, 384, "mxfp4", "fp8", 14, 0.0),   # 120 rows/expert -> 160-row tiles, tails
    (300, 5, 2, 256, 384, "int4", "fp8", 15, 2.0),
    (300, 5, 2, 256, 384, "mxfp4", "bf16", 16, 2.0),
    (400, 4, 2, 384, 384, "mxfp4", "fp8", 21, 0.0),   # 200 rows/expert, full + ragged tiles, N tail
    (400, 4, 2, 384, 640, "int4", "fp8", 22, 1.0),
    (9, 40, 4, 512, 128, "mxfp4", "fp8", 17, 0.0),    # <1 row/expert -> 16-row tiles, empties
    (9, 40, 4, 512, 128, "mxfp4", "bf16", 18, 0.0),
    (9, 40, 4, 512, 128, "int4", "fp8", 19, 0.0),
    (1, 3, 3, 128, 128, "mxfp4", "fp8", 20, 0.0),     # single token, k = E
    (40, 1024, 16, 128, 128, "mxfp4", "fp8", 24, 0.0),  # the most experts and the largest top-k
    (6, 1, 1, 8320, 4224, "mxfp4", "fp8", 23, 0.0),   # rows longer than the quantisers keep in registers
    (70, 6, 2, 256, 3072, "int4", "fp8", 25, 0.0),   # FC2 rows of 2048-4096 columns (requant, 16 float4 per lane)
    # MXFP8 activations: every tile configuration, K not a multiple of 512
    # (a partial 4-step scale group), ragged row and N tails
    (70, 6, 3, 384, 256, "mxfp4", "mxfp8", 31, 0.0),  # 64-row tiles
    (300, 5, 2, 256, 384, "mxfp4", "mxfp8", 32, 2.0), # 160-row tiles, tails
    (400, 4, 2, 384, 640, "mxfp4", "mxfp8", 33, 1.0), # full + ragged 160-row tiles, N tail
    (9, 40, 4, 512, 128, "mxfp4", "mxfp8", 34, 0.0),  # 16-row tiles, empty experts
    (6, 1, 1, 8320, 4224, "mxfp4", "mxfp8", 35, 0.0), # long rows, 17 scale groups (last partial)
    # K steps past whole 4-step groups: 6 and 7 (one full group, then a
    # remainder of 2 or 3 steps) in both GEMMs
    (300, 5, 2, 768, 896, "mxfp4", "mxfp8", 36, 1.0),
    (300, 5, 2, 896, 768, "mxfp4", "fp8", 37, 0.0),
    # several 160-row M-tiles per expert and several 512-column N-tiles in
    # both GEMMs (N tails of 256 columns in GEMM2 for H = 1280)
    (900, 6, 2, 1536, 512, "mxfp4", "fp8", 38, 0.0),
    (1500, 3, 2, 2048, 1536, "mxfp4", "fp8", 39, 0.0),
    (700, 5, 2, 1280, 1024, "mxfp4", "mxfp8", 40, 0.0),
    (600, 8, 2, 1536, 512, "int4", "fp8", 41, 0.0),
    # 2048+ tokens: the finalize's one-block-per-token form (top-2, top-6 and
    # the generic top-3 kernel) and a routing index over several 16-chunk
    # groups, the last one partial
    (2100, 8, 2, 256, 128, "mxfp4", "fp8", 42, 0.0),
    (2500, 16, 6, 128, 128, "mxfp4", "bf16", 43, 1.0),
    (2200, 12, 3, 128, 256, "int4", "fp8", 44, 0.0),
    # W4A4 (MXFP4 activations): every tile configuration, partial scale groups
    (70, 6, 3, 384, 256, "mxfp4", "mxfp4", 51, 0.0),  # 64-row tiles
    (300, 5, 2, 256, 384, "mxfp4", "mxfp4", 52, 2.0), # 160-row tiles, tails
    (400, 4, 2, 384, 640, "mxfp4", "mxfp4", 53, 1.0), # full + ragged 160-row tiles, N tail
    (9, 40, 4, 512, 128, "mxfp4", "mxfp4", 54, 0.0),  # 16-row tiles, empty experts
    (6, 1, 1, 8320, 4224, "mxfp4", "mxfp4", 55, 0.0), # long rows
    (900, 6, 2, 1536, 512, "mxfp4", "mxfp4", 56, 0.0), # several M- and N-tiles
]


@pytest.mark.parametrize("case", SMALL, ids=[f"T{c[0]}E{c[1]}k{c[2]}H{c[3]}I{c[4]}-{c[5]}x{c[6]}" for c in SMALL])
def test_small_layer_matches_oracle(case):
    T, E, k, H, I, wf, af, seed, bias = case
    wl = MI.small_workload(T, E, k, H, I, wf, af, seed, bias)
    p = Problem(wl)
    g = p.run_gpu()
    r = p.run_oracle()
    rel, mx = compare_all(g, r, wl)
    print(f"{wl.key} tile_m={g['tile_m']} tiles={g['num_tiles']} rel-L2={rel:.2e} max-abs={mx:.2e}")
    # prepared weight codes and scales are bit-identical to the oracle's quantiser
    q1, s1, q2, s2 = p.unpack(0, E)
    for e in range(E):
        ow = p.oracle_w[e]
        assert np.array_equal(q1[e], ow.w1q) and np.array_equal(q2[e], ow.w2q), e
        assert np.array_equal(s1[e].view(np.uint8), np.ascontiguousarray(ow.w1s).view(np.uint8)), e
        assert np.array_equal(s2[e].view(np.uint8), np.ascontiguousarray(ow.w2s).view(np.uint8)), e


def test_tiny_workload_all_stages():
    """The 16-token, 8-expert, top-2, hidden 256, intermediate 512 MXFP4 x FP8 layer."""
    wl = MI.WORKLOADS["tiny_mxfp4_fp8"]
    p = Problem(wl)
    g = p.run_gpu()
    r = p.run_oracle()
    compare_all(g, r, wl)
    # deterministic: a second run gives identical bits everywhere
    g2 = p.run_gpu()
    for key in ("out", "h", "y2", "row_token", "fc2_codes"):
        assert np.array_equal(g[key], g2[key]), key
    # the library-managed workspace form gives the same output
    g3 = p.run_gpu(use_arena=True)
    assert np.array_equal(g3["out"], g["out"])


def test_trace_gemm1_only():
    """GEMM1-only tracing times GEMM1 and leaves every other stage at zero;
    full tracing times every stage."""
    import mixed_precision_moe_topk_amd as M

    wl = MI.WORKLOADS["tiny_mxfp4_fp8"]
    p = Problem(wl, experts_for_oracle=[])
    M.trace_read()  # forget anything recorded before
    M.trace_enable(M.TRACE_GEMM1)
    p.run_gpu()
    M.trace_enable(M.TRACE_OFF)
    calls, st = M.trace_read()
    assert calls == 1 and st["gemm1"] > 0
    assert all(v == 0 for k, v in st.items() if k != "gemm1")
    M.trace_enable(M.TRACE_ALL)
    p.run_gpu()
    M.trace_enable(M.TRACE_OFF)
    calls, st = M.trace_read()
    assert calls == 1 and all(v > 0 for k, v in st.items() if k != "quant" or wl.afmt == "fp8")


@pytest.mark.parametrize("T", [96, 40])  # chunked routing kernels / single-block kernel
@pytest.mark.parametrize("E,k", [(8, 2), (64, 6), (256, 8), (384, 6), (1024, 16)])
def test_router_ties_bit_exact(E, k, T):
    """Logits drawn from few values force exact ties at the top-k boundary;
    ids must follow the lower-index rule exactly."""
    rng = np.random.default_rng(E * 31 + k)
    pool = np.float32([-2.0, -0.5, -0.0, 0.0, 0.5, 0.5, 1.25, 3.0])
    logits = rng.choice(pool, size=(T, E)).astype(np.float32)
    wl = MI.small_workload(T, E, k, 128, 128, "mxfp4", "fp8", 40 + k)
    p = Problem(wl, experts_for_oracle=[], logits=logits)
    g = p.run_gpu()
    import oracle as O
    ids, w = O.route(logits, k)
    assert np.array_equal(g["ids"], ids)
    assert np.max(np.abs(g["weights"] - w)) <= 1e-6
    off, tok, slot, slot_row = O.expand(ids, E)
    assert np.array_equal(g["offsets"], off.astype(np.int32))
    assert np.array_equal(g["row_token"], tok.astype(np.int32))
    assert np.array_equal(g["slot_row"], slot_row.astype(np.int32))


@pytest.mark.parametrize("af,lo,hi", [("fp8", -20, 20), ("bf16", -20, 20), ("mxfp8", -4, 4),
                                      ("mxfp4", -6, 6)])
def test_zero_and_extreme_token_rows(af, lo, hi):
    """Token rows that are all zero (amax = 0: token scale 1 / E8M0 code 127),
    a zero 32-element block inside a row, and rows scaled by 2^lo and 2^hi
    (exact in bf16), through every stage; each group of rows is checked
    against its own magnitude."""
    from oracle import formats as F

    wl = MI.small_workload(48, 6, 2, 256, 256, "mxfp4", af, 61, 0.0)
    x = F.bf16_to_f32(MI.hidden_bf16(wl.seed, wl.tokens, wl.hidden)).copy()
    x[0] = 0.0
    x[1] = -0.0
    x[2, :32] = 0.0
    x[3:10] *= np.float32(2.0 ** lo)
    x[10:17] *= np.float32(2.0 ** hi)
    hb = F.bf16_rne(x)
    assert np.array_equal(F.bf16_to_f32(hb), x)
    p = Problem(wl, hidden=hb)
    g = p.run_gpu()
    r = p.run_oracle()
    compare_all(g, r, wl)
    assert np.all(F.bf16_to_f32(g["out"][:2]) == 0.0)
    for rows in (slice(2, 3), slice(3, 10), slice(10, 17), slice(17, 48)):
        check_output(g["out"][rows], r["out"][rows])


@pytest.mark.parametrize("wf,af", [("mxfp4", "bf16"), ("int4", "fp8"), ("mxfp4", "mxfp8"),
                                   ("mxfp4", "mxfp4")])
def test_library_workspace_matches_caller_workspace(wf, af):
    """moe_run (workspace kept by the library per device and stream, grown on
    demand) gives the same bits as moe_run_ws, also after a smaller and a
    larger call on the same stream."""
    import torch

    import mixed_precision_moe_topk_amd as M

    outs = []
    for T in (40, 8, 130):
        wl = MI.small_workload(T, 6, 2, 256, 256, wf, af, 81, 0.5)
        p = Problem(wl, experts_for_oracle=[])
        ref = p.run_gpu()["out"]
        out = torch.empty((T, wl.hidden), dtype=torch.int16, device="cuda")
        M.run(p.dims, p.h_dev, p.l_dev, p.weights, p.scales, wl.top_k, out)
        torch.cuda.synchronize()
        outs.append((ref, out.cpu().numpy().view(np.uint16)))
    for ref, got in outs:
        assert np.array_equal(ref, got)


def test_empty_batch_is_noop():
    import torch

    import mixed_precision_moe_topk_amd as M

    d = M.LayerDims(8, 256, 512, "mxfp4", "fp8")
    wb, sb = M.weights_query(d)
    w = torch.zeros(wb, dtype=torch.uint8, device="cuda")
    s = torch.zeros(sb, dtype=torch.uint8, device="cuda")
    h = torch.zeros((0, 256), dtype=torch.int16, device="cuda")
    lg = torch.zeros((0, 8), dtype=torch.float32, device="cuda")
    out = torch.zeros((0, 256), dtype=torch.int16, device="cuda")
    M.run_ws(d, h, lg, w, s, 2, out, None)
    M.run(d, h, lg, w, s, 2, out)
    torch.cuda.synchronize()
