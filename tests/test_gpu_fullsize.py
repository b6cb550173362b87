"""GPU parity at the full DeepSeek-V3 / V4-Pro sizes, in the launch
configuration the benchmark times: routing ids, expert row maps and E4M3
token codes for every token (bit-exact); prepared weight codes for sampled
experts (bit-exact); SwiGLU output, GEMM2 output and the bf16 layer output
for a sample of tokens, computed one by one by the oracle (the layer is
independent per token), within the output contract.

Only experts that receive tokens are prepared (the others are never read)."""
import numpy as np
import pytest

import moe_inputs as MI
import oracle as O
from oracle import formats as F
from tests.harness import Problem, check_output, expected_work_map, rel_l2

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

CASES = ["dsv3_decode_mxfp4_bf16", "dsv3_int4_fp8", "dsv3_prefill_mxfp4_fp8",
         "dsv4pro_prefill_mxfp4_fp8", "dsv3_prefill_mxfp4_mxfp8", "dsv3_prefill_mxfp4_mxfp4"]
SAMPLE = 3  # tokens checked against the oracle end to end


class ActiveProblem(Problem):
    """Problem whose device weights cover only the experts with routed rows."""

    def __init__(self, wl, sample_tokens):
        import torch

        import mixed_precision_moe_topk_amd as M

        self.wl = wl
        self.dims = M.LayerDims(wl.experts, wl.hidden, wl.inter, wl.wfmt, wl.afmt)
        self.hidden = MI.hidden_bf16(wl.seed, wl.tokens, wl.hidden)
        self.logits = MI.router_logits(wl.seed, wl.tokens, wl.experts, wl.bias_sigma)
        ids, _ = O.route(self.logits, wl.top_k)
        self.ref_ids = ids
        active = sorted(set(ids.reshape(-1).tolist()))
        want = set(ids[sample_tokens].reshape(-1).tolist()) | {active[0], active[-1]}
        self.oracle_w = {}
        wb, sb = M.weights_query(self.dims)
        self.weights = torch.zeros(wb, dtype=torch.uint8, device="cuda")
        self.scales = torch.zeros(sb, dtype=torch.uint8, device="cuda")
        g1 = torch.empty((1, 2 * wl.inter, wl.hidden), dtype=torch.float32, device="cuda")
        g2 = torch.empty((1, wl.hidden, wl.inter), dtype=torch.float32, device="cuda")
        for e, w1, w2 in MI.expert_weights_many(wl.seed, active, wl.hidden, wl.inter):
            if e in want:
                self.oracle_w[e] = O.quantize_expert(w1, w2, wl.wfmt)
            g1[0].copy_(torch.from_numpy(w1))
            g2[0].copy_(torch.from_numpy(w2))
            M.prepare_weights(self.dims, g1, g2, e, self.weights, self.scales)
        torch.cuda.synchronize()
        self.active = active
        self.h_dev = torch.from_numpy(self.hidden.view(np.int16)).cuda()
        self.l_dev = torch.from_numpy(self.logits).cuda()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", CASES)
def test_fullsize_sampled(name):
    wl = MI.WORKLOADS[name]
    rng = np.random.default_rng(wl.seed)
    sample = np.sort(rng.choice(wl.tokens, size=SAMPLE, replace=False))
    p = ActiveProblem(wl, sample)
    g = p.run_gpu()
    print(f"{name}: tile_m={g['tile_m']} tiles={g['num_tiles']} active={len(p.active)}")
    # routing and row maps for every token
    assert np.array_equal(g["ids"], p.ref_ids)
    off, tok, slot, slot_row = O.expand(p.ref_ids, wl.experts)
    assert np.array_equal(g["offsets"], off.astype(np.int32))
    assert np.array_equal(g["row_token"], tok.astype(np.int32))
    assert np.array_equal(g["slot_row"], slot_row.astype(np.int32))
    # GEMM work map (main and tail tiles) from the expert row ranges
    assert np.array_equal(g["tiles"], expected_work_map(off, g["tile_m"]))
    # E4M3 token codes and their scales (per token, or E8M0 per 32) for every token
    if wl.afmt == "fp8":
        q, s = O.quant.e4m3_rows(F.bf16_to_f32(p.hidden))
        assert np.array_equal(g["token_codes"], q)
        assert np.array_equal(g["token_scales"].view(np.uint32), s.view(np.uint32))
    if wl.afmt in ("mxfp8", "mxfp4"):
        quant = O.quant.mxfp8_rows if wl.afmt == "mxfp8" else O.quant.mxfp4_quantize
        q, sx = quant(F.bf16_to_f32(p.hidden))
        assert np.array_equal(g["token_codes"], q)
        assert np.array_equal(g["token_block_scales"], sx)
    # prepared weight codes of two experts
    for e in (p.active[0], p.active[-1]):
        q1, s1, q2, s2 = p.unpack(e, 1)
        ow = p.oracle_w[e]
        assert np.array_equal(q1[0], ow.w1q) and np.array_equal(q2[0], ow.w2q)
        assert np.array_equal(s1[0].view(np.uint8), np.ascontiguousarray(ow.w1s).view(np.uint8))
        assert np.array_equal(s2[0].view(np.uint8), np.ascontiguousarray(ow.w2s).view(np.uint8))
    # sampled tokens end to end
    r = p.run_oracle(tokens=sample)
    rows = g["slot_row"][sample].reshape(-1)
    ref_rows = r["slot_row"].reshape(-1)
    if g["h"] is not None:
        assert rel_l2(g["h"][rows], r["h"][ref_rows]) <= 1e-4
    assert rel_l2(g["y2"][rows], r["y2"][ref_rows]) <= 2e-3
    rel, mx = check_output(g["out"][sample], r["out"])
    print(f"{name}: sampled tokens {sample.tolist()} rel-L2 {rel:.2e} max-abs {mx:.2e}")
