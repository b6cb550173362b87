"""GPU parity at the full DeepSeek-V3 / V4-Pro sizes, in the launch
configuration the benchmark times: routing ids, expert row maps and E4M3
token codes for every token (bit-exact); prepared weight codes for sampled
experts (bit-exact); the per-token E4M3 FC2 codes of every row against the
oracle's quantiser of the GPU's h (bit-exact); SwiGLU and GEMM2 output of
chosen rows (every row of the last, partial M-tile and of the second 16-row
group of the first tile, for the hottest, the coldest and random experts:
the tile tails and the second wave row), against the oracle's pass of that
one expert; the whole h and y2 rows of the last row of every active expert
(every expert's last M-tile, every N-tile of both GEMMs); the finalize of
every token from the GPU's own weights and y2 (bit-exact); and the bf16
layer output for random tokens, computed token by token by the oracle (the
layer is independent per token), within the output contract.

Only experts that receive tokens are prepared (the others are never read)."""
import numpy as np
import pytest

import moe_inputs as MI
import oracle as O
from oracle import formats as F
from tests import oracle_rows as OR
from tests.harness import Problem, check_output, expected_work_map, rel_l2

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

CASES = ["dsv3_decode_mxfp4_bf16", "dsv3_int4_fp8", "dsv3_prefill_mxfp4_fp8",
         "dsv4pro_prefill_mxfp4_fp8", "dsv3_prefill_mxfp4_mxfp8", "dsv3_prefill_mxfp4_mxfp4"]
SAMPLE = 3  # tokens checked against the oracle end to end
CHECK_EXPERTS = 6  # experts whose tile tails are checked row by row


class ActiveProblem(Problem):
    """Problem whose device weights cover only the experts with routed rows."""

    def __init__(self, wl, sample_tokens, extra_experts=()):
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
        want |= set(extra_experts)
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
    # experts whose tile tails are checked: the hottest, the coldest, random
    logits = MI.router_logits(wl.seed, wl.tokens, wl.experts, wl.bias_sigma)
    counts = np.bincount(O.route(logits, wl.top_k)[0].reshape(-1), minlength=wl.experts)
    act = np.flatnonzero(counts)
    chk = {int(act[np.argmax(counts[act])]), int(act[np.argmin(counts[act])])}
    chk |= set(rng.choice(act, size=CHECK_EXPERTS, replace=False).tolist())
    chk = sorted(chk)[:CHECK_EXPERTS + 2]
    p = ActiveProblem(wl, sample, chk)
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
    # the finalize of every token: the oracle's finalize applied to the GPU's
    # own weights and y2 rows, bit for bit
    assert np.array_equal(g["out"], O.finalize(g["weights"], g["y2"], g["slot_row"])[0])
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
    # per-token E4M3 FC2 input of every row: the oracle's quantiser of the
    # GPU's h, bit for bit
    if wl.afmt == "fp8":
        qc, qs = O.quant.e4m3_rows(g["h"])
        assert np.array_equal(g["fc2_codes"], qc)
        assert np.array_equal(g["fc2_scales"].view(np.uint32), qs.view(np.uint32))
    # FC2 input written by GEMM1's epilogue (MX formats, BF16): equal, bit
    # for bit, to the separate quantiser's output on the stored h, which is
    # the oracle's quantiser applied to that h
    if wl.afmt in ("mxfp8", "mxfp4", "bf16"):
        import mixed_precision_moe_topk_amd as M

        assert g["fc2_fused"]
        M.set_fc2_fused(False)
        try:
            gu = p.run_gpu()
        finally:
            M.set_fc2_fused(True)
        if wl.afmt == "bf16":
            assert np.array_equal(gu["fc2_codes"], F.bf16_rne(gu["h"]))
        else:
            quant = O.quant.mxfp8_rows if wl.afmt == "mxfp8" else O.quant.mxfp4_quantize
            qc, qs = quant(gu["h"])
            assert np.array_equal(gu["fc2_codes"], qc)
            assert np.array_equal(gu["fc2_block_scales"], qs)
            assert np.array_equal(g["fc2_block_scales"], gu["fc2_block_scales"])
        assert np.array_equal(g["fc2_codes"], gu["fc2_codes"])
        assert np.array_equal(g["out"], gu["out"])
        g["h"] = gu["h"]
        del gu
    # tile tails of chosen experts: every row of the last (partial) M-tile and
    # of rows 16-31 of the first tile (the second wave row), against the
    # oracle's pass of that one expert over those rows' tokens
    tm = g["tile_m"]
    for e in chk:
        r0, r1 = int(off[e]), int(off[e + 1])
        last = r0 + ((r1 - r0 - 1) // tm) * tm
        rows_e = sorted(set(range(last, r1)) | set(range(min(r0 + 16, r1), min(r0 + 32, r1))))
        toks = np.unique(tok[rows_e])
        sub = O.forward(p.hidden[toks], p.logits[toks], wl.top_k, lambda x: p.oracle_w[x],
                        wl.wfmt, wl.afmt, only_experts={e})
        ti, tj = np.nonzero(sub["ids"] == e)
        grow = g["slot_row"][toks[ti], tj]
        orow = sub["slot_row"][ti, tj]
        if g["h"] is not None:
            assert rel_l2(g["h"][grow], sub["h"][orow]) <= 1e-4, e
        assert rel_l2(g["y2"][grow], sub["y2"][orow]) <= 2e-3, e
        print(f"{name}: expert {e} ({r1 - r0} rows, tile_m {tm}): {len(grow)} tail rows checked")
    # the last row of every active expert (a row of its last, partial M-tile),
    # whole h and y2 rows, so every GEMM1 and GEMM2 N-tile of every expert has
    # a checked row; the oracle's expert passes run in worker processes
    last_rows = [int(off[e + 1]) - 1 for e in p.active]
    jobs = [(name, e, p.hidden[[tok[r]]], p.logits[[tok[r]]]) for e, r in zip(p.active, last_rows)]
    got_h, got_y2, ref_h, ref_y2 = [], [], [], []
    for (e, h_ref, y2_ref), r in zip(OR.expert_rows_many(jobs), last_rows):
        got_y2.append(g["y2"][r])
        ref_y2.append(y2_ref[0])
        # a wrong row or tile is off by O(1); the bound leaves room for an
        # FC2 code that flipped on h's float32 rounding
        assert rel_l2(g["y2"][r], y2_ref[0]) <= 2e-2, (e, r)
        if g["h"] is not None:
            got_h.append(g["h"][r])
            ref_h.append(h_ref[0])
            assert rel_l2(g["h"][r], h_ref[0]) <= 1e-4, (e, r)
    assert rel_l2(np.stack(got_y2), np.stack(ref_y2)) <= 2e-3
    if got_h:
        assert rel_l2(np.stack(got_h), np.stack(ref_h)) <= 1e-4
    print(f"{name}: last rows of all {len(p.active)} active experts checked")
    # sampled tokens end to end
    r = p.run_oracle(tokens=sample)
    rows = g["slot_row"][sample].reshape(-1)
    ref_rows = r["slot_row"].reshape(-1)
    if g["h"] is not None:
        assert rel_l2(g["h"][rows], r["h"][ref_rows]) <= 1e-4
    assert rel_l2(g["y2"][rows], r["y2"][ref_rows]) <= 2e-3
    rel, mx = check_output(g["out"][sample], r["out"])
    print(f"{name}: sampled tokens {sample.tolist()} rel-L2 {rel:.2e} max-abs {mx:.2e}")
