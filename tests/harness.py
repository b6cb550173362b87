"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI,
run the CPU oracle on the same seeded inputs, compare stage by stage."""
from __future__ import annotations

import numpy as np

import moe_inputs as MI
import oracle as O
from oracle import formats as F
from oracle import quant as Q


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / den) if den > 0 else float(np.linalg.norm(a))


def check_output(out_bits, ref_bits, rel=2e-3, maxabs=2e-2):
    """The output contract: bf16 out vs the oracle's bf16 out, relative L2
    <= 2e-3 and max |diff| <= 2e-2 * max |ref|."""
    a = F.bf16_to_f32(out_bits).astype(np.float64)
    b = F.bf16_to_f32(ref_bits).astype(np.float64)
    assert np.all(np.isfinite(a))
    r = rel_l2(a, b)
    m = float(np.max(np.abs(a - b))) if a.size else 0.0
    bound = maxabs * (float(np.max(np.abs(b))) if b.size else 0.0)
    assert r <= rel, f"rel-L2 {r:.3e} > {rel}"
    assert m <= bound + 1e-30, f"max-abs {m:.3e} > {bound:.3e}"
    return r, m


class Problem:
    """Inputs of one workload, its oracle weights and its GPU weights."""

    def __init__(self, wl: MI.Workload, experts_for_oracle=None, logits=None, hidden=None):
        import torch

        import mixed_precision_moe_topk_amd as M
        from mixed_precision_moe_topk_amd.staging import prepare_from_host

        self.wl = wl
        self.dims = M.LayerDims(wl.experts, wl.hidden, wl.inter, wl.wfmt, wl.afmt)
        self.hidden = hidden if hidden is not None else MI.hidden_bf16(wl.seed, wl.tokens, wl.hidden)
        self.logits = logits if logits is not None else MI.router_logits(
            wl.seed, wl.tokens, wl.experts, wl.bias_sigma)
        self.oracle_w = {}
        want = set(range(wl.experts)) if experts_for_oracle is None else set(experts_for_oracle)

        def it():
            for e, w1, w2 in MI.expert_weights_many(wl.seed, range(wl.experts), wl.hidden, wl.inter):
                if e in want:
                    self.oracle_w[e] = O.quantize_expert(w1, w2, wl.wfmt)
                yield e, w1, w2

        self.weights, self.scales = prepare_from_host(self.dims, it())
        self.h_dev = torch.from_numpy(self.hidden.view(np.int16)).cuda()
        self.l_dev = torch.from_numpy(self.logits).cuda()

    def run_gpu(self, rows_of=None, use_arena=False):
        """Runs the layer; returns dict of numpy intermediates + out bits."""
        import torch

        import mixed_precision_moe_topk_amd as M

        wl = self.wl
        T, k = wl.tokens, wl.top_k
        out = torch.empty((T, wl.hidden), dtype=torch.int16, device="cuda")
        if use_arena:
            M.run(self.dims, self.h_dev, self.l_dev, self.weights, self.scales, k, out)
            torch.cuda.synchronize()
            return dict(out=out.cpu().numpy().view(np.uint16))
        L = M.workspace_layout(self.dims, T, k)
        ws = torch.empty(L.total, dtype=torch.uint8, device="cuda")
        M.run_ws(self.dims, self.h_dev, self.l_dev, self.weights, self.scales, k, out, ws)
        torch.cuda.synchronize()
        w = ws.cpu().numpy()
        rows = T * k

        def view(off, dtype, count):
            return w[off:off + count * np.dtype(dtype).itemsize].view(dtype)

        r = dict(out=out.cpu().numpy().view(np.uint16))
        r["ids"] = view(L.ids, np.int32, rows).reshape(T, k)
        r["weights"] = view(L.topk_w, np.float32, rows).reshape(T, k)
        r["offsets"] = view(L.offsets, np.int32, wl.experts + 1)
        r["row_token"] = view(L.row_token, np.int32, rows)
        r["slot_row"] = view(L.slot_row, np.int32, rows).reshape(T, k)
        e4m3 = wl.afmt in ("fp8", "mxfp8")
        e2m1 = wl.afmt == "mxfp4"
        if e4m3 or e2m1:
            hc = wl.hidden // 2 if e2m1 else wl.hidden  # E2M1: two codes per byte
            r["token_codes"] = view(L.tok_codes, np.uint8, T * hc).reshape(T, hc)
            r["token_scales"] = view(L.tok_scales, np.float32, T)
        if wl.afmt in ("mxfp8", "mxfp4"):
            rb = mx_scale_row_bytes(wl.hidden)
            r["token_block_scales"] = mx_scales_canonical(
                view(L.tok_bscales, np.uint8, T * rb).reshape(T, rb), wl.hidden)
            rb = mx_scale_row_bytes(wl.inter)
            r["fc2_block_scales"] = mx_scales_canonical(
                view(L.fc2_bscales, np.uint8, rows * rb).reshape(rows, rb), wl.inter)
        # h is not materialised when GEMM1 quantises the FC2 input itself
        r["fc2_fused"] = bool(L.fc2_fused)
        r["h"] = None if L.fc2_fused else view(L.h, np.float32, rows * wl.inter).reshape(rows, wl.inter)
        qdt = np.uint8 if e4m3 or e2m1 else np.uint16
        ic = wl.inter // 2 if e2m1 else wl.inter
        r["fc2_codes"] = view(L.fc2_codes, qdt, rows * ic).reshape(rows, ic)
        r["fc2_scales"] = view(L.fc2_scales, np.float32, rows)
        r["y2"] = view(L.y2, np.float32, rows * wl.hidden).reshape(rows, wl.hidden)
        r["num_tiles"] = int(view(L.num_tiles, np.int32, 1)[0])
        r["tile_m"] = L.tile_m
        r["gemm_cfg"] = L.gemm_cfg
        tl = view(L.tiles, np.int32, 4 * L.max_tiles).reshape(-1, 4)
        r["tiles"] = tl[:r["num_tiles"], :3].copy()
        return r

    def unpack(self, first: int, count: int):
        import torch

        import mixed_precision_moe_topk_amd as M

        wl = self.wl
        H, I = wl.hidden, wl.inter
        if wl.wfmt == "mxfp4":
            s1 = torch.empty((count, 2 * I, H // 32), dtype=torch.uint8, device="cuda")
            s2 = torch.empty((count, H, I // 32), dtype=torch.uint8, device="cuda")
        else:
            s1 = torch.empty((count, 2 * I, H // 128), dtype=torch.float32, device="cuda")
            s2 = torch.empty((count, H, I // 128), dtype=torch.float32, device="cuda")
        q1 = torch.empty((count, 2 * I, H // 2), dtype=torch.uint8, device="cuda")
        q2 = torch.empty((count, H, I // 2), dtype=torch.uint8, device="cuda")
        M.unpack_weights(self.dims, self.weights, self.scales, first, q1, s1, q2, s2)
        torch.cuda.synchronize()
        return q1.cpu().numpy(), s1.cpu().numpy(), q2.cpu().numpy(), s2.cpu().numpy()

    def run_oracle(self, tokens=None):
        wl = self.wl
        hb, lg = self.hidden, self.logits
        if tokens is not None:
            hb, lg = hb[tokens], lg[tokens]
        return O.forward(hb, lg, wl.top_k, lambda e: self.oracle_w[e], wl.wfmt, wl.afmt)


def mx_scale_row_bytes(cols):
    """Bytes per row of the library's MXFP8 block scales (16 per 512 columns)."""
    return 16 * ((cols + 511) // 512)


def mx_scales_canonical(stored, cols):
    """Library MXFP8 block scales [rows, mx_scale_row_bytes(cols)], kept in the
    matrix cores' order (block b at byte 16*(b//16) + 4*(b%4) + (b//4)%4), as
    the canonical [rows, cols/32] row-major E8M0 codes."""
    b = np.arange(cols // 32)
    return stored[:, 16 * (b >> 4) + 4 * (b & 3) + ((b >> 2) & 3)]


def expected_work_map(offsets, tile_m):
    """GEMM work map from the per-expert row ranges: (expert, row0, nrows) of
    every tile, in expert order; each expert's rows are cut into tile_m-row
    tiles, the last one partial."""
    tiles = [(e, int(offsets[e]) + r, min(tile_m, int(offsets[e + 1] - offsets[e]) - r))
             for e in range(len(offsets) - 1)
             for r in range(0, int(offsets[e + 1] - offsets[e]), tile_m)]
    return np.array(tiles, np.int32).reshape(-1, 3)


def compare_all(g, r, wl, exact_rows=True):
    """Stage-by-stage comparison of GPU results g with oracle results r."""
    assert np.array_equal(g["ids"], r["ids"]), "routing ids differ"
    assert np.max(np.abs(g["weights"] - r["weights"])) <= 1e-6
    assert np.array_equal(g["offsets"], r["offsets"].astype(np.int32))
    assert np.array_equal(g["tiles"], expected_work_map(r["offsets"], g["tile_m"])), "work map differs"
    if exact_rows:
        assert np.array_equal(g["row_token"], r["row_token"].astype(np.int32))
        assert np.array_equal(g["slot_row"], r["slot_row"].astype(np.int32))
    if wl.afmt == "fp8":
        assert np.array_equal(g["token_codes"], r["token_codes"]), "token E4M3 codes differ"
        assert np.array_equal(g["token_scales"].view(np.uint32), r["token_scales"].view(np.uint32))
    if wl.afmt in ("mxfp8", "mxfp4"):
        assert np.array_equal(g["token_codes"], r["token_codes"]), "token element codes differ"
        assert np.array_equal(g["token_block_scales"], r["token_block_scales"]), "token E8M0 differ"
    if g["h"] is not None:
        assert rel_l2(g["h"], r["h"]) <= 1e-4, rel_l2(g["h"], r["h"])
    if wl.afmt == "fp8":
        # The FC2 codes and row scales are the oracle's per-row E4M3
        # quantiser applied to the GPU's own h, bit for bit (h itself is
        # checked against the oracle's above: it differs by float32
        # accumulation rounding, so against the oracle's codes a few differ)
        qc, qs = Q.e4m3_rows(g["h"])
        assert np.array_equal(g["fc2_codes"], qc), np.count_nonzero(g["fc2_codes"] != qc)
        assert np.array_equal(g["fc2_scales"].view(np.uint32), qs.view(np.uint32))
        same = np.mean(g["fc2_codes"] == r["fc2_codes"])
        assert same > 0.97, same
    if g["h"] is not None and wl.afmt in ("mxfp8", "mxfp4", "bf16"):
        # h stored (the separate FC2 quantiser ran): its bytes are the
        # oracle's quantiser applied to the GPU's own h, bit for bit
        if wl.afmt == "bf16":
            assert np.array_equal(g["fc2_codes"], F.bf16_rne(g["h"])), "FC2 bf16 bits"
        else:
            quant = Q.mxfp8_rows if wl.afmt == "mxfp8" else Q.mxfp4_quantize
            qc, qs = quant(g["h"])
            assert np.array_equal(g["fc2_codes"], qc), np.count_nonzero(g["fc2_codes"] != qc)
            assert np.array_equal(g["fc2_block_scales"], qs), "FC2 E8M0 codes"
    if wl.afmt in ("mxfp8", "mxfp4"):
        # secondary check against the oracle's own FC2 input (quantised from
        # the oracle's h): codes (and, rarely, a block exponent at a
        # power-of-two boundary) differ where h rounds differently
        same = np.mean(g["fc2_codes"] == r["fc2_codes"])
        assert same > 0.97, same
        assert np.mean(g["fc2_block_scales"] == r["fc2_block_scales"]) > 0.99
        dec = Q.mxfp8_decode if wl.afmt == "mxfp8" else Q.mxfp4_decode
        dq = dec(g["fc2_codes"], g["fc2_block_scales"])
        dr = dec(r["fc2_codes"], r["fc2_block_scales"])
        assert rel_l2(dq, dr) <= 1e-3
    if wl.afmt == "bf16":
        # secondary check against the oracle's own bf16(h): h differs from
        # the oracle's by float32 rounding, so a few values round to the
        # neighbouring bf16
        same = np.mean(g["fc2_codes"] == r["fc2_codes"])
        assert same > 0.97, same
        assert rel_l2(F.bf16_to_f32(g["fc2_codes"]), F.bf16_to_f32(r["fc2_codes"])) <= 1e-3
    assert rel_l2(g["y2"], r["y2"]) <= 2e-3, rel_l2(g["y2"], r["y2"])
    # the output is the oracle's finalize of the GPU's own weights and y2
    # rows, bit for bit (float32 products and slot-order sum, one bf16
    # rounding); against the oracle's own output it is within the contract
    fo = O.finalize(g["weights"], g["y2"], g["slot_row"])[0]
    assert np.array_equal(g["out"], fo), np.count_nonzero(g["out"] != fo)
    return check_output(g["out"], r["out"])
