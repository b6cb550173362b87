"""The fused MoE layer, step by step, on the CPU (float64 accumulation).

TEST INFRASTRUCTURE ONLY: only tests, the smoke check and the benchmark's CPU
baseline may call this module; the GPU path never does.

The layer is the one flashinfer PR #3738 ("perf: optimize MXFP4xBF16 & INT4xFP8
and add MXFP4xFP8 CUTLASS MoE backend for SM90") builds: its Description and
Implementation Notes name runtime per-token FP8 activation quantisation during
row expansion, grouped GEMMs over MXFP4 or INT4 expert weights against FP8 or
BF16 activations with per-token-scale epilogues, and the activation step
between the GEMMs; PR #4793 ("Unify MoE CuTe DSL dispatch to be dtype
agnostic") passes top-k expert ids and their final scales (token_final_scales)
and fuses the router-weighted reduction into a finalize step after GEMM2.

Steps, each rounded only at its storage point:
  route     top-k by float32 logit (ties -> lower expert index), weights =
            softmax over the k selected logits (float64 exp), stored float32.
  quantize  per-token E4M3 (FP8 activations), MXFP8 (E4M3 with one E8M0
            scale per 32 elements of a token; the token scale is then 1),
            MXFP4 (W4A4: E2M1 with one E8M0 scale per 32, the weights' own
            quantiser; PR #4793's walkthrough passes an MXFP4 activation pack
            and its scales to the fused MoE in its w4a4 mode) or the bf16
            values (BF16).
  expand    rows grouped by expert, then token, then slot.
  gemm1     acc = A . W1^T exactly in float64; y1 = fl32(acc * token scale).
  swiglu    h = fl32(silu(gate) * up), gate = y1[:, :I], up = y1[:, I:],
            silu(g) = g / (1 + exp(-g)).
  fc2 input FP8: per-row E4M3 of h (same quantiser as the tokens);
            MXFP8 / MXFP4: per-row MXFP8 / MXFP4 of h (row scale 1); BF16:
            bf16(h), scale 1.
  gemm2     acc2 = A2 . W2^T in float64; y2 = fl32(acc2 * row scale).
  finalize  out[t] = bf16(sum_j fl32(w[t,j] * y2[row(t,j)])), the sum kept
            in float32 and taken in slot order.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable

import numpy as np

from . import formats as F
from . import quant as Q


def route(logits: np.ndarray, top_k: int):
    """logits float32 [T, E] -> (ids int32 [T, k], weights float32 [T, k]).

    The pages say nothing of non-finite logits.  Reading taken here (and by
    the GPU router): a NaN logit ranks as -inf, so every id stays a valid
    expert index; infinite logits rank as their values.  When the largest
    selected logit is infinite the softmax is undefined and the weights come
    out NaN (exp(inf - inf))."""
    logits = np.asarray(logits, dtype=np.float32)
    logits = np.where(np.isnan(logits), np.float32(-np.inf), logits)
    t, e = logits.shape
    assert 1 <= top_k <= e
    idx = np.broadcast_to(np.arange(e), (t, e))
    # lexsort: the last key is the primary one; -logit ascending == logit
    # descending; equal logits keep ascending expert index.
    order = np.lexsort((idx, -logits.astype(np.float64)), axis=-1)
    ids = order[:, :top_k].astype(np.int32)
    sel = np.take_along_axis(logits, ids.astype(np.int64), axis=1).astype(np.float64)
    with np.errstate(invalid="ignore"):  # inf - inf: undefined softmax -> NaN weights
        p = np.exp(sel - sel[:, :1])
        w = (p / p.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, w


def expand(ids: np.ndarray, num_experts: int):
    """Group the T*k (token, slot) pairs by expert.

    Returns (offsets int64 [E+1], row_token int64 [rows], row_slot int64 [rows],
    slot_row int64 [T, k]) where rows [offsets[e], offsets[e+1]) belong to
    expert e in ascending (token, slot) order and slot_row[t, j] is the row of
    pair (t, j)."""
    t, k = ids.shape
    flat = ids.reshape(-1).astype(np.int64)
    order = np.argsort(flat, kind="stable")  # flat index t*k+j is ascending
    counts = np.bincount(flat, minlength=num_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    slot_row = np.empty(t * k, dtype=np.int64)
    slot_row[order] = np.arange(t * k)
    return offsets, order // k, order % k, slot_row.reshape(t, k)


@dataclass
class ExpertWeights:
    """Canonical packed weights of one expert.

    MXFP4: w1q uint8 [2I, H/2], w1s uint8 [2I, H/32], w2q uint8 [H, I/2],
           w2s uint8 [H, I/32].
    INT4:  same codes, w1s float32 [2I, H/128], w2s float32 [H, I/128]."""

    w1q: np.ndarray
    w1s: np.ndarray
    w2q: np.ndarray
    w2s: np.ndarray


def quantize_expert(w1: np.ndarray, w2: np.ndarray, wfmt: str) -> ExpertWeights:
    if wfmt == "mxfp4":
        a, b = Q.mxfp4_quantize(w1)
        c, d = Q.mxfp4_quantize(w2)
    elif wfmt == "int4":
        a, b = Q.int4_quantize(w1)
        c, d = Q.int4_quantize(w2)
    else:
        raise ValueError(wfmt)
    return ExpertWeights(a, b, c, d)


def decode_weight(codes, scales, wfmt: str) -> np.ndarray:
    if wfmt == "mxfp4":
        return Q.mxfp4_decode(codes, scales)
    return Q.int4_decode(codes, scales)


def silu_mul(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    g = g.astype(np.float64)
    return (g / (1.0 + np.exp(-g)) * u.astype(np.float64)).astype(np.float32)


def finalize(w: np.ndarray, y2: np.ndarray, slot_row: np.ndarray):
    """The router-weighted top-k reduction after GEMM2 (PR #4793, the
    finalize step that consumes token_final_scales): out[t] =
    bf16(sum_j fl32(w[t,j] * y2[slot_row[t,j]])), each product rounded to
    float32 and the sum kept in float32, taken in slot order.  w float32
    [T, k], y2 float32 [rows, H], slot_row [T, k].  Returns (bf16 bits
    uint16 [T, H], the float32 sum)."""
    t, k = w.shape
    acc = np.zeros((t, y2.shape[1]), dtype=np.float32)
    for j in range(k if t else 0):
        term = (w[:, j:j + 1] * y2[slot_row[:, j]]).astype(np.float32)
        acc = (acc + term).astype(np.float32)
    return F.bf16_rne(acc), acc


def forward(hidden_bits: np.ndarray, logits: np.ndarray, top_k: int,
            expert_fn: Callable[[int], ExpertWeights], wfmt: str, afmt: str,
            check_exact: bool = True, keep_y1: bool = False,
            only_experts=None) -> dict:
    """Runs the layer.  hidden_bits: bf16 bits uint16 [T, H]; logits float32
    [T, E]; expert_fn(e) returns the canonical weights of expert e (called
    once per expert that receives rows).  Returns every intermediate.

    only_experts (a set of expert ids, or None for all): the expert passes
    (GEMM1, SwiGLU, FC2 input, GEMM2) run for these experts only and the
    rows of the others keep h = y2 = 0; routing, token quantisation and the
    finalize always run over all tokens.  Used to time the oracle on a
    sample of whole experts; the arithmetic of a pass that runs is the
    same."""
    t, h = hidden_bits.shape
    e_num = logits.shape[1]
    ids, w = route(logits, top_k)
    x = F.bf16_to_f32(hidden_bits)
    sx_tok = None
    if afmt == "fp8":
        q, s_tok = Q.e4m3_rows(x)
        a_dec = F.e4m3_decode(q)
    elif afmt == "mxfp8":
        q, sx_tok = Q.mxfp8_rows(x)
        s_tok = np.ones(t, dtype=np.float32)
        a_dec = Q.mxfp8_decode(q, sx_tok)
    elif afmt == "mxfp4":
        # W4A4: activations in the weights' own MXFP4 format (E2M1 elements,
        # E8M0 per 32, the OCP MX rule), packed two codes per byte
        q, sx_tok = Q.mxfp4_quantize(x)
        s_tok = np.ones(t, dtype=np.float32)
        a_dec = Q.mxfp4_decode(q, sx_tok)
    elif afmt == "bf16":
        q, s_tok = None, np.ones(t, dtype=np.float32)
        a_dec = x.astype(np.float64)
    else:
        raise ValueError(afmt)
    offsets, row_tok, row_slot, slot_row = expand(ids, e_num)
    rows = t * top_k
    inter = None
    h_all = y2 = q2 = s2 = sx2 = y1_all = None
    for e in range(e_num):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0 or (only_experts is not None and e not in only_experts):
            continue
        wts = expert_fn(e)
        toks = row_tok[r0:r1]
        w1 = decode_weight(wts.w1q, wts.w1s, wfmt)
        if inter is None:
            inter = w1.shape[0] // 2
            h_all = np.zeros((rows, inter), dtype=np.float32)
            y2 = np.zeros((rows, h), dtype=np.float32)
            q2 = np.zeros((rows, inter // 2 if afmt == "mxfp4" else inter),
                          dtype=np.uint16 if afmt == "bf16" else np.uint8)
            s2 = np.ones(rows, dtype=np.float32)
            if afmt in ("mxfp8", "mxfp4"):
                sx2 = np.full((rows, inter // Q.MX_BLOCK), 127, dtype=np.uint8)
            if keep_y1:
                y1_all = np.zeros((rows, 2 * inter), dtype=np.float32)
        if check_exact and wfmt == "mxfp4" and afmt == "fp8":
            assert Q.mx_exponent_spread(wts.w1s) <= 18 and Q.mx_exponent_spread(wts.w2s) <= 18
        if check_exact and wfmt == "mxfp4" and afmt == "mxfp8":
            assert Q.mx_exponent_spread(wts.w1s) + Q.mx_exponent_spread(sx_tok[toks]) <= 18
        if check_exact and wfmt == "mxfp4" and afmt == "mxfp4":
            # E2M1 x E2M1 products are multiples of 2^(Xa+Xw-2) below 36 * 2^(Xa+Xw):
            # K <= 8192 terms stay exact in float64 for an exponent spread <= 32
            assert Q.mx_exponent_spread(wts.w1s) + Q.mx_exponent_spread(sx_tok[toks]) <= 32
        acc = a_dec[toks] @ w1.T
        y1 = (acc * s_tok[toks][:, None].astype(np.float64)).astype(np.float32)
        if keep_y1:
            y1_all[r0:r1] = y1
        hh = silu_mul(y1[:, :inter], y1[:, inter:])
        h_all[r0:r1] = hh
        if afmt == "fp8":
            qq, ss = Q.e4m3_rows(hh)
            a2 = F.e4m3_decode(qq)
        elif afmt == "mxfp8":
            qq, sxx = Q.mxfp8_rows(hh)
            ss = np.ones(r1 - r0, dtype=np.float32)
            a2 = Q.mxfp8_decode(qq, sxx)
            sx2[r0:r1] = sxx
            if check_exact and wfmt == "mxfp4":
                assert Q.mx_exponent_spread(wts.w2s) + Q.mx_exponent_spread(sxx) <= 18
        elif afmt == "mxfp4":
            qq, sxx = Q.mxfp4_quantize(hh)
            ss = np.ones(r1 - r0, dtype=np.float32)
            a2 = Q.mxfp4_decode(qq, sxx)
            sx2[r0:r1] = sxx
            if check_exact and wfmt == "mxfp4":
                assert Q.mx_exponent_spread(wts.w2s) + Q.mx_exponent_spread(sxx) <= 32
        else:
            qq = F.bf16_rne(hh)
            ss = np.ones(r1 - r0, dtype=np.float32)
            a2 = F.bf16_to_f32(qq).astype(np.float64)
        q2[r0:r1] = qq
        s2[r0:r1] = ss
        w2 = decode_weight(wts.w2q, wts.w2s, wfmt)
        acc2 = a2 @ w2.T
        y2[r0:r1] = (acc2 * ss[:, None].astype(np.float64)).astype(np.float32)
    if y2 is None:  # no expert pass ran (empty batch, or an empty only_experts)
        y2 = np.zeros((rows, h), dtype=np.float32)
    out, acc_out = finalize(w, y2, slot_row)
    return dict(ids=ids, weights=w, token_codes=q, token_scales=s_tok,
                token_block_scales=sx_tok, offsets=offsets, row_token=row_tok,
                row_slot=row_slot, slot_row=slot_row, h=h_all, fc2_codes=q2,
                fc2_scales=s2, fc2_block_scales=sx2, y2=y2, out_f32=acc_out,
                out=out, y1=y1_all)
