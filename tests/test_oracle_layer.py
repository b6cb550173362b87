"""Pins of the oracle's layer: brute-force router, exact rational GEMMs, a
hand-derived single-expert example, reductions (E=1/k=1, identical experts),
per-token independence and empty inputs (CPU only)."""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import moe_inputs as MI
import oracle as O
from oracle import formats as F
from oracle import quant as Q


def frac_to_f32(fr: Fraction) -> float:
    """Exact rational -> nearest float32 (ties to even), by integer arithmetic."""
    if fr == 0:
        return 0.0
    sign = -1.0 if fr < 0 else 1.0
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)                      # subnormals share the 2^-149 quantum
    m = a / Fraction(2) ** (e - 23)       # in [2^23, 2^24) for normals
    fl = math.floor(m)
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * float(np.float32(math.ldexp(fl, e - 23)))


def _make_experts(seed, e_num, hidden, inter, wfmt):
    out = {}
    for e, w1, w2 in MI.expert_weights_many(seed, range(e_num), hidden, inter, threads=4):
        out[e] = O.quantize_expert(w1, w2, wfmt)
    return out


# ----------------------------------------------------------------------------- router

def test_router_brute_force_with_ties():
    rng = np.random.default_rng(12)
    for trial in range(300):
        e = int(rng.integers(2, 9))
        k = int(rng.integers(1, e + 1))
        # few distinct values -> many exact ties; include -0.0 and 0.0
        pool = np.float32([-1.5, -0.0, 0.0, 0.25, 0.25, 1.0, 2.0])
        logits = rng.choice(pool, size=(3, e)).astype(np.float32)
        ids, w = O.route(logits, k)
        for t in range(3):
            l = logits[t]
            valid = []
            for sub in itertools.combinations(range(e), k):
                s = set(sub)
                if all((l[i] > l[j]) or (l[i] == l[j] and i < j) for i in s for j in range(e) if j not in s):
                    valid.append(sub)
            assert len(valid) == 1
            order = sorted(valid[0], key=lambda i: (-float(l[i]), i))
            assert ids[t].tolist() == order, (l, ids[t], order)
            ref = scipy.special.softmax(l[order].astype(np.float64))
            assert np.allclose(w[t], ref, rtol=1e-6, atol=1e-7)


def test_router_invariants():
    rng = np.random.default_rng(1)
    logits = rng.standard_normal((50, 16)).astype(np.float32)
    ids, w = O.route(logits, 1)
    assert np.all(w == 1.0)
    assert np.array_equal(ids[:, 0], np.argmax(logits, axis=1))
    ids, w = O.route(logits, 16)
    full = scipy.special.softmax(logits.astype(np.float64), axis=1)
    assert np.allclose(w, np.take_along_axis(full, ids.astype(np.int64), 1), rtol=1e-6)
    ids, w = O.route(logits, 5)
    assert np.all(np.diff(w, axis=1) <= 0)
    assert np.allclose(w.sum(1), 1.0, atol=1e-6)
    assert all(len(set(r)) == 5 for r in ids.tolist())
    # permuting expert columns permutes the ids (no ties in N(0,1) draws)
    perm = rng.permutation(16)
    ids_p, w_p = O.route(logits[:, perm], 5)
    assert np.array_equal(perm[ids_p], ids) and np.array_equal(w_p, w)


def test_expand_structure():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((40, 10)).astype(np.float32)
    ids, _ = O.route(logits, 3)
    off, tok, slot, slot_row = O.expand(ids, 10)
    assert off[0] == 0 and off[-1] == 120
    assert np.array_equal(np.diff(off), np.bincount(ids.reshape(-1), minlength=10))
    for e in range(10):
        r = np.arange(off[e], off[e + 1])
        assert np.all(ids[tok[r], slot[r]] == e)
        assert np.all(np.diff(tok[r]) > 0)
    assert np.array_equal(slot_row[tok, slot], np.arange(120))


# ----------------------------------------------------------------------------- exact GEMMs

@pytest.mark.parametrize("wfmt,afmt", [("mxfp4", "fp8"), ("mxfp4", "bf16"), ("int4", "fp8"),
                                       ("mxfp4", "mxfp8"), ("mxfp4", "mxfp4")])
def test_gemms_against_exact_rationals(wfmt, afmt):
    wl = MI.small_workload(tokens=3, experts=4, top_k=2, hidden=128, inter=128,
                           wfmt=wfmt, afmt=afmt, seed=77)
    hb = MI.hidden_bf16(wl.seed, wl.tokens, wl.hidden)
    lg = MI.router_logits(wl.seed, wl.tokens, wl.experts)
    ex = _make_experts(wl.seed, wl.experts, wl.hidden, wl.inter, wfmt)
    r = O.forward(hb, lg, wl.top_k, lambda e: ex[e], wfmt, afmt, keep_y1=True)
    x = F.bf16_to_f32(hb)
    if afmt == "fp8":
        a_dec = [[Fraction(float(v)) for v in F.e4m3_decode(row)] for row in r["token_codes"]]
    elif afmt == "mxfp8":
        # element times 2^(code - 127) of its 32-element block, as exact rationals
        a_dec = [[Fraction(float(F.e4m3_decode(c))) * Fraction(2) ** (int(sc[i // 32]) - 127)
                  for i, c in enumerate(row)]
                 for row, sc in zip(r["token_codes"], r["token_block_scales"])]
    elif afmt == "mxfp4":
        a_dec = [[Fraction(float(F.e2m1_decode(c))) * Fraction(2) ** (int(sc[i // 32]) - 127)
                  for i, c in enumerate(F.unpack_nibbles(row[None])[0])]
                 for row, sc in zip(r["token_codes"], r["token_block_scales"])]
    else:
        a_dec = [[Fraction(float(v)) for v in row] for row in x]
    off = r["offsets"]
    mism = 0
    total = 0
    for e in range(wl.experts):
        if off[e + 1] == off[e]:
            continue
        w1 = O.layer.decode_weight(ex[e].w1q, ex[e].w1s, wfmt)
        w2 = O.layer.decode_weight(ex[e].w2q, ex[e].w2s, wfmt)
        w1f = [[Fraction(float(v)) for v in row] for row in w1]
        w2f = [[Fraction(float(v)) for v in row] for row in w2]
        for row in range(off[e], off[e + 1]):
            t = r["row_token"][row]
            s = Fraction(float(r["token_scales"][t]))
            for n in range(0, 2 * wl.inter, 7):
                acc = sum(a * b for a, b in zip(a_dec[t], w1f[n]))
                exp = frac_to_f32(acc * s)
                got = float(r["y1"][row, n])
                total += 1
                if got != exp:
                    mism += 1
                    assert abs(got - exp) <= abs(exp) * 2.0 ** -23, (row, n, got, exp)
            if afmt == "fp8":
                a2 = [Fraction(float(v)) for v in F.e4m3_decode(r["fc2_codes"][row])]
            elif afmt == "mxfp8":
                sc2 = r["fc2_block_scales"][row]
                a2 = [Fraction(float(F.e4m3_decode(c))) * Fraction(2) ** (int(sc2[i // 32]) - 127)
                      for i, c in enumerate(r["fc2_codes"][row])]
            elif afmt == "mxfp4":
                sc2 = r["fc2_block_scales"][row]
                a2 = [Fraction(float(F.e2m1_decode(c))) * Fraction(2) ** (int(sc2[i // 32]) - 127)
                      for i, c in enumerate(F.unpack_nibbles(r["fc2_codes"][row][None])[0])]
            else:
                a2 = [Fraction(float(v)) for v in F.bf16_to_f32(r["fc2_codes"][row])]
            s2 = Fraction(float(r["fc2_scales"][row]))
            for n in range(0, wl.hidden, 5):
                acc = sum(a * b for a, b in zip(a2, w2f[n]))
                exp = frac_to_f32(acc * s2)
                got = float(r["y2"][row, n])
                total += 1
                if got != exp:
                    mism += 1
                    assert abs(got - exp) <= abs(exp) * 2.0 ** -23, (row, n, got, exp)
    assert mism <= max(1, total // 100)


def test_fp64_gemm_is_order_independent():
    wl = MI.small_workload(tokens=8, experts=2, top_k=1, hidden=2048, inter=256, seed=5)
    hb = MI.hidden_bf16(wl.seed, wl.tokens, wl.hidden)
    q, s = Q.e4m3_rows(F.bf16_to_f32(hb))
    w1, _ = MI.expert_weights(wl.seed, 0, wl.hidden, wl.inter)
    wq, ws = Q.mxfp4_quantize(w1)
    a = F.e4m3_decode(q)
    w = Q.mxfp4_decode(wq, ws)
    r1 = a @ w.T
    r2 = a[:, ::-1] @ w[:, ::-1].T
    r3 = sum(a[:, i::7] @ w[:, i::7].T for i in range(7))
    assert np.array_equal(r1, r2) and np.array_equal(r1, r3)


# ----------------------------------------------------------------------------- whole layer

def test_hand_derived_single_expert():
    """T=1, E=1, k=1, H=32, I=32, MXFP4 x FP8; values chosen so every step is
    derivable by hand.  gate rows 0.5, up rows 0.25 (up row 0: -0.25),
    W2 rows 1.0 (even n) / 0.5 (odd n), hidden all 1.0."""
    h, i = 32, 32
    hb = F.bf16_rne(np.ones((1, h), dtype=np.float32))
    w1 = np.concatenate([np.full((i, h), 0.5), np.full((i, h), 0.25)]).astype(np.float32)
    w1[i] = -0.25
    w2 = np.where(np.arange(h)[:, None] % 2 == 0, 1.0, 0.5) * np.ones((h, i))
    ew = O.quantize_expert(w1, w2.astype(np.float32), "mxfp4")
    r = O.forward(hb, np.zeros((1, 1), dtype=np.float32), 1, lambda e: ew, "mxfp4", "fp8")
    s = frac_to_f32(Fraction(1, 448))                # token scale = amax/448
    assert float(r["token_scales"][0]) == s
    assert np.all(r["token_codes"] == 0x7E)          # 1/s rounds to 448
    g = frac_to_f32(Fraction(448 * 32) * Fraction(0.5) * Fraction(s))
    u = frac_to_f32(Fraction(448 * 32) * Fraction(0.25) * Fraction(s))
    hv = float(np.float32(g / (1.0 + math.exp(-g)) * u))
    exp_h = np.full(i, hv, dtype=np.float32)
    exp_h[0] = -hv
    assert np.array_equal(r["h"][0], exp_h)
    s2 = frac_to_f32(Fraction(hv) / 448)
    assert float(r["fc2_scales"][0]) == s2
    assert r["fc2_codes"][0, 0] == 0xFE and np.all(r["fc2_codes"][0, 1:] == 0x7E)
    acc_even = Fraction(448 * 30)                    # 31 positive, 1 negative
    y_even = frac_to_f32(acc_even * Fraction(s2))
    y_odd = frac_to_f32(acc_even / 2 * Fraction(s2))
    exp_y = np.where(np.arange(h) % 2 == 0, y_even, y_odd).astype(np.float32)
    assert np.array_equal(r["y2"][0], exp_y)
    assert np.array_equal(r["out"][0], F.bf16_rne(exp_y))


def _torch_mxfp8(x):
    """MXFP8 of float32 rows with torch ops: per 32-element block X from the
    exact binary exponent of the block's amax (torch.frexp), E4M3 codes of
    x / 2^X, returned decoded (float64)."""
    r, c = x.shape
    b = x.reshape(r, c // 32, 32).double()
    amax = b.abs().amax(dim=-1)
    _, e = torch.frexp(torch.where(amax > 0, amax, torch.ones_like(amax)))
    xe = torch.where(amax > 0, e.double() - 1 - 8, torch.zeros_like(amax)).clamp(-127, 127)
    v = (b / torch.pow(2.0, xe)[..., None]).numpy()
    dec = torch.from_numpy(F.e4m3_decode(F.e4m3_encode(v)))
    return (dec * torch.pow(2.0, xe)[..., None]).reshape(r, c)


def _torch_mxfp4(x):
    """MXFP4 of float32 rows with torch ops: per 32-element block X =
    floor(log2 amax) - 2 (torch.frexp), each x / 2^X rounded to the nearest
    E2M1 magnitude {0, .5, 1, 1.5, 2, 3, 4, 6} (ties to the even code,
    saturating at 6), returned decoded (float64)."""
    r, c = x.shape
    b = x.reshape(r, c // 32, 32).double()
    amax = b.abs().amax(dim=-1)
    _, e = torch.frexp(torch.where(amax > 0, amax, torch.ones_like(amax)))
    xe = torch.where(amax > 0, e.double() - 1 - 2, torch.zeros_like(amax)).clamp(min=-127)
    v = b / torch.pow(2.0, xe)[..., None]
    grid = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=torch.float64)
    dist = (v.abs().clamp(max=6.0)[..., None] - grid).abs()
    dist = dist + 1e-12 * (torch.arange(8) % 2).double()  # exact ties -> even code
    mag = grid[dist.argmin(dim=-1)]
    return (torch.sign(v) * mag * torch.pow(2.0, xe)[..., None]).reshape(r, c)


@pytest.mark.parametrize("wfmt,afmt", [("mxfp4", "fp8"), ("mxfp4", "bf16"), ("int4", "fp8"),
                                       ("mxfp4", "mxfp8"), ("mxfp4", "mxfp4")])
def test_single_expert_equals_independent_mlp(wfmt, afmt):
    """E = 1, k = 1: out = bf16(MLP(x)) computed here with torch float64 ops on
    the decoded operands (an independent composition of the steps)."""
    wl = MI.small_workload(tokens=9, experts=1, top_k=1, hidden=256, inter=128,
                           wfmt=wfmt, afmt=afmt, seed=21)
    hb = MI.hidden_bf16(wl.seed, wl.tokens, wl.hidden)
    lg = MI.router_logits(wl.seed, wl.tokens, 1)
    ex = _make_experts(wl.seed, 1, wl.hidden, wl.inter, wfmt)[0]
    r = O.forward(hb, lg, 1, lambda e: ex, wfmt, afmt)
    assert np.all(r["weights"] == 1.0)
    x = torch.from_numpy(F.bf16_to_f32(hb).copy())
    if afmt == "fp8":
        amax = x.abs().amax(dim=1)
        s = amax / 448.0                             # float32 tensor division
        a = torch.from_numpy(F.e4m3_decode(F.e4m3_encode((x / s[:, None]).numpy())))
    elif afmt == "mxfp8":
        s = torch.ones(wl.tokens)
        a = _torch_mxfp8(x)
    elif afmt == "mxfp4":
        s = torch.ones(wl.tokens)
        a = _torch_mxfp4(x)
    else:
        s = torch.ones(wl.tokens)
        a = x.double()
    w1 = torch.from_numpy(O.layer.decode_weight(ex.w1q, ex.w1s, wfmt))
    w2 = torch.from_numpy(O.layer.decode_weight(ex.w2q, ex.w2s, wfmt))
    y1 = (torch.matmul(a, w1.t()) * s.double()[:, None]).float()
    g, u = y1[:, :wl.inter].double(), y1[:, wl.inter:].double()
    hh = (torch.nn.functional.silu(g) * u).float()
    if afmt == "fp8":
        s2 = hh.abs().amax(dim=1) / 448.0
        a2 = torch.from_numpy(F.e4m3_decode(F.e4m3_encode((hh / s2[:, None]).numpy())))
    elif afmt == "mxfp8":
        s2 = torch.ones(wl.tokens)
        a2 = _torch_mxfp8(hh)
    elif afmt == "mxfp4":
        s2 = torch.ones(wl.tokens)
        a2 = _torch_mxfp4(hh)
    else:
        s2 = torch.ones(wl.tokens)
        a2 = hh.to(torch.bfloat16).double()
    y2 = (torch.matmul(a2, w2.t()) * s2.double()[:, None]).float()
    ref = y2.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # torch's silu may differ from exp-based silu by an ulp -> allow 1 bf16 ulp
    diff = np.abs(r["out"].astype(np.int64) - ref.astype(np.int64))
    assert diff.max() <= 1 and np.mean(diff == 0) > 0.97


def test_identical_experts_reduce_to_one_expert():
    wl = MI.small_workload(tokens=12, experts=5, top_k=3, hidden=128, inter=128, seed=8)
    hb = MI.hidden_bf16(wl.seed, wl.tokens, wl.hidden)
    lg = MI.router_logits(wl.seed, wl.tokens, wl.experts)
    ex = _make_experts(wl.seed, 1, wl.hidden, wl.inter, "mxfp4")[0]
    many = O.forward(hb, lg, 3, lambda e: ex, "mxfp4", "fp8")
    one = O.forward(hb, lg[:, :1], 1, lambda e: ex, "mxfp4", "fp8")
    assert np.array_equal(one["out"], F.bf16_rne(one["y2"][one["slot_row"][:, 0]]))
    a = F.bf16_to_f32(many["out"]).astype(np.float64)
    b = F.bf16_to_f32(one["out"]).astype(np.float64)
    assert np.all(np.abs(a - b) <= np.abs(b) * 2.0 ** -7 + 1e-30)


def test_per_token_independence_and_empty():
    wl = MI.small_workload(tokens=20, experts=6, top_k=2, hidden=128, inter=128, seed=31)
    hb = MI.hidden_bf16(wl.seed, wl.tokens, wl.hidden)
    lg = MI.router_logits(wl.seed, wl.tokens, wl.experts, bias_sigma=2.0)
    ex = _make_experts(wl.seed, wl.experts, wl.hidden, wl.inter, "mxfp4")
    full = O.forward(hb, lg, 2, lambda e: ex[e], "mxfp4", "fp8")
    sub = [3, 7, 19]
    part = O.forward(hb[sub], lg[sub], 2, lambda e: ex[e], "mxfp4", "fp8")
    assert np.array_equal(part["out"], full["out"][sub])
    empty = O.forward(hb[:0], lg[:0], 2, lambda e: ex[e], "mxfp4", "fp8")
    assert empty["out"].shape == (0, wl.hidden)


def test_router_nan_logits_rank_as_minus_infinity():
    """Reading for non-finite logits (the pages are silent): NaN ranks as
    -inf.  Brute force over all k-subsets of the logits with NaN replaced
    by -inf (ties by the smaller index), ids always valid; an all-NaN row
    selects experts 0..k-1 with NaN weights (softmax of -inf - -inf)."""
    rng = np.random.default_rng(77)
    for trial in range(200):
        e = int(rng.integers(2, 9))
        k = int(rng.integers(1, e + 1))
        pool = np.float32([np.nan, -np.inf, -1.0, 0.0, 0.5, 0.5, 2.0])
        logits = rng.choice(pool, size=(2, e)).astype(np.float32)
        ids, w = O.route(logits, k)
        for t in range(2):
            key = [(-np.inf if np.isnan(x) else float(x)) for x in logits[t]]
            best = None
            for sub in itertools.combinations(range(e), k):
                s = set(sub)
                if all(key[i] > key[j] or (key[i] == key[j] and i < j)
                       for i in s for j in range(e) if j not in s):
                    best = sorted(sub, key=lambda i: (-key[i], i))
            assert ids[t].tolist() == best
            if np.isfinite(key[best[0]]):
                sel = np.array([key[i] for i in best])
                ref = np.exp(sel - sel[0]) / np.exp(sel - sel[0]).sum()
                assert np.allclose(w[t], ref, rtol=1e-6, atol=1e-7)
            else:
                assert np.all(np.isnan(w[t]))
    ids, w = O.route(np.full((1, 6), np.nan, np.float32), 3)
    assert ids[0].tolist() == [0, 1, 2] and np.all(np.isnan(w))


def test_finalize_pairs_each_slot_weight_with_its_own_expert_row():
    """The router-weighted top-k sum (the finalize of the pages'
    grouped-GEMM + finalize fusion, token_final_scales): with distinct
    experts and k = 3, out[t] = bf16(sum_j fl32(w_tj * y2_{e_tj}(x_t))) in
    float32 and slot order, where the weights come from scipy's softmax over
    the brute-force top-k logits and each (token, expert) MLP is composed
    here with torch float64 ops on the decoded weights, not through
    oracle.forward.  Any other pairing of slot weights with expert rows must
    miss the tolerance, so a pairing error in the oracle fails this test."""
    T, E, k, H, I = 6, 5, 3, 64, 64
    wl = MI.small_workload(tokens=T, experts=E, top_k=k, hidden=H, inter=I, seed=41)
    hb = MI.hidden_bf16(wl.seed, T, H)
    lg = MI.router_logits(wl.seed, T, E)
    ex = _make_experts(wl.seed, E, H, I, "mxfp4")
    r = O.forward(hb, lg, k, lambda e: ex[e], "mxfp4", "fp8")

    # per-token quantised activations, independent of the oracle's quantiser
    x = torch.from_numpy(F.bf16_to_f32(hb).copy())
    s = x.abs().amax(dim=1) / 448.0
    a = torch.from_numpy(F.e4m3_decode(F.e4m3_encode((x / s[:, None]).numpy())))

    def mlp(t, e):
        w1 = torch.from_numpy(O.layer.decode_weight(ex[e].w1q, ex[e].w1s, "mxfp4"))
        w2 = torch.from_numpy(O.layer.decode_weight(ex[e].w2q, ex[e].w2s, "mxfp4"))
        y1 = (torch.matmul(a[t:t + 1], w1.t()) * float(s[t])).float()
        hh = (torch.nn.functional.silu(y1[:, :I].double()) * y1[:, I:].double()).float()
        s2 = hh.abs().amax(dim=1) / 448.0
        a2 = torch.from_numpy(F.e4m3_decode(F.e4m3_encode((hh / s2[:, None]).numpy())))
        return (torch.matmul(a2, w2.t()) * s2.double()[:, None]).float().numpy()[0]

    sel, wts = [], []
    for t in range(T):
        order = sorted(range(E), key=lambda i: (-float(lg[t, i]), i))[:k]
        sel.append(order)
        wts.append(scipy.special.softmax(lg[t, order].astype(np.float64)).astype(np.float32))
    y2 = {(t, j): mlp(t, sel[t][j]) for t in range(T) for j in range(k)}
    assert len({tuple(v) for v in sel}) > 1 and all(len(set(v)) == k for v in sel)

    def combine(perm):
        out = np.zeros((T, H), np.float32)
        for t in range(T):
            acc = np.zeros(H, np.float32)
            for j in range(k):
                acc = (acc + (wts[t][j] * y2[(t, perm[j])]).astype(np.float32)).astype(np.float32)
            out[t] = acc
        return F.bf16_rne(out)

    def close(a_bits, b_bits):
        # torch's silu may differ from the oracle's exp-based one by an ulp
        d = np.abs(a_bits.astype(np.int64) - b_bits.astype(np.int64))
        return d.max() <= 1 and np.mean(d == 0) > 0.97

    assert np.array_equal(r["ids"], np.array(sel, np.int32))
    assert close(r["out"], combine(list(range(k))))
    for perm in itertools.permutations(range(k)):
        if list(perm) != list(range(k)):
            assert not close(r["out"], combine(list(perm))), perm


def test_finalize_rounds_each_product_to_float32_before_adding():
    """The finalize keeps the sum in float32 and rounds each weighted term
    to float32 before the add (no fused multiply-add, no wider sum).  Here
    w0 * y0 = (1 + 2^-12)^2 = 1 + 2^-11 + 2^-24 is a float32 tie that rounds
    to 1 + 2^-11 (even mantissa), which the second slot cancels exactly: the
    float32 sum is 0, while a fused multiply-add or a float64 sum leaves
    2^-24 (bf16 0x3380)."""
    a = np.float32(1 + 2.0 ** -12)
    w = np.array([[a, 1.0]], dtype=np.float32)
    y2 = np.array([[a], [-(1 + 2.0 ** -11)]], dtype=np.float32)
    slot_row = np.array([[0, 1]])
    out, acc = O.finalize(w, y2, slot_row)
    assert acc.dtype == np.float32 and acc[0, 0] == 0.0
    assert out[0, 0] == 0
    assert F.bf16_rne(np.array([2.0 ** -24], dtype=np.float32))[0] == 0x3380
    # slot order: the same terms in the other order give the same sum here,
    # and a three-term case where order matters follows the slots
    w3 = np.array([[1.0, 1.0, 1.0]], dtype=np.float32)
    y3 = np.array([[2.0 ** 24], [1.0], [-(2.0 ** 24)]], dtype=np.float32)
    _, acc3 = O.finalize(w3, y3, np.array([[0, 1, 2]]))
    assert acc3[0, 0] == 0.0  # (2^24 + 1) rounds to 2^24 in float32, then cancels
    _, acc3b = O.finalize(w3, y3, np.array([[0, 2, 1]]))
    assert acc3b[0, 0] == 1.0
