"""The E4M3 quantisers on the device replace the IEEE quotient fl32(x / s)
by x * fl32(1 / s) except near E4M3 rounding midpoints (within 2 ulp), below
2^-6 and for non-finite products, where they take the IEEE quotient.  This
checks that rule in NumPy float32 arithmetic (round-to-nearest multiply and
divide, as on the device): wherever the product is kept, it encodes to the
same E4M3 code as the IEEE quotient.  Inputs: random scales and elements,
quotients placed on and within a few ulp of every E4M3 midpoint, and scales
down to the subnormal range (CPU only)."""
import numpy as np

from oracle import formats as F


def rule(x, s):
    x = x.astype(np.float32)
    s = s.astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        inv = (np.float32(1.0) / s).astype(np.float32)
        q = (x * inv).astype(np.float32)
        exact = (x / s).astype(np.float32)
    a = q.view(np.uint32) & np.uint32(0x7FFFFFFF)
    t = a & np.uint32(0xFFFFF)
    fallback = (a < 0x3C800000) | (a >= 0x7F800000) | (np.abs(t.astype(np.int64) - 0x80000) <= 2)
    return q, exact, fallback


def check(x, s):
    q, exact, fb = rule(x, s)
    keep = ~fb
    qc = F.e4m3_encode(np.clip(q[keep], -448, 448))
    ec = F.e4m3_encode(np.clip(exact[keep], -448, 448))
    bad = np.flatnonzero(qc != ec)
    assert bad.size == 0, (x[keep][bad[:5]], s[keep][bad[:5]])
    return keep.mean()


def test_random_quotients():
    rng = np.random.default_rng(5)
    n = 2_000_000
    amax = np.abs(rng.standard_normal(n)).astype(np.float32) * np.float32(4) + np.float32(1e-3)
    s = (amax / np.float32(448)).astype(np.float32)
    x = (rng.uniform(-1, 1, n) * amax).astype(np.float32)
    assert check(x, s) > 0.99


def test_quotients_at_and_around_every_midpoint():
    """For every E4M3 midpoint M (normal range) and random s: x = fl32(M s)
    and its neighbours a few ulp away, so x / s lands on or next to M."""
    codes = np.arange(0x08, 0x7E, dtype=np.uint8)
    v = F.e4m3_decode(codes).astype(np.float64)
    nxt = F.e4m3_decode(codes + 1).astype(np.float64)
    mids = ((v + nxt) / 2).astype(np.float32)
    rng = np.random.default_rng(6)
    s = (np.abs(rng.standard_normal(4096)) / 448 + 1e-6).astype(np.float32)
    xs, ss = [], []
    for m in mids:
        base = (m * s).astype(np.float32)
        for d in range(-6, 7):
            xs.append((base.view(np.int32) + d).view(np.float32))
            ss.append(s)
    x = np.concatenate(xs)
    s_all = np.concatenate(ss)
    x = np.concatenate([x, -x])
    s_all = np.concatenate([s_all, s_all])
    check(x, s_all)
    _, _, fb = rule(x, s_all)
    assert fb.mean() > 0.1  # the near-midpoint cases do take the exact quotient


def test_tiny_and_subnormal_scales():
    rng = np.random.default_rng(7)
    for e in (-100, -119, -122, -126, -128, -131, -140):
        amax = np.float32(2.0 ** e) * np.float32(1.7)
        s = np.full(100_000, amax / np.float32(448), np.float32)
        x = (rng.uniform(-1, 1, s.size) * amax).astype(np.float32)
        check(x, s)
