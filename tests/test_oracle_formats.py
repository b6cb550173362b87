"""Pins of the oracle's number formats against the OCP code tables and against
brute-force nearest-value search (CPU only)."""
import math

import numpy as np
import pytest
import torch

from oracle import formats as F
from tests.conftest import parse_value, read_golden


def _golden(fmt):
    return [(int(c, 16), parse_value(v)) for f, c, v in read_golden("format_codes.txt") if f == fmt]


@pytest.mark.parametrize("fmt,dec", [("e4m3", F.e4m3_decode), ("e2m1", F.e2m1_decode),
                                     ("e8m0", F.e8m0_decode)])
def test_code_tables_match_spec(fmt, dec):
    rows = _golden(fmt)
    assert rows
    for code, val in rows:
        got = float(dec(np.array([code]))[0])
        if math.isnan(val):
            assert math.isnan(got), (fmt, hex(code))
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), (fmt, hex(code), got, val)


def _brute_nearest(x, values, codes, even_of, sat):
    """Brute force: distance to every finite code, min distance, ties to the
    code with even mantissa, |x| beyond sat clamps; sign from x."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), sat)
    mags = np.abs(values)
    d = np.abs(a[:, None] - mags[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    # among candidates prefer even mantissa, then the smaller magnitude code
    score = np.where(cand, 0, 10) + np.where(even_of[None, :], 0, 1)
    pick = np.argmin(score, axis=1)
    return codes[pick], np.signbit(x)


def _e4m3_brute(x):
    codes = np.arange(0x7F)  # non-negative finite codes
    vals = F.E4M3_TABLE[codes]
    c, neg = _brute_nearest(x, vals, codes, (codes & 1) == 0, 448.0)
    return (c | (neg.astype(np.int64) << 7)).astype(np.uint8)


def _e4m3_test_values():
    rng = np.random.default_rng(7)
    # every finite bf16 value (covers all binades, sign, zero, subnormals)
    b = np.arange(1 << 16, dtype=np.uint32)
    b = b[((b >> 7) & 0xFF) != 0xFF]
    vals = [(b << 16).view(np.float32)]
    # exact midpoints between adjacent codes and one float32 ulp around them
    pos = F.E4M3_TABLE[:0x7F]
    mid = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    vals += [mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9))]
    vals += [np.float32([448, 448.5, 464, 464.1, 480, 1e6, 3.4e38])]
    # random float32 spread over the range and a log-uniform sample
    vals.append(rng.standard_normal(200000).astype(np.float32) * np.float32(50))
    vals.append((np.exp(rng.uniform(-30, 7, 200000)) * rng.choice([-1, 1], 200000)).astype(np.float32))
    v = np.concatenate(vals).astype(np.float32)
    return np.concatenate([v, -v])


def test_e4m3_encoder_equals_brute_force():
    x = _e4m3_test_values()
    got = F.e4m3_encode(x)
    for i in range(0, x.size, 20000):
        exp = _e4m3_brute(x[i:i + 20000])
        bad = np.nonzero(got[i:i + 20000] != exp)[0]
        assert bad.size == 0, (x[i + bad[0]], hex(got[i + bad[0]]), hex(exp[bad[0]]))


def test_e4m3_roundtrip_and_signed_zero():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(F.e4m3_encode(F.e4m3_decode(codes)), codes)
    assert F.e4m3_encode(np.float32([-1e-9, -0.0]))[0] == 0x80
    assert F.e4m3_encode(np.float32([-0.0]))[0] == 0x80
    # ties: 2^-10 is halfway between 0 and 2^-9 -> even (0); 17 between 16 and 18 -> 16
    assert F.e4m3_encode(np.float32([2.0 ** -10, 17.0, 19.0, 464.0]))[:4].tolist() == [0x00, 0x58, 0x5A, 0x7E]


def test_e2m1_encoder_equals_brute_force():
    rng = np.random.default_rng(3)
    grid = F.E2M1_MAG
    mids = (grid[:-1] + grid[1:]) / 2
    x = np.concatenate([rng.uniform(-8, 8, 100000), mids, -mids, np.nextafter(mids, 0),
                        np.nextafter(mids, 10), grid, -grid, [6.5, 7.99, 100.0, -100.0, -0.0]])
    codes = np.arange(8)
    c, neg = _brute_nearest(x, grid, codes, (codes & 1) == 0, 6.0)
    exp = (c | (neg.astype(np.int64) << 3)).astype(np.uint8)
    assert np.array_equal(F.e2m1_encode(x), exp)


def test_bf16_rne_matches_torch_cast():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(300000).astype(np.float32) * 100,
                        (np.arange(1 << 16, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
                        (np.arange(1 << 16, dtype=np.uint32) << 16 | 0x7FFF).view(np.float32),
                        (np.arange(1 << 16, dtype=np.uint32) << 16 | 0x8001).view(np.float32)])
    x = x[np.isfinite(x) & (np.abs(x) < 3e38)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.bf16_rne(x), ref)


def test_nibble_order():
    # element 2i in the low nibble, 2i+1 in the high nibble
    assert F.pack_nibbles(np.array([[1, 2, 3, 4]], dtype=np.uint8)).tolist() == [[0x21, 0x43]]
    rng = np.random.default_rng(0)
    c = rng.integers(0, 16, (5, 64)).astype(np.uint8)
    assert np.array_equal(F.unpack_nibbles(F.pack_nibbles(c)), c)


def test_int4_decode_range():
    assert F.int4_decode(np.arange(16)).tolist() == [0, 1, 2, 3, 4, 5, 6, 7, -8, -7, -6, -5, -4, -3, -2, -1]
