"""Pins of the oracle's quantisers: a hand-worked MX block, brute-force scale
search, invariants of MXFP4/INT4/E4M3 quantisation (CPU only)."""
from fractions import Fraction

import numpy as np

from oracle import formats as F
from oracle import quant as Q
from tests.conftest import read_golden


def test_mx_block_hand_example():
    rows = read_golden("mx_block_example.txt")
    assert rows[0][0] == "scale"
    scale = int(rows[0][1])
    vals = [float(v) for v, _ in rows[1:]]
    codes = [int(c, 16) for _, c in rows[1:]]
    w = np.zeros((1, 32), dtype=np.float32)
    w[0, :len(vals)] = vals
    q, s = Q.mxfp4_quantize(w)
    assert int(s[0, 0]) == scale
    got = F.unpack_nibbles(q)[0]
    assert got[:len(codes)].tolist() == codes
    assert np.all(got[len(codes):] == 0)


def _brute_scale(amax):
    # the X with 4 <= amax / 2^X < 8, found by search over all integers
    for x in range(-160, 130):
        r = amax / 2.0 ** x
        if 4.0 <= r < 8.0:
            return max(x, -127)
    raise AssertionError(amax)


def test_mxfp4_scale_and_elements_brute_force():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-20, 20, (64, 1)))).astype(np.float32)
    w[3, 32:64] = 0.0
    w[4, 64:96] = -0.0
    w[5, :32] = np.float32(2.0 ** -140)  # shared exponent below the E8M0 range
    q, s = Q.mxfp4_quantize(w)
    codes = F.unpack_nibbles(q)
    blk = w.reshape(64, 8, 32).astype(np.float64)
    for n in range(64):
        for b in range(8):
            amax = np.max(np.abs(blk[n, b]))
            if amax == 0:
                assert s[n, b] == 127
                exp_codes = np.signbit(blk[n, b]).astype(np.uint8) << 3
            else:
                x = _brute_scale(amax)
                assert s[n, b] == x + 127, (n, b)
                v = blk[n, b] / 2.0 ** x
                # brute force nearest-even on the E2M1 grid
                d = np.abs(np.minimum(np.abs(v), 6.0)[:, None] - F.E2M1_MAG[None, :])
                best = d.min(axis=1, keepdims=True)
                sc = np.where(d == best, 0, 10) + (np.arange(8)[None, :] & 1)
                exp_codes = np.argmin(sc, axis=1).astype(np.uint8) | (np.signbit(v).astype(np.uint8) << 3)
            assert np.array_equal(codes[n, b * 32:(b + 1) * 32], exp_codes), (n, b)
    assert s[5, 0] == 0


def test_mxfp4_invariants():
    rng = np.random.default_rng(9)
    w = (rng.standard_normal((128, 1024)) * 0.02).astype(np.float32)
    q, s = Q.mxfp4_quantize(w)
    mag = F.unpack_nibbles(q) & 7
    bmax = mag.reshape(128, 32, 32).max(axis=-1)
    # amax * 2^-X lies in [4, 8): its code is 4 (value 4) or 6 (value 6) -> codes 6 or 7
    assert np.all(np.isin(bmax, [6, 7]))
    d = Q.mxfp4_decode(q, s)
    # per-element error: half the local grid spacing (<= 1 * 2^X) inside the
    # grid, and up to 2 * 2^X for magnitudes in [6, 8) * 2^X that clamp to 6
    sc = F.e8m0_decode(s).repeat(32, axis=1)
    err = np.abs(d - w)
    inside = np.abs(w) <= 6 * sc
    assert np.all(err[inside] <= sc[inside])
    assert np.all(err <= 2 * sc)
    # decode(encode(decoded)) is a fixed point
    q2, s2 = Q.mxfp4_quantize(d.astype(np.float32))
    assert np.array_equal(q2, q) and np.array_equal(s2, s)


def test_int4_invariants():
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((64, 512)) * 0.02).astype(np.float32)
    w[7, 128:256] = 0
    q, s = Q.int4_quantize(w)
    v = F.int4_decode(F.unpack_nibbles(q)).reshape(64, 4, 128)
    nz = np.abs(w.reshape(64, 4, 128)).max(axis=-1) > 0
    assert np.all(np.abs(v).max(axis=-1)[nz] == 7)
    assert np.all(v >= -7) and np.all(v <= 7)
    assert s[7, 1] == 1.0 and np.all(v[7, 1] == 0)
    err = np.abs(Q.int4_decode(q, s) - w).reshape(64, 4, 128)
    assert np.all(err <= s[..., None].astype(np.float64) * (0.5 + 1e-6))
    # the scale is the float32 quotient amax / 7
    amax = np.abs(w.reshape(64, 4, 128)).max(axis=-1)
    assert np.array_equal(s[nz], (amax / np.float32(7))[nz])


def test_int4_round_half_even_ties():
    """INT4 codes round w/s to the nearest integer with ties to even.  Group
    amax 7 gives s = 7/7 = 1 exactly and amax 3.5 gives s = 0.5, so the
    quotients below are exact half-integers; the expected codes are written
    out by hand (round-half-away would give 3, 1, -1, -3, 5, 7, -7)."""
    w = np.zeros((2, 128), np.float32)
    w[0, :9] = [7.0, 2.5, 0.5, -0.5, -2.5, 4.5, 6.5, -6.5, 1.5]
    w[1, :4] = [3.5, 1.25, -0.75, 0.25]          # s = 0.5: 7, 2.5, -1.5, 0.5
    q, s = Q.int4_quantize(w)
    assert s[0, 0] == 1.0 and s[1, 0] == 0.5
    v = F.int4_decode(F.unpack_nibbles(q))
    assert v[0, :9].tolist() == [7, 2, 0, 0, -2, 4, 6, -6, 2]
    assert v[1, :4].tolist() == [7, 2, -2, 0]
    assert np.all(v[0, 9:] == 0) and np.all(v[1, 4:] == 0)


def test_token_quant_amax_maps_to_448_for_every_bf16_amax():
    b = np.arange(1, 0x7F80, dtype=np.uint32)  # every positive finite bf16
    amax = (b << 16).view(np.float32)
    x = np.stack([amax, -amax * np.float32(0.5), np.zeros_like(amax)], axis=1)
    q, s = Q.e4m3_rows(x)
    assert np.all(q[:, 0] == 0x7E)
    assert np.array_equal(s, amax / np.float32(448))


def test_token_quant_power_of_two_invariance():
    rng = np.random.default_rng(4)
    x = F.bf16_to_f32(F.bf16_rne(rng.standard_normal((16, 512)).astype(np.float32)))
    q0, s0 = Q.e4m3_rows(x)
    for j in (-20, -3, 5, 30):
        q1, s1 = Q.e4m3_rows((x * np.float32(2.0 ** j)).astype(np.float32))
        assert np.array_equal(q0, q1)
        assert np.array_equal(s1, (s0 * np.float32(2.0 ** j)).astype(np.float32))


def test_zero_token_gets_unit_scale():
    q, s = Q.e4m3_rows(np.zeros((2, 64), dtype=np.float32))
    assert np.all(s == 1.0) and np.all(q == 0)


# ----------------------------------------------------------------------------- MXFP8

def _brute_scale8(amax):
    """Largest integer X (clamped to [-127, 127]) with 2^(X + 8) <= amax: the
    OCP MX shared exponent for an E4M3 element (emax 8), found by search."""
    for x in range(127, -128, -1):
        if Fraction(2) ** (x + 8) <= Fraction(float(amax)):
            return x
    return -127


def test_mxfp8_scale_and_elements_brute_force():
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((32, 256)) * np.exp(rng.uniform(-30, 30, (32, 1)))).astype(np.float32)
    x[2, 64:96] = 0.0
    x[3, 96:128] = -0.0
    x[4, :32] = np.float32(2.0 ** -140)   # shared exponent below the E8M0 range -> -127
    x[5, 32:64] = np.float32(448.0 * 2.0 ** 20)  # block amax exactly 448 * 2^20
    q, s = Q.mxfp8_rows(x)
    blk = x.reshape(32, 8, 32).astype(np.float64)
    pos = F.E4M3_TABLE[:0x7F]
    for r in range(32):
        for b in range(8):
            amax = np.max(np.abs(blk[r, b]))
            if amax == 0:
                assert s[r, b] == 127
                exp_codes = np.signbit(blk[r, b]).astype(np.uint8) << 7
            else:
                xe = _brute_scale8(amax)
                assert s[r, b] == xe + 127, (r, b)
                v = blk[r, b] / 2.0 ** xe
                mag = np.minimum(np.abs(v), 448.0)
                d = np.abs(mag[:, None] - pos[None, :])
                best = d.min(axis=1, keepdims=True)
                # nearest, exact ties to the even code (mantissa lsb 0)
                sc = np.where(d == best, 0, 10) + (np.arange(len(pos))[None, :] & 1)
                exp_codes = np.argmin(sc, axis=1).astype(np.uint8) | (np.signbit(v).astype(np.uint8) << 7)
            assert np.array_equal(q[r, b * 32:(b + 1) * 32], exp_codes), (r, b)
    assert s[4, 0] == 0
    assert s[5, 1] == 20 + 127 and np.all(q[5, 32:64] == 0x7E)


def test_mxfp8_invariants():
    rng = np.random.default_rng(17)
    x = rng.standard_normal((64, 1024)).astype(np.float32)
    q, s = Q.mxfp8_rows(x)
    # amax * 2^-X lies in [256, 512): its code decodes to [256, 448]
    bmax = np.abs(F.e4m3_decode(q)).reshape(64, 32, 32).max(axis=-1)
    assert np.all((bmax >= 256) & (bmax <= 448))
    d = Q.mxfp8_decode(q, s)
    sc = F.e8m0_decode(s).repeat(32, axis=1)
    err = np.abs(d - x)
    # inside the grid the error is at most half a spacing (<= 2^-4 |x|, and
    # <= 16 * 2^X at the top binade); [448, 512) * 2^X clamps to 448
    inside = np.abs(x) <= 448 * sc
    assert np.all(err[inside] <= np.maximum(np.abs(x[inside]) * 2.0 ** -4, 2.0 ** -10 * sc[inside]))
    assert np.all(err <= 64 * sc)
    # decode(encode(decoded)) is a fixed point
    q2, s2 = Q.mxfp8_rows(d.astype(np.float32))
    assert np.array_equal(q2, q) and np.array_equal(s2, s)
    # scaling a row by 2^k shifts its scale codes by k and keeps its codes
    q3, s3 = Q.mxfp8_rows((x * np.float32(2.0 ** 5)).astype(np.float32))
    assert np.array_equal(q3, q) and np.array_equal(s3.astype(int), s.astype(int) + 5)
