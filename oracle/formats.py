"""Number formats used by the fused MoE layer, written from their definitions.

TEST INFRASTRUCTURE ONLY (part of the CPU oracle): nothing on the GPU path may
import this module.

Formats (the pages name them; their definitions are the public OCP specs):

* E4M3 ("FN" flavour of the OCP 8-bit floating point spec): sign, 4 exponent
  bits with bias 7, 3 mantissa bits; exponent field 0 encodes subnormals
  m/8 * 2^-6; S.1111.111 is NaN; no infinities; largest finite 448.  The FP8
  activations of flashinfer PR #3738 ("perf: optimize MXFP4xBF16 & INT4xFP8 and
  add MXFP4xFP8 CUTLASS MoE backend for SM90", Description: "MXFP4 weight + FP8
  activation") are this format.
* E2M1 (OCP Microscaling spec, FP4 element): sign, 2 exponent bits with bias 1,
  1 mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no NaN or infinity.
  Two codes share a byte (the pages' fp4x2 storage): element 2i in the low
  nibble, element 2i+1 in the high nibble.
* E8M0 (OCP Microscaling spec, shared scale): value 2^(c-127), 0xFF is NaN.
  PR #3614 ("fix: make the cutlass MoE gemm profiler MXFP8-aware"), review
  thread, fills scale-factor buffers with 0x7F as the exponent meaning 1.0.
* bf16: the upper 16 bits of an IEEE float32.

Every encoder here picks the NEAREST representable value by direct comparison
against the decoded code table, breaking exact ties towards the code whose
least significant mantissa bit is 0 (round-to-nearest-even), saturating at the
largest finite magnitude, and keeping the sign of the input even when the
magnitude rounds to zero.
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------
# E4M3


def _e4m3_decode_scalar(code: int) -> float:
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        mag = (m / 8.0) * 2.0 ** -6
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


E4M3_TABLE = np.array([_e4m3_decode_scalar(c) for c in range(256)], dtype=np.float64)
E4M3_MAX = 448.0
E4M3_EMAX = 8  # largest power of two in E4M3 (448 = 1.75 * 2^8); the MX element emax
# Non-negative finite codes 0x00..0x7E; their values increase with the code.
_E4M3_POS = E4M3_TABLE[:0x7F].copy()
assert np.all(np.diff(_E4M3_POS) > 0)


def _nearest_even(a: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index of the grid value nearest to each a (a >= 0, a <= grid[-1]);
    exact ties go to the even index (even index == mantissa lsb 0 for both the
    E4M3 and E2M1 positive code orders).  Works through large arrays in
    chunks (same result, less memory traffic)."""
    flat = a.reshape(-1)
    out = np.empty(flat.shape, dtype=np.int64)
    step = 1 << 16
    for i in range(0, flat.size, step):
        out[i:i + step] = _nearest_even_chunk(flat[i:i + step], grid)
    return out.reshape(a.shape)


def _nearest_even_chunk(a: np.ndarray, grid: np.ndarray) -> np.ndarray:
    hi = np.searchsorted(grid, a, side="left")
    hi = np.clip(hi, 0, len(grid) - 1)
    lo = np.clip(hi - 1, 0, len(grid) - 1)
    # Compare 2a with the midpoint; all terms are exact in float64.
    mid = grid[lo] + grid[hi]
    two_a = 2.0 * a
    pick_hi = (two_a > mid) | ((two_a == mid) & (hi % 2 == 0))
    return np.where(pick_hi, hi, lo)


def e4m3_encode(x) -> np.ndarray:
    """Round x (finite float32/float64 values) to E4M3 codes (uint8)."""
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    idx = _nearest_even(a, _E4M3_POS).astype(np.uint8)
    return idx | (neg.astype(np.uint8) << 7)


def e4m3_decode(codes) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


# ----------------------------------------------------------------------------
# E2M1 and E8M0

E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_TABLE = np.concatenate([E2M1_MAG, -E2M1_MAG])  # code 8 is -0
E2M1_MAX = 6.0
E2M1_EMAX = 2  # 6 = 1.5 * 2^2


def e2m1_encode(x) -> np.ndarray:
    """Round x to 4-bit E2M1 codes (uint8 values 0..15)."""
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), E2M1_MAX)
    idx = _nearest_even(a, E2M1_MAG).astype(np.uint8)
    return idx | (neg.astype(np.uint8) << 3)


def e2m1_decode(codes) -> np.ndarray:
    return E2M1_TABLE[np.asarray(codes, dtype=np.uint8)]


def e8m0_decode(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64)
    v = np.ldexp(1.0, c - 127)
    return np.where(c == 255, np.nan, v)


# ----------------------------------------------------------------------------
# INT4 nibbles (two's complement, range -8..7)


def int4_decode(nibbles) -> np.ndarray:
    n = np.asarray(nibbles, dtype=np.int64) & 0xF
    return np.where(n >= 8, n - 16, n)


# ----------------------------------------------------------------------------
# nibble packing


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[..., K] 4-bit codes -> [..., K/2] bytes (element 2i low, 2i+1 high)."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


# ----------------------------------------------------------------------------
# bf16


def bf16_to_f32(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def bf16_rne(x) -> np.ndarray:
    """float32 -> nearest bf16 (ties to even mantissa), returned as uint16 bits.
    Finite inputs whose rounded value stays finite."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    lo_bits = u & np.uint32(0xFFFF0000)        # truncation towards zero
    hi_bits = lo_bits + np.uint32(0x10000)     # next bf16 away from zero
    lo = np.abs(lo_bits.view(np.float32).astype(np.float64))
    hi = np.abs(hi_bits.view(np.float32).astype(np.float64))
    a = np.abs(f.astype(np.float64))
    mid = lo + hi
    lo_even = ((lo_bits >> 16) & 1) == 0
    pick_hi = (2.0 * a > mid) | ((2.0 * a == mid) & ~lo_even)
    out = np.where(pick_hi, hi_bits, lo_bits) >> 16
    return out.astype(np.uint16)


def f32(x) -> np.ndarray:
    """Round to float32 (IEEE round-to-nearest-even)."""
    return np.asarray(x).astype(np.float32)
