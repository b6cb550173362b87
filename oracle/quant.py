"""Weight and activation quantisers of the fused MoE layer (CPU oracle).

TEST INFRASTRUCTURE ONLY: nothing on the GPU path may import this module.

* MXFP4 weights (flashinfer PR #3738, "perf: optimize MXFP4xBF16 & INT4xFP8 and
  add MXFP4xFP8 CUTLASS MoE backend for SM90", Description): E2M1 elements with
  one E8M0 scale per 32 consecutive elements along K.  The shared exponent
  follows the OCP Microscaling v1.0 conversion: X = floor(log2(max|v|)) - emax,
  emax = 2 for E2M1, then each element is v / 2^X rounded to nearest-even on
  the E2M1 grid and clamped to +-6.  A block whose magnitudes are all zero gets
  scale code 127 (1.0).  X below -127 is clamped to -127 (the smallest E8M0).
* INT4 weights (same page, Description: "INT4 weight + FP8 activation"; group
  size named in the review of prepare()): symmetric two's complement codes with
  one float32 scale per 128 consecutive K elements, s = amax/7 (float32
  division), q = round-half-even(w/s) clamped to [-8, 7]; an all-zero group
  gets s = 1.
* Per-token E4M3 activations (same page, Implementation Notes: per-token
  activation scales computed while expanding routed rows): s = amax/448 in
  float32, q = E4M3(x/s) with float32 division; an all-zero token gets s = 1.
* MXFP8 activations (the MXFP8 inputs of PR #4793, "Unify MoE CuTe DSL
  dispatch to be dtype agnostic", and of PR #3614's MXFP8xMXFP8 profiling):
  E4M3 elements with one E8M0 scale per 32 consecutive elements of a row, by
  the same OCP MX v1.0 conversion as the weights with the E4M3 element's
  emax = 8: X = floor(log2(max|v|)) - 8 (clamped to [-127, 127]), elements
  E4M3(v / 2^X) rounded to nearest-even and saturated at 448; an all-zero
  block gets scale code 127.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os

import numpy as np

from . import formats as F

_POOL = None


def _rows_parallel(n_rows: int, fn, min_rows: int = 64):
    """Runs fn(slice) over row ranges on a thread pool (rows are independent;
    NumPy releases the GIL inside its loops).  Same result as fn(slice(0, n))."""
    global _POOL
    workers = min(16, os.cpu_count() or 1)
    if n_rows < 2 * min_rows or workers == 1:
        fn(slice(0, n_rows))
        return
    if _POOL is None:
        _POOL = _cf.ThreadPoolExecutor(max_workers=workers)
    step = max(min_rows, -(-n_rows // (4 * workers)))
    list(_POOL.map(fn, [slice(i, min(i + step, n_rows)) for i in range(0, n_rows, step)]))

MX_BLOCK = 32
INT4_GROUP = 128


def floor_log2(a: np.ndarray) -> np.ndarray:
    """floor(log2(a)) for positive finite a, exactly (via frexp: a = m*2^e with
    m in [0.5, 1), so floor(log2 a) = e - 1)."""
    _, e = np.frexp(np.asarray(a, dtype=np.float64))
    return e.astype(np.int64) - 1


def mxfp4_quantize(w: np.ndarray):
    """w: float32 [N, K] (K % 32 == 0) -> (codes uint8 [N, K/2], scales uint8 [N, K/32])."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    assert k % MX_BLOCK == 0
    packed = np.empty((n, k // 2), dtype=np.uint8)
    scale_code = np.empty((n, k // MX_BLOCK), dtype=np.uint8)

    def rows(sl):
        blk = w[sl].reshape(-1, k // MX_BLOCK, MX_BLOCK).astype(np.float64)
        amax = np.max(np.abs(blk), axis=-1)
        nz = amax > 0
        x = np.where(nz, floor_log2(np.where(nz, amax, 1.0)) - F.E2M1_EMAX, 0)
        x = np.maximum(x, -127)
        scale_code[sl] = (x + 127).astype(np.uint8)
        v = np.ldexp(blk, -x[..., None])  # exact power-of-two scaling in float64
        packed[sl] = F.pack_nibbles(F.e2m1_encode(v).reshape(-1, k))

    _rows_parallel(n, rows)
    return packed, scale_code


def mxfp4_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Packed MXFP4 [N, K/2] + E8M0 [N, K/32] -> float64 [N, K] (exact)."""
    n = codes.shape[0]
    k = codes.shape[1] * 2
    out = np.empty((n, k), dtype=np.float64)

    def rows(sl):
        el = F.e2m1_decode(F.unpack_nibbles(codes[sl]))
        sc = F.e8m0_decode(scales[sl])
        out[sl] = (el.reshape(-1, k // MX_BLOCK, MX_BLOCK) * sc[..., None]).reshape(-1, k)

    _rows_parallel(n, rows)
    return out


def int4_quantize(w: np.ndarray):
    """w: float32 [N, K] (K % 128 == 0) -> (codes uint8 [N, K/2], scales float32 [N, K/128])."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    assert k % INT4_GROUP == 0
    packed = np.empty((n, k // 2), dtype=np.uint8)
    s_all = np.empty((n, k // INT4_GROUP), dtype=np.float32)

    def rows(sl):
        grp = w[sl].reshape(-1, k // INT4_GROUP, INT4_GROUP)
        amax = np.max(np.abs(grp), axis=-1)
        s = np.where(amax > 0, amax / np.float32(7.0), np.float32(1.0)).astype(np.float32)
        r = (grp / s[..., None]).astype(np.float32)
        q = np.clip(np.rint(r), -8, 7).astype(np.int64).reshape(-1, k)
        packed[sl] = F.pack_nibbles((q & 0xF).astype(np.uint8))
        s_all[sl] = s

    _rows_parallel(n, rows)
    return packed, s_all


def int4_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    n = codes.shape[0]
    k = codes.shape[1] * 2
    out = np.empty((n, k), dtype=np.float64)

    def rows(sl):
        q = F.int4_decode(F.unpack_nibbles(codes[sl])).astype(np.float64)
        out[sl] = (q.reshape(-1, k // INT4_GROUP, INT4_GROUP)
                   * scales[sl].astype(np.float64)[..., None]).reshape(-1, k)

    _rows_parallel(n, rows)
    return out


def e4m3_rows(x: np.ndarray):
    """Row-wise E4M3 quantisation: x float32 [R, C] -> (codes uint8 [R, C], s float32 [R])."""
    x = np.asarray(x, dtype=np.float32)
    codes = np.empty(x.shape, dtype=np.uint8)
    s_all = np.empty(x.shape[0], dtype=np.float32)

    def rows(sl):
        xs = x[sl]
        amax = np.max(np.abs(xs), axis=-1)
        s = np.where(amax > 0, amax / np.float32(F.E4M3_MAX), np.float32(1.0)).astype(np.float32)
        v = (xs / s[:, None]).astype(np.float32)
        codes[sl] = F.e4m3_encode(v)
        s_all[sl] = s

    _rows_parallel(x.shape[0], rows)
    return codes, s_all


def mxfp8_rows(x: np.ndarray):
    """Row-wise MXFP8: x float32 [R, C] (C % 32 == 0) -> (E4M3 codes uint8
    [R, C], E8M0 scale codes uint8 [R, C/32])."""
    x = np.asarray(x, dtype=np.float32)
    r, c = x.shape
    assert c % MX_BLOCK == 0
    codes = np.empty((r, c), dtype=np.uint8)
    scale_code = np.empty((r, c // MX_BLOCK), dtype=np.uint8)

    def rows(sl):
        blk = x[sl].reshape(-1, c // MX_BLOCK, MX_BLOCK).astype(np.float64)
        amax = np.max(np.abs(blk), axis=-1)
        nz = amax > 0
        xe = np.where(nz, floor_log2(np.where(nz, amax, 1.0)) - F.E4M3_EMAX, 0)
        xe = np.clip(xe, -127, 127)
        scale_code[sl] = (xe + 127).astype(np.uint8)
        v = np.ldexp(blk, -xe[..., None])  # exact power-of-two scaling in float64
        codes[sl] = F.e4m3_encode(v).reshape(-1, c)

    _rows_parallel(r, rows)
    return codes, scale_code


def mxfp8_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """E4M3 codes [R, C] + E8M0 [R, C/32] -> float64 [R, C] (exact)."""
    r, c = codes.shape
    el = F.e4m3_decode(codes).reshape(r, c // MX_BLOCK, MX_BLOCK)
    return (el * F.e8m0_decode(scales)[..., None]).reshape(r, c)


def mx_exponent_spread(scales: np.ndarray) -> int:
    """Largest per-row spread of E8M0 codes (max - min).  The float64 GEMM of
    E4M3 x MXFP4 operands is exact, whatever the summation order, when this
    spread stays small (each product is a multiple of 2^(Xmin-10) and the sum
    stays below 2^(24.4+Xmax) for K <= 8192, so it needs at most 34.4 + spread
    significant bits)."""
    s = np.asarray(scales, dtype=np.int64)
    if s.size == 0:
        return 0
    return int(np.max(s.max(axis=-1) - s.min(axis=-1)))
