// Operand helpers and epilogue shared by the grouped GEMM kernels of the fused
// MoE on CDNA4 matrix cores (gfx950).
//
// flashinfer PR #3738 ("perf: optimize MXFP4xBF16 & INT4xFP8 and add MXFP4xFP8
// CUTLASS MoE backend for SM90"), Description and Implementation Notes: grouped
// MoE GEMMs over MXFP4 or INT4 expert weights against FP8 or BF16 activations,
// a precomputed work map, per-token-scale epilogues, and (for MXFP4 x FP8) the
// E8M0 weight scale applied inside the matrix product.  On gfx950 the block-
// scaled MFMA V_MFMA_SCALE_F32_16X16X128_F8F6F4 takes E2M1 weights and E8M0
// scales directly, so no pre-MMA scale folding is needed:
//   * MXFP4 x FP8 : scaled MFMA, A = E4M3 token codes (scale 1), B = E2M1
//                   weights with their E8M0 scales; the token scale is applied
//                   in the epilogue.
//   * MXFP4 x MXFP8: the same MFMA with the activations' E8M0 block scales as
//                   its A scale operand (no epilogue scale).
//   * MXFP4 x MXFP4 (W4A4): the same MFMA with E2M1 activations (A format
//                   code 4, four operand registers, twice the FP8 rate).
//   * MXFP4 x BF16: weights expanded to bf16 in registers with the E8M0 scale
//                   folded in (exact), then bf16 MFMA 16x16x32.
//   * INT4 x FP8  : INT4 codes mapped to E4M3 (exact) in registers, one FP8
//                   MFMA per 128-element group, then the group's float32 scale
//                   multiplies the partial sum (post-MMA scaling).
// Operand lane layouts (16x16x128): an FP8 operand lane l holds row l%16 with
// bytes 0-15 at k = 16*(l/16)+b and bytes 16-31 at k = 64+16*(l/16)+(b-16); an
// FP4 operand lane holds 32 consecutive k = 32*(l/16)+n; E8M0 scale of lane l
// covers row l%16, k-block l/16; the output lane l holds column l%16 of rows
// 4*(l/16)+[0,4).  For the unscaled paths any k permutation shared by both
// operands gives the same sum, which the INT4 and bf16 paths use.
//
// Blocks of WAVES_M x WAVES_N waves; each wave owns WM x WN 16x16 output
// tiles.  FC1 writes h = silu(gate) * up (gate/up rows interleaved per 16-row
// block by the weight layout); FC2 writes y2 = acc * row scale.
#pragma once

#include <type_traits>

#include "moe_common.h"

namespace moe {

template <int V>
struct Frag;

template <>
struct Frag<kMxfp4Fp8> {
  static constexpr int kA = 2;  // uint4 per A row fragment
};
template <>
struct Frag<kMxfp4Mxfp8> {
  static constexpr int kA = 2;
};
template <>
struct Frag<kMxfp4Mxfp4> {
  static constexpr int kA = 1;
};
template <>
struct Frag<kInt4Fp8> {
  static constexpr int kA = 2;
};
template <>
struct Frag<kMxfp4Bf16> {
  static constexpr int kA = 4;
};

__device__ __forceinline__ v8i as_v8i(const uint4& lo, const uint4& hi) {
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

__device__ __forceinline__ v8i fp4_operand(const uint4& b) {
  v8i r;
  r[0] = b.x; r[1] = b.y; r[2] = b.z; r[3] = b.w;
  r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
  return r;
}

__device__ __forceinline__ v8i int4_operand(const uint4& b) {
  const uint32_t w[4] = {b.x, b.y, b.z, b.w};
  v8i r;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    r[2 * d] = int4sm_to_e4m3(w[d] & 0x0F0F0F0Fu);
    r[2 * d + 1] = int4sm_to_e4m3((w[d] >> 4) & 0x0F0F0F0Fu);
  }
  return r;
}

__device__ __forceinline__ v8bf as_bf16x8(const uint4& u) {
  v8bf r;
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[2 * i] = __builtin_bit_cast(__bf16, (unsigned short)(w[i] & 0xFFFF));
    r[2 * i + 1] = __builtin_bit_cast(__bf16, (unsigned short)(w[i] >> 16));
  }
  return r;
}

// 8 E2M1 codes (one dword) -> 8 bf16 values times `scale` (exact conversion).
__device__ __forceinline__ v8bf fp4x8_to_bf16(uint32_t w, float scale) {
  v8bf r;
  const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// SiLU g / (1 + e^-g) with the hardware exp2 and reciprocal (relative error
// about 1e-6, against the 1e-4 tolerance on h): the accurate expf and an IEEE
// division cost ~25 VALU instructions per output, which in a one-block-per-CU
// GEMM is time the matrix cores sit idle.
__device__ __forceinline__ float silu(float g) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.44269504088896341f);
  return g * __builtin_amdgcn_rcpf(1.0f + e);
}

// Epilogue shared by the GEMM kernels.  Output tile (i, j) of a wave holds, in
// lane l, column 16*(nb0+j) + l%16 of rows row_base + RS*i + 4*(l/16) + [0, 4)
// (RS = 16: the wave's subtiles are consecutive 16-row groups; 32: every
// second group).
//   FC1: tiles (2q, 2q+1) are the gate and up halves of intermediate block
//        (nb0 + 2q)/2; h = silu(g*s) * (u*s), s = token scale.
//   FC2: y2 = acc * s, s = row scale.
// These row-per-register epilogues (INT4 only) write with streaming
// (non-temporal) 4-byte stores: h and y2 are read once, by the next kernel,
// long after the block is gone, and keeping them out of the caches measured
// 1-4 % faster there (an L2-resident y2 for a fused finalize by float
// atomics, tried as well, made GEMM2 2.1x slower).  epilogue_sc takes the
// row scales loaded beforehand (load_row_scales), epilogue loads them itself.

// Row scales of this lane's accumulator rows (1 without row scales).
template <bool FC1, int WM, int RS = 16>
__device__ __forceinline__ void load_row_scales(const GemmParams& p, int row_base, int row_end,
                                                int lane, float (&sc)[WM][4]) {
  const int row_lane = 4 * (lane >> 4);
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = min(row_base + RS * i + row_lane + v, row_end - 1);
      sc[i][v] = !p.row_scale ? 1.0f
                 : FC1       ? p.row_scale[p.row_token[r]]
                             : p.row_scale[r];
    }
}

// 4 x 4 transpose inside each quad of lanes (DPP quad permutes): on entry
// lane 4a + b holds m[v] = M[b][v], on exit M[v][b].  Swapping bit 0 and then
// bit 1 of (lane, value) transposes the 2-bit indices.
__device__ __forceinline__ v4f quad_transpose(const v4f& m, int lane) {
  const int b = lane & 3;
  v4f t, r;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float x = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m[v ^ 1]), 0xB1, 0xF, 0xF, false));
    t[v] = ((b ^ v) & 1) ? x : m[v];
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float x = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(t[v ^ 2]), 0x4E, 0xF, 0xF, false));
    r[v] = ((b ^ v) & 2) ? x : t[v];
  }
  return r;
}

// Row-per-register epilogue (INT4): lane l of tile (i, j) holds rows
// 4 (l / 16) + [0, 4) of column l % 16.  The four lanes of a quad transpose
// their 4 x 4 block first, so each holds four consecutive columns of one row,
// and two neighbouring subtiles leave as whole 128-byte lines with 16-byte
// streaming stores (same box: INT4 GEMM2 0.424 -> 0.411 ms; the transpose
// alone, 16 rows x 64 bytes per store, changed nothing).
template <bool FC1, int WM, int WN, int RS = 16>
__device__ __forceinline__ void epilogue_sc(const GemmParams& p, const v4f (&acc)[WM][WN],
                                            const float (&sc)[WM][4], int row_base, int row_end,
                                            int nvalid, int64_t nb0, int jvalid, int lane) {
  const int row_lane = 4 * (lane >> 4);
  const int rq = lane & 3;                 // row of the quad's block after the transpose
  const int cq = 4 * ((lane & 15) >> 2);   // its first column
  // output subtile pairs: lanes of rows 8-15 (lane bit 5) swap their first
  // block for the second block of rows 0-7, so each store writes 8 rows x
  // 128 bytes (one pair of 16-column h blocks for FC1, of y2 subtiles for FC2)
  const bool lo = (lane & 32) == 0;
  const int rbase = 4 * ((lane >> 4) & 1) + rq;  // row within the 8-row half
  auto store_pair = [&](int i, const v4f& y0, const v4f& y1, int64_t col0)
                        __attribute__((always_inline)) {
    const v4f t0 = quad_transpose(y0, lane), t1 = quad_transpose(y1, lane);
    const v4f snd = lo ? t1 : t0;
    v4f rcv;
#pragma unroll
    for (int c = 0; c < 4; ++c) rcv[c] = __shfl_xor(snd[c], 32);
    const int64_t col = col0 + (lo ? 0 : 16) + cq;
    const v4f va = lo ? t0 : rcv, vb = lo ? rcv : t1;
    const int ra = row_base + RS * i + rbase, rb = ra + 8;
    if (ra < row_end)
      __builtin_nontemporal_store(va, reinterpret_cast<v4f*>(&p.out[(int64_t)ra * p.out_stride + col]));
    if (rb < row_end)
      __builtin_nontemporal_store(vb, reinterpret_cast<v4f*>(&p.out[(int64_t)rb * p.out_stride + col]));
  };
  if constexpr (FC1 && WN % 4 != 0) {
    // one h block per wave: 16 rows x 64 bytes per store
#pragma unroll
    for (int q = 0; q < WN / 2; ++q) {
      if (2 * q >= jvalid) continue;
      const int64_t ib = (nb0 + 2 * q) >> 1;
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        if (i >= nvalid) continue;
        v4f h;
#pragma unroll
        for (int v = 0; v < 4; ++v)
          h[v] = silu(acc[i][2 * q][v] * sc[i][v]) * (acc[i][2 * q + 1][v] * sc[i][v]);
        const v4f t = quad_transpose(h, lane);
        const int r = row_base + RS * i + row_lane + rq;
        if (r < row_end)
          __builtin_nontemporal_store(t, reinterpret_cast<v4f*>(&p.out[(int64_t)r * p.out_stride + ib * 16 + cq]));
      }
    }
  } else if constexpr (FC1) {
#pragma unroll
    for (int q = 0; q < WN / 2; q += 2) {
      if (2 * q >= jvalid) continue;
      const int64_t ib = (nb0 + 2 * q) >> 1;  // first of two intermediate 16-column blocks
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        if (i >= nvalid) continue;
        v4f h0, h1;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          h0[v] = silu(acc[i][2 * q][v] * sc[i][v]) * (acc[i][2 * q + 1][v] * sc[i][v]);
          h1[v] = silu(acc[i][2 * q + 2][v] * sc[i][v]) * (acc[i][2 * q + 3][v] * sc[i][v]);
        }
        store_pair(i, h0, h1, ib * 16);
      }
    }
  } else {
    static_assert(WN % 2 == 0, "pairs of y2 subtiles");
#pragma unroll
    for (int j = 0; j < WN; j += 2) {
      if (j >= jvalid) continue;
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        if (i >= nvalid) continue;
        v4f y0, y1;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          y0[v] = acc[i][j][v] * sc[i][v];
          y1[v] = acc[i][j + 1][v] * sc[i][v];
        }
        store_pair(i, y0, y1, (nb0 + j) * 16);
      }
    }
  }
}

// Row scales loaded once before any store (the output may alias the scale
// arrays as far as the compiler knows, so loads placed between stores would
// each wait for the store before them).
template <bool FC1, int WM, int WN, int RS = 16>
__device__ __forceinline__ void epilogue(const GemmParams& p, const v4f (&acc)[WM][WN],
                                         int row_base, int row_end, int nvalid, int64_t nb0,
                                         int jvalid, int lane) {
  float sc[WM][4];
  load_row_scales<FC1, WM, RS>(p, row_base, row_end, lane, sc);
  epilogue_sc<FC1, WM, WN, RS>(p, acc, sc, row_base, row_end, nvalid, nb0, jvalid, lane);
}

// End of a GEMM block with row-per-register accumulators (INT4 weights).
template <int V, bool FC1, int WM, int WN, int RS = 16>
__device__ __forceinline__ void finish_tile(const GemmParams& p, const v4f (&acc)[WM][WN],
                                            int row_base, int row_end, int nvalid, int64_t nb0,
                                            int jvalid, int lane) {
  static_assert(V == kInt4Fp8, "the other formats use transposed accumulators");
  epilogue<FC1, WM, WN, RS>(p, acc, row_base, row_end, nvalid, nb0, jvalid, lane);
}

// ---------------------------------------------------------------------------
// Transposed accumulators.  For every format except INT4 the kernels give the
// matrix core the weights as its A operand and the activations as B, which
// computes the transpose of the output tile: lane l of tile (i, j) then holds
// columns 16 (nb0 + j) + 4 (l / 16) + [0, 4) of the single row
// row_base + RS i + l % 16.  Four consecutive columns of one row make one
// 16-byte store, so the epilogue issues a quarter of the store instructions of
// the row-per-register layout above (which INT4 keeps: its post-MMA group
// scale is per output column, one per lane there), and a lane needs one row
// scale per subtile instead of four.  Both operand layouts are the same for
// rows and columns (lane l holds row / column l % 16 and the same K range), so
// only the argument order and the scale operands swap.
template <int AF, int SW, int SA>
__device__ __forceinline__ v4f mfma_wt(const v8i& w, const v8i& a, const v4f& c, int scale_w,
                                       int scale_a) {
  // D^T = W . A^T: weights E2M1 (format 4) with their E8M0 scale word and
  // byte select SW; activations in format AF with scale word / byte select SA
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, a, c, 4, AF, SW, scale_w, SA, scale_a);
}

// Row scale of this lane's row in each subtile (1 without row scales).
template <bool FC1, int WM, int RS = 16>
__device__ __forceinline__ void load_row_scales_t(const GemmParams& p, int row_base, int row_end,
                                                  int lane, float (&sc)[WM]) {
#pragma unroll
  for (int i = 0; i < WM; ++i) {
    const int r = min(row_base + RS * i + (lane & 15), row_end - 1);
    sc[i] = !p.row_scale ? 1.0f : FC1 ? p.row_scale[p.row_token[r]] : p.row_scale[r];
  }
}

__device__ __forceinline__ void store4_nt(float* dst, float x, float y, float z, float w) {
  __builtin_nontemporal_store(v4f{x, y, z, w}, reinterpret_cast<v4f*>(dst));
}
__device__ __forceinline__ void store4(float* dst, float x, float y, float z, float w) {
  *reinterpret_cast<v4f*>(dst) = v4f{x, y, z, w};
}

// FC1: h = silu(g * s) * (u * s) for tiles (2q, 2q+1) = gate / up of
// intermediate block (nb0 + 2q) / 2; FC2: y2 = acc * s.  A lane holds 4
// columns of one row, so a 16-byte store covers 16 rows x 64 bytes; the lanes
// of rows r and r ^ 8 first swap the halves of two neighbouring subtiles, so
// each store writes 8 rows x 128 bytes, whole cache lines, and both outputs
// leave with streaming stores.  Same-box timings on the DeepSeek prefill
// shapes: whole lines made GEMM1 1.3 % faster; for y2, streaming stores were
// 6 % slower than plain ones with half lines and are 1.4 % faster with whole
// lines (and the finalize that reads y2 back 2-4 % faster).  Subtiles
// [i0, i1) only (the peeled last K step writes them one by one).
template <bool FC1, int WM, int WN, int RS = 16>
__device__ __forceinline__ void epilogue_t(const GemmParams& p, const v4f (&acc)[WM][WN],
                                           const float (&sc)[WM], int row_base, int row_end,
                                           int nvalid, int64_t nb0, int jvalid, int lane,
                                           int i0 = 0, int i1 = WM) {
  const int c4 = 4 * (lane >> 4);
  if constexpr (!FC1 && WN % 2 == 0) {
    const bool lo = (lane & 8) == 0;
    const int rr = lane & 7;
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      if (i >= nvalid) continue;
      if (i < i0 || i >= i1) continue;
      const float s = sc[i];
      const int r0 = row_base + RS * i;
#pragma unroll
      for (int j = 0; j < WN; j += 2) {
        if (j >= jvalid) continue;
        const v4f a0 = acc[i][j] * s, a1 = acc[i][j + 1] * s;
        const v4f snd = lo ? a1 : a0;
        v4f rcv;
#pragma unroll
        for (int c = 0; c < 4; ++c) rcv[c] = __shfl_xor(snd[c], 8);
        const int64_t col = (nb0 + j + (lo ? 0 : 1)) * 16 + c4;
        const v4f v0 = lo ? a0 : rcv, v1 = lo ? rcv : a1;
        if (r0 + rr < row_end)
          store4_nt(p.out + (int64_t)(r0 + rr) * p.out_stride + col, v0[0], v0[1], v0[2], v0[3]);
        if (r0 + 8 + rr < row_end)
          store4_nt(p.out + (int64_t)(r0 + 8 + rr) * p.out_stride + col, v1[0], v1[1], v1[2], v1[3]);
      }
    }
  } else if constexpr (FC1 && WN % 4 == 0) {
    const bool lo = (lane & 8) == 0;
    const int rr = lane & 7;
#pragma unroll
    for (int i = 0; i < WM; ++i) { if (i < i0 || i >= i1) continue;
      if (i >= nvalid) continue;
      const float s = sc[i];
      const int r0 = row_base + RS * i;
#pragma unroll
      for (int q = 0; q < WN / 2; q += 2) {
        if (2 * q >= jvalid) continue;
        v4f h0, h1;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          h0[c] = silu(acc[i][2 * q][c] * s) * (acc[i][2 * q + 1][c] * s);
          h1[c] = silu(acc[i][2 * q + 2][c] * s) * (acc[i][2 * q + 3][c] * s);
        }
        // rows 0-7 keep subtile q and receive q + 1 of row r ^ 8; rows 8-15
        // the reverse
        const v4f snd = lo ? h1 : h0;
        v4f rcv;
#pragma unroll
        for (int c = 0; c < 4; ++c) rcv[c] = __shfl_xor(snd[c], 8);
        const int64_t col = ((nb0 + 2 * q) >> 1) * 16 + (lo ? 0 : 16) + c4;
        const v4f v0 = lo ? h0 : rcv, v1 = lo ? rcv : h1;
        if (r0 + rr < row_end)
          store4_nt(p.out + (int64_t)(r0 + rr) * p.out_stride + col, v0[0], v0[1], v0[2], v0[3]);
        if (r0 + 8 + rr < row_end)
          store4_nt(p.out + (int64_t)(r0 + 8 + rr) * p.out_stride + col, v1[0], v1[1], v1[2], v1[3]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < WM; ++i) { if (i < i0 || i >= i1) continue;
      if (i >= nvalid) continue;
      const int r = row_base + RS * i + (lane & 15);
      if (r >= row_end) continue;
      float* orow = p.out + (int64_t)r * p.out_stride;
      const float s = sc[i];
      if (FC1) {
#pragma unroll
        for (int q = 0; q < WN / 2; ++q) {
          if (2 * q >= jvalid) continue;
          const int64_t c = ((nb0 + 2 * q) >> 1) * 16 + c4;
          const v4f g = acc[i][2 * q], u = acc[i][2 * q + 1];
          store4_nt(orow + c, silu(g[0] * s) * (u[0] * s), silu(g[1] * s) * (u[1] * s),
                    silu(g[2] * s) * (u[2] * s), silu(g[3] * s) * (u[3] * s));
        }
      } else {
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          if (j >= jvalid) continue;
          const v4f a = acc[i][j];
          store4(orow + (nb0 + j) * 16 + c4, a[0] * s, a[1] * s, a[2] * s, a[3] * s);
        }
      }
    }
  }
}

// FC1 epilogue for MX activation formats, transposed layout: MX block
// b = nb0 / 4 + m covers intermediate blocks 2m, 2m+1 of the wave (device
// tiles 4m .. 4m+3); lane l holds its row's columns 4 (l/16) + [0, 4) of both
// halves, so the block amax is a reduction over the four lanes l % 16 + 16 g.
// Same h values, exponent rule and encoders as the separate FC2 quantiser.
template <bool E2M1, int WM, int WN, int RS = 16>
__device__ __forceinline__ void epilogue_fc1_mx_t(const GemmParams& p, const v4f (&acc)[WM][WN],
                                                  int row_base, int row_end, int nvalid,
                                                  int64_t nb0, int jvalid, int lane,
                                                  int i0 = 0, int i1 = WM) {
  static_assert(WN % 4 == 0, "whole 32-column MX blocks per wave");
  if (jvalid < WN) return;  // columns past N (N is a multiple of 256)
  const int g4 = lane >> 4;
#pragma unroll
  for (int i = 0; i < WM; ++i) { if (i < i0 || i >= i1) continue;
    if (i >= nvalid) continue;
    const int r = row_base + RS * i + (lane & 15);
    const bool live = r < row_end;
    uint8_t* qrow = p.q_out + (int64_t)r * p.q_stride;
#pragma unroll
    for (int m = 0; m < WN / 4; ++m) {
      const int64_t b = (nb0 >> 2) + m;  // MX block: h columns [32b, 32b + 32)
      float x0[4], x1[4];
      float amax = 0.0f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        x0[v] = silu(acc[i][4 * m][v]) * acc[i][4 * m + 1][v];
        x1[v] = silu(acc[i][4 * m + 2][v]) * acc[i][4 * m + 3][v];
        amax = fmaxf(amax, fmaxf(fabsf(x0[v]), fabsf(x1[v])));
      }
      amax = fmaxf(amax, __shfl_xor(amax, 16));
      amax = fmaxf(amax, __shfl_xor(amax, 32));
      const int x = mx_exponent<E2M1 ? 2 : 8>(amax);
      const float inv = __uint_as_float((uint32_t)(127 - x) << 23);  // 2^-X
      if (E2M1) {
        uint32_t n0 = 0, n1 = 0;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          n0 |= (e2m1_magnitude_code(fabsf(x0[v]) * inv) | ((__float_as_uint(x0[v]) >> 31) << 3)) << (4 * v);
          n1 |= (e2m1_magnitude_code(fabsf(x1[v]) * inv) | ((__float_as_uint(x1[v]) >> 31) << 3)) << (4 * v);
        }
        if (live) {  // columns 32b + 4g + v -> byte 16b + 2g (+ 8 for the second half)
          *reinterpret_cast<uint16_t*>(qrow + 16 * b + 2 * g4) = (uint16_t)n0;
          *reinterpret_cast<uint16_t*>(qrow + 16 * b + 8 + 2 * g4) = (uint16_t)n1;
        }
      } else if (live) {
        // x * 2^-X is below 512 in magnitude; saturate at 448 as the encoder does
        float y0[4], y1[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          y0[v] = fminf(fmaxf(x0[v] * inv, -448.0f), 448.0f);
          y1[v] = fminf(fmaxf(x1[v] * inv, -448.0f), 448.0f);
        }
        const uint32_t w0 = e4m3_pk(y0[0], y0[1]) | (e4m3_pk(y0[2], y0[3]) << 16);
        const uint32_t w1 = e4m3_pk(y1[0], y1[1]) | (e4m3_pk(y1[2], y1[3]) << 16);
        *reinterpret_cast<uint32_t*>(qrow + 32 * b + 4 * g4) = w0;
        *reinterpret_cast<uint32_t*>(qrow + 32 * b + 16 + 4 * g4) = w1;
      }
      if (live && g4 == 0)
        p.q_bscales[(int64_t)r * p.q_bstride + mx_scale_offset(b)] = (uint8_t)(x + 127);
    }
  }
}

// FC1 epilogue for BF16 activations, transposed layout: bf16(h) of the
// lane's four columns, one 8-byte store.
template <int WM, int WN, int RS = 16>
__device__ __forceinline__ void epilogue_fc1_bf16_t(const GemmParams& p, const v4f (&acc)[WM][WN],
                                                    int row_base, int row_end, int nvalid,
                                                    int64_t nb0, int jvalid, int lane,
                                                    int i0 = 0, int i1 = WM) {
  const int c4 = 4 * (lane >> 4);
#pragma unroll
  for (int i = 0; i < WM; ++i) { if (i < i0 || i >= i1) continue;
    if (i >= nvalid) continue;
    const int r = row_base + RS * i + (lane & 15);
    if (r >= row_end) continue;
    uint16_t* qrow = reinterpret_cast<uint16_t*>(p.q_out + (int64_t)r * p.q_stride);
#pragma unroll
    for (int q = 0; q < WN / 2; ++q) {
      if (2 * q >= jvalid) continue;
      const int64_t c = ((nb0 + 2 * q) >> 1) * 16 + c4;
      uint32_t h[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) h[v] = bf16_bits(silu(acc[i][2 * q][v]) * acc[i][2 * q + 1][v]);
      *reinterpret_cast<uint2*>(qrow + c) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
    }
  }
}

// End of a GEMM block with transposed accumulators: the fused FC1 + FC2-input
// epilogue when the caller asks for it (q_out set) and the format and tile
// allow it, else the plain one with the given row scales.
template <int V, bool FC1, int WM, int WN, int RS = 16>
__device__ __forceinline__ void finish_tile_t(const GemmParams& p, const v4f (&acc)[WM][WN],
                                              const float (&sc)[WM], int row_base, int row_end,
                                              int nvalid, int64_t nb0, int jvalid, int lane,
                                              int i0 = 0, int i1 = WM) {
  if constexpr (FC1 && a_blockscaled(V) && WN % 4 == 0) {
    if (p.q_out) {
      epilogue_fc1_mx_t<a_fp4(V), WM, WN, RS>(p, acc, row_base, row_end, nvalid, nb0, jvalid, lane, i0, i1);
      return;
    }
  }
  if constexpr (FC1 && V == kMxfp4Bf16) {
    if (p.q_out) {
      epilogue_fc1_bf16_t<WM, WN, RS>(p, acc, row_base, row_end, nvalid, nb0, jvalid, lane, i0, i1);
      return;
    }
  }
  epilogue_t<FC1, WM, WN, RS>(p, acc, sc, row_base, row_end, nvalid, nb0, jvalid, lane, i0, i1);
}

hipError_t launch_gemm_direct(int variant, bool fc1, int cfg, const GemmParams& p,
                              int64_t max_tiles, hipStream_t st);
hipError_t launch_gemm_lds(int variant, bool fc1, int cfg, const GemmParams& p,
                           int64_t max_tiles, hipStream_t st);

}  // namespace moe
