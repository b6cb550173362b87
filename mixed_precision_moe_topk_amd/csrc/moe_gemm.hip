// Grouped GEMMs of the fused MoE on CDNA4 matrix cores (gfx950).
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
// Block = 4 waves (WAVES_M x WAVES_N); each wave owns WM x WN 16x16 output
// tiles.  FC1 writes h = silu(gate) * up (gate/up rows interleaved per 16-row
// block by the weight layout); FC2 writes y2 = acc * row scale.
#include "moe_common.h"

namespace moe {

template <int V>
struct Frag;

template <>
struct Frag<kMxfp4Fp8> {
  static constexpr int kA = 2;  // uint4 per A row fragment
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

template <int V, bool FC1, int WAVES_M, int WM, int WN>
__global__ __launch_bounds__(256) void k_gemm(GemmParams p) {
  constexpr int WAVES_N = 4 / WAVES_M;
  constexpr int NA = Frag<V>::kA;
  static_assert(!FC1 || WN % 2 == 0, "FC1 pairs gate/up tiles");
  const int64_t item = blockIdx.x;
  const int64_t mt = item / p.n_tiles;
  const int nt = (int)(item - mt * p.n_tiles);
  if (mt >= *p.num_tiles) return;
  const Tile tile = p.tiles[mt];
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int row_base = tile.row0 + 16 * WM * wm;
  const int row_end = tile.row0 + tile.nrows;
  const int nvalid = min(WM, (row_end - row_base + 15) / 16);
  if (nvalid <= 0) return;

  const int K = p.K;
  const int KS = K / kKStep, KS4 = (KS + 3) / 4;
  const int64_t e = tile.expert;
  const uint8_t* wbase = p.w + e * p.w_expert_stride;
  const uint8_t* sbase = p.s + e * p.s_expert_stride;
  const int64_t nb0 = (int64_t)nt * (WAVES_N * WN) + wn * WN;

  // A row pointers (rows past the tile end re-read its last row; their
  // outputs are never stored)
  const uint8_t* arow[WM];
#pragma unroll
  for (int i = 0; i < WM; ++i) {
    const int r = min(row_base + 16 * i + (lane & 15), row_end - 1);
    const int64_t src = FC1 ? (int64_t)p.row_token[r] : (int64_t)r;
    int64_t off;
    if (V == kMxfp4Fp8) off = 16 * (lane >> 4);
    else if (V == kInt4Fp8) off = 32 * (lane >> 4);
    else off = 64 * (lane >> 4);  // bf16: 32 elements * 2 bytes
    arow[i] = p.a + src * p.a_stride + off;
  }

  v4f acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  uint4 ac[WM][NA], an[WM][NA];
  uint4 bc[WN], bn[WN];
  uint32_t scc[WN], scn[WN];  // E8M0 dword (MXFP4) or float bits (INT4 group scale)

  auto load = [&](int ks, uint4 (&a)[WM][NA], uint4 (&b)[WN], uint32_t (&sc)[WN]) {
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      if (i < nvalid) {
        if (V == kMxfp4Fp8) {
          a[i][0] = *reinterpret_cast<const uint4*>(arow[i] + ks * kKStep);
          a[i][1] = *reinterpret_cast<const uint4*>(arow[i] + ks * kKStep + 64);
        } else if (V == kInt4Fp8) {
          a[i][0] = *reinterpret_cast<const uint4*>(arow[i] + ks * kKStep);
          a[i][1] = *reinterpret_cast<const uint4*>(arow[i] + ks * kKStep + 16);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            a[i][q] = *reinterpret_cast<const uint4*>(arow[i] + 2 * ks * kKStep + 16 * q);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int64_t nb = nb0 + j;
      b[j] = *reinterpret_cast<const uint4*>(wbase + ((nb * KS + ks) * 64 + lane) * 16);
      if (V == kInt4Fp8)
        sc[j] = *reinterpret_cast<const uint32_t*>(sbase + ((nb * KS + ks) * 16 + (lane & 15)) * 4);
      else
        sc[j] = *reinterpret_cast<const uint32_t*>(sbase + ((nb * KS4 + (ks >> 2)) * 64 + lane) * 4);
    }
  };

  auto compute = [&](int ks, const uint4 (&a)[WM][NA], const uint4 (&b)[WN],
                     const uint32_t (&sc)[WN]) {
    if (V == kMxfp4Fp8) {
      v8i bop[WN];
#pragma unroll
      for (int j = 0; j < WN; ++j) bop[j] = fp4_operand(b[j]);
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        if (i < nvalid) {
          const v8i aop = as_v8i(a[i][0], a[i][1]);
#pragma unroll
          for (int j = 0; j < WN; ++j) {
            switch (ks & 3) {
              case 0: acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop[j], acc[i][j], 0, 4, 0, 127, 0, (int)sc[j]); break;
              case 1: acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop[j], acc[i][j], 0, 4, 0, 127, 1, (int)sc[j]); break;
              case 2: acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop[j], acc[i][j], 0, 4, 0, 127, 2, (int)sc[j]); break;
              default: acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop[j], acc[i][j], 0, 4, 0, 127, 3, (int)sc[j]); break;
            }
          }
        }
      }
    } else if (V == kInt4Fp8) {
      v8i bop[WN];
#pragma unroll
      for (int j = 0; j < WN; ++j) bop[j] = int4_operand(b[j]);
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        if (i < nvalid) {
          const v8i aop = as_v8i(a[i][0], a[i][1]);
#pragma unroll
          for (int j = 0; j < WN; ++j) {
            const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                aop, bop[j], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
            const float gs = __uint_as_float(sc[j]);
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[i][j][v] += part[v] * gs;
          }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const float scale = e8m0_to_float((sc[j] >> (8 * (ks & 3))) & 0xFFu);
        const uint32_t bw[4] = {b[j].x, b[j].y, b[j].z, b[j].w};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const v8bf bop = fp4x8_to_bf16(bw[s], scale);
#pragma unroll
          for (int i = 0; i < WM; ++i) {
            if (i < nvalid)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[i][s]), bop,
                                                                  acc[i][j], 0, 0, 0);
          }
        }
      }
    }
  };

  load(0, ac, bc, scc);
  for (int ks = 0; ks < KS; ks += 2) {
    if (ks + 1 < KS) load(ks + 1, an, bn, scn);
    compute(ks, ac, bc, scc);
    if (ks + 1 < KS) {
      if (ks + 2 < KS) load(ks + 2, ac, bc, scc);
      compute(ks + 1, an, bn, scn);
    }
  }

  // epilogue
  const int col_lane = lane & 15;
  const int row_lane = 4 * (lane >> 4);
  if (FC1) {
#pragma unroll
    for (int q = 0; q < WN / 2; ++q) {
      const int64_t ib = (nb0 + 2 * q) >> 1;  // intermediate 16-column block
      const int64_t c = ib * 16 + col_lane;
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        if (i >= nvalid) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = row_base + 16 * i + row_lane + v;
          if (r < row_end) {
            const float s = p.row_scale ? p.row_scale[p.row_token[r]] : 1.0f;
            const float g = acc[i][2 * q][v] * s;
            const float u = acc[i][2 * q + 1][v] * s;
            p.out[(int64_t)r * p.out_stride + c] = g / (1.0f + expf(-g)) * u;
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int64_t c = (nb0 + j) * 16 + col_lane;
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        if (i >= nvalid) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = row_base + 16 * i + row_lane + v;
          if (r < row_end) {
            const float s = p.row_scale ? p.row_scale[r] : 1.0f;
            p.out[(int64_t)r * p.out_stride + c] = acc[i][j][v] * s;
          }
        }
      }
    }
  }
}

template <int V, bool FC1>
static hipError_t launch_v(int cfg, const GemmParams& p, int64_t max_tiles, hipStream_t st) {
  const int64_t blocks = max_tiles * p.n_tiles;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  switch (cfg) {
    case 0: k_gemm<V, FC1, 1, 1, 2><<<(unsigned)blocks, 256, 0, st>>>(p); break;
    case 1: k_gemm<V, FC1, 1, 3, 2><<<(unsigned)blocks, 256, 0, st>>>(p); break;
    default: k_gemm<V, FC1, 2, 4, 4><<<(unsigned)blocks, 256, 0, st>>>(p); break;
  }
  return hipGetLastError();
}

hipError_t launch_gemm(int variant, bool fc1, int cfg, const GemmParams& p, int64_t max_tiles,
                       hipStream_t st) {
  switch (variant) {
    case kMxfp4Fp8: return fc1 ? launch_v<kMxfp4Fp8, true>(cfg, p, max_tiles, st)
                               : launch_v<kMxfp4Fp8, false>(cfg, p, max_tiles, st);
    case kMxfp4Bf16: return fc1 ? launch_v<kMxfp4Bf16, true>(cfg, p, max_tiles, st)
                                : launch_v<kMxfp4Bf16, false>(cfg, p, max_tiles, st);
    default: return fc1 ? launch_v<kInt4Fp8, true>(cfg, p, max_tiles, st)
                        : launch_v<kInt4Fp8, false>(cfg, p, max_tiles, st);
  }
}

}  // namespace moe
