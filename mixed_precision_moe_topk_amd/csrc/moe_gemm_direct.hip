// Register-direct grouped GEMM of the fused MoE (gfx950): each wave loads its
// own activation and weight fragments straight into MFMA operand registers,
// one or two K steps ahead.  Used for BF16 activations (the weights are expanded from
// E2M1 to bf16 in registers with the E8M0 scale folded in) and for the 16-row
// tiles of decode-sized batches, where the weight stream from HBM dominates.
#include "moe_gemm_common.h"

namespace moe {

// Block = 4 waves, WAVES_M x (4 / WAVES_M); each wave owns WM x WN 16x16
// output tiles (transposed accumulators, weights as the MFMA's A operand,
// except for INT4: see moe_gemm_common.h).
template <int V, bool FC1, int WAVES_M, int WM, int WN>
__global__ __launch_bounds__(256) void k_gemm(GemmParams p) {
  constexpr int WAVES_N = 4 / WAVES_M;
  constexpr int NA = Frag<V>::kA;
  constexpr bool MXA = a_blockscaled(V);
  constexpr int AF = a_fmt(V);
  static_assert(!FC1 || WN % 2 == 0, "FC1 pairs gate/up tiles");
  Tile tile;
  int nt;
  if (!work_item(p.tiles, p.num_tiles, p.n_tiles, p.pair_m, &tile, &nt)) return;
  // wave-uniform values are made scalar: a branch on a per-lane value is an
  // exec-masked branch, after which the compiler waits for every outstanding
  // load (that drained the one-step prefetch before each step's MFMAs)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = lane_id();
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int row_base = tile.row0 + 16 * WM * wm;
  const int row_end = tile.row0 + tile.nrows;
  const int nvalid = __builtin_amdgcn_readfirstlane(min(WM, (row_end - row_base + 15) / 16));
  if (nvalid <= 0) return;

  const int K = p.K;
  const int KS = K / kKStep, KS4 = (KS + 3) / 4;
  const int64_t e = tile.expert;
  const uint8_t* wbase = p.w + e * p.w_expert_stride;
  const uint8_t* sbase = p.s + e * p.s_expert_stride;
  const int64_t nb0 = (int64_t)nt * (WAVES_N * WN) + wn * WN;
  // N tail: 16-column blocks left
  const int jvalid = __builtin_amdgcn_readfirstlane((int)min<int64_t>(WN, p.N / 16 - nb0));
  if (jvalid <= 0) return;
  const int64_t nb_last = p.N / 16 - 1;

  // A row pointers (rows past the tile end re-read its last row; their
  // outputs are never stored)
  const uint8_t* arow[WM];
  const uint8_t* asrow[WM];
#pragma unroll
  for (int i = 0; i < WM; ++i) {
    const int r = min(row_base + 16 * i + (lane & 15), row_end - 1);
    const int64_t src = FC1 ? (int64_t)p.row_token[r] : (int64_t)r;
    int64_t off;
    if (scaled_fp4(V)) off = 16 * (lane >> 4);  // E4M3: bytes 16g.. (+64); E2M1: k 32g..
    else if (V == kInt4Fp8) off = 32 * (lane >> 4);
    else off = 64 * (lane >> 4);  // bf16: 32 elements * 2 bytes
    arow[i] = p.a + src * p.a_stride + off;
    // MXFP8: lane l supplies the E8M0 scales of its row for k-block l/16
    // (one dword per four steps, byte = step % 4)
    if (a_blockscaled(V)) asrow[i] = p.a_scale + src * p.a_scale_stride + 4 * (lane >> 4);
  }

  v4f acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  uint4 ac[WM][NA], an[WM][NA];
  uint4 bc[WN], bn[WN];
  uint32_t scc[WN], scn[WN];  // E8M0 dword (MXFP4) or float bits (INT4 group scale)
  uint32_t asc[WM], asn[WM];  // E8M0 A scale of this lane's row and k-block (MXFP8)

  // Loads are unconditional (subtiles past the tile end re-read its last row,
  // column blocks past N the last block; neither is stored), so no branch
  // sits between a load and its use.
  auto load = [&](int ks, uint4 (&a)[WM][NA], uint4 (&b)[WN], uint32_t (&sc)[WN],
                  uint32_t (&as)[WM]) {
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      if (a_fp4(V)) {
        a[i][0] = *reinterpret_cast<const uint4*>(arow[i] + ks * (kKStep / 2));
        as[i] = *reinterpret_cast<const uint32_t*>(asrow[i] + 16 * (ks >> 2));
      } else if (scaled_fp4(V)) {
        a[i][0] = *reinterpret_cast<const uint4*>(arow[i] + ks * kKStep);
        a[i][1] = *reinterpret_cast<const uint4*>(arow[i] + ks * kKStep + 64);
        if (a_blockscaled(V))
          as[i] = *reinterpret_cast<const uint32_t*>(asrow[i] + 16 * (ks >> 2));
      } else if (V == kInt4Fp8) {
        a[i][0] = *reinterpret_cast<const uint4*>(arow[i] + ks * kKStep);
        a[i][1] = *reinterpret_cast<const uint4*>(arow[i] + ks * kKStep + 16);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          a[i][q] = *reinterpret_cast<const uint4*>(arow[i] + 2 * ks * kKStep + 16 * q);
      }
    }
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int64_t nb = min(nb0 + j, nb_last);
      b[j] = *reinterpret_cast<const uint4*>(wbase + ((nb * KS + ks) * 64 + lane) * 16);
      if (V == kInt4Fp8)
        sc[j] = *reinterpret_cast<const uint32_t*>(sbase + ((nb * KS + ks) * 16 + (lane & 15)) * 4);
      else
        sc[j] = *reinterpret_cast<const uint32_t*>(sbase + ((nb * KS4 + (ks >> 2)) * 64 + lane) * 4);
    }
  };

  auto compute = [&](int ks, const uint4 (&a)[WM][NA], const uint4 (&b)[WN],
                     const uint32_t (&sc)[WN], const uint32_t (&as)[WM]) {
    if (scaled_fp4(V)) {
      v8i bop[WN];
#pragma unroll
      for (int j = 0; j < WN; ++j) bop[j] = fp4_operand(b[j]);
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        if (i < nvalid) {
          const v8i aop = a_fp4(V) ? fp4_operand(a[i][0]) : as_v8i(a[i][0], a[i][NA - 1]);
          const int sa = MXA ? (int)as[i] : 127;
#pragma unroll
          for (int j = 0; j < WN; ++j) {
            if (j >= jvalid) continue;
            // weights as the MFMA's A operand: transposed accumulators
            switch (ks & 3) {
              case 0: acc[i][j] = mfma_wt<AF, 0, 0>(bop[j], aop, acc[i][j], (int)sc[j], sa); break;
              case 1: acc[i][j] = mfma_wt<AF, 1, MXA ? 1 : 0>(bop[j], aop, acc[i][j], (int)sc[j], sa); break;
              case 2: acc[i][j] = mfma_wt<AF, 2, MXA ? 2 : 0>(bop[j], aop, acc[i][j], (int)sc[j], sa); break;
              default: acc[i][j] = mfma_wt<AF, 3, MXA ? 3 : 0>(bop[j], aop, acc[i][j], (int)sc[j], sa); break;
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
            if (j >= jvalid) continue;
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
        if (j >= jvalid) continue;
        const float scale = e8m0_to_float((sc[j] >> (8 * (ks & 3))) & 0xFFu);
        const uint32_t bw[4] = {b[j].x, b[j].y, b[j].z, b[j].w};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const v8bf bop = fp4x8_to_bf16(bw[s], scale);
#pragma unroll
          for (int i = 0; i < WM; ++i) {
            if (i < nvalid)  // weights as the A operand: transposed accumulators
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bop, as_bf16x8(a[i][s]),
                                                                  acc[i][j], 0, 0, 0);
          }
        }
      }
    }
  };

  // Prefetch step indices are clamped (the last step is reloaded, unused) so
  // every iteration issues the same loads and no load sits under a branch.
  // 16-row tiles (one subtile per wave, few registers) load two steps ahead
  // through three register sets (2 % faster on the decode GEMMs than one
  // step ahead); larger tiles one step ahead through two.
  int ks = 0;
  if constexpr (WM == 1) {
    uint4 a2[WM][NA];
    uint4 b2[WN];
    uint32_t sc2[WN], as2[WM];
    load(0, ac, bc, scc, asc);
    load(min(1, KS - 1), an, bn, scn, asn);
    for (; ks + 3 <= KS; ks += 3) {
      load(min(ks + 2, KS - 1), a2, b2, sc2, as2);
      compute(ks, ac, bc, scc, asc);
      load(min(ks + 3, KS - 1), ac, bc, scc, asc);
      compute(ks + 1, an, bn, scn, asn);
      load(min(ks + 4, KS - 1), an, bn, scn, asn);
      compute(ks + 2, a2, b2, sc2, as2);
    }
    if (ks < KS) compute(ks, ac, bc, scc, asc);
    if (ks + 1 < KS) compute(ks + 1, an, bn, scn, asn);
  } else {
    load(0, ac, bc, scc, asc);
    for (; ks + 2 <= KS; ks += 2) {
      load(min(ks + 1, KS - 1), an, bn, scn, asn);
      compute(ks, ac, bc, scc, asc);
      load(min(ks + 2, KS - 1), ac, bc, scc, asc);
      compute(ks + 1, an, bn, scn, asn);
    }
    if (ks < KS) compute(ks, ac, bc, scc, asc);
  }

  if constexpr (V == kInt4Fp8) {
    finish_tile<V, FC1, WM, WN>(p, acc, row_base, row_end, nvalid, nb0, jvalid, lane);
  } else {
    float sc[WM];
    load_row_scales_t<FC1, WM>(p, row_base, row_end, lane, sc);
    finish_tile_t<V, FC1, WM, WN>(p, acc, sc, row_base, row_end, nvalid, nb0, jvalid, lane);
  }
}


template <int V, bool FC1>
static hipError_t launch_v(int cfg, const GemmParams& p, int64_t blocks, hipStream_t st) {
  switch (cfg) {
    case 0: k_gemm<V, FC1, 1, 1, 4><<<(unsigned)blocks, 256, 0, st>>>(p); break;
    case 1: k_gemm<V, FC1, 1, 3, 2><<<(unsigned)blocks, 256, 0, st>>>(p); break;
    default: k_gemm<V, FC1, 2, 4, 4><<<(unsigned)blocks, 256, 0, st>>>(p); break;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_direct(int variant, bool fc1, int cfg, const GemmParams& p,
                              int64_t max_tiles, hipStream_t st) {
  const int64_t blocks = gemm_blocks(max_tiles, p.n_tiles);
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  switch (variant) {
    case kMxfp4Fp8: return fc1 ? launch_v<kMxfp4Fp8, true>(cfg, p, blocks, st)
                               : launch_v<kMxfp4Fp8, false>(cfg, p, blocks, st);
    case kMxfp4Bf16: return fc1 ? launch_v<kMxfp4Bf16, true>(cfg, p, blocks, st)
                                : launch_v<kMxfp4Bf16, false>(cfg, p, blocks, st);
    case kMxfp4Mxfp8: return fc1 ? launch_v<kMxfp4Mxfp8, true>(cfg, p, blocks, st)
                                 : launch_v<kMxfp4Mxfp8, false>(cfg, p, blocks, st);
    case kMxfp4Mxfp4: return fc1 ? launch_v<kMxfp4Mxfp4, true>(cfg, p, blocks, st)
                                 : launch_v<kMxfp4Mxfp4, false>(cfg, p, blocks, st);
    default: return fc1 ? launch_v<kInt4Fp8, true>(cfg, p, blocks, st)
                        : launch_v<kInt4Fp8, false>(cfg, p, blocks, st);
  }
}

// Tile configuration -> kernel: the register-direct kernel for 16-row tiles
// and BF16 activations, the LDS-staged kernels otherwise.
hipError_t launch_gemm(int variant, bool fc1, int cfg, const GemmParams& p, int64_t max_tiles,
                       hipStream_t st) {
  if (cfg == 0 || variant == kMxfp4Bf16) return launch_gemm_direct(variant, fc1, cfg, p, max_tiles, st);
  return launch_gemm_lds(variant, fc1, cfg, p, max_tiles, st);
}

}  // namespace moe
