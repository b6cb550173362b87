// LDS-staged grouped GEMMs of the fused MoE for E4M3 activations (gfx950):
// MXFP4 x FP8 on the block-scaled MFMA (per-token activation scales applied
// in the epilogue, or MXFP8 block scales as the MFMA's A scales), INT4 x FP8
// with codes mapped to E4M3 in registers and the group scale applied after
// each 128-wide K step.
#include "moe_gemm_common.h"

namespace moe {

// Scheduling hint for one K step: NMFMA MFMAs with NVMEM global loads and NDS
// LDS reads spread between them (two LDS reads first, for the first A
// fragment).  Only ordering hints; no effect on results.
template <int NMFMA, int NVMEM, int NDS>
__device__ __forceinline__ void interleave_schedule() {
  __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read
#pragma unroll
  for (int m = 0; m < NMFMA; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    if (m < NVMEM) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
    if (m + 1 < NMFMA && (m + 1) * (NDS - 2) / NMFMA != m * (NDS - 2) / NMFMA)
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
}

// ----------------------------------------------------------------------------
// LDS-staged grouped GEMM for E4M3 activations (MXFP4 x FP8, INT4 x FP8).
// Block = NW waves, WAVES_M x WAVES_N; each wave owns 16*WM rows and 16*WN
// device columns.  Per 128-wide K step the block stages the tile's A rows
// (gathered token rows for FC1) into LDS in MFMA fragment order: fragment
// (i, h) is 1 KB holding the 16-byte operand pieces of its 64 lanes; lane
// L = rho + 16g sits in 16-byte slot 16g + (rho ^ ((2g + h) | (rho & 1) << 3)),
// an XOR swizzle that keeps both the staging writes (8 threads = one row's 8
// chunks, 16 threads = two rows) and the fragment reads (consecutive lanes)
// on distinct LDS banks at 8- and 16-lane granularity.  Two LDS buffers, one
// barrier per step.  Global loads run two steps ahead:
// A into two register staging sets, weights (pre-shuffled, straight into the
// MFMA operand registers) into four register sets, so a load has two steps of
// MFMA work to arrive.  An MXFP4 scale word covers four K steps (one E8M0 byte
// per step), so it is loaded once per four steps; so are the INT4 group
// scales (one float per lane covering four steps of a 16-column block, read
// across lanes with ds_bpermute).  Rows past the tile end are loaded as
// copies of its last row and never stored; 16-row subtiles past the end are
// skipped.
// Body of k_gemm_lds for one work item.  FULL: the tile has BM rows and the
// wave's columns lie inside N (known per block), so every step is one basic
// block: no per-subtile branches, which lets the scheduling hints interleave
// MFMAs with the step's memory instructions.
template <int V, bool FC1, int NW, int WAVES_M, int WM, int WN, int PB, int AD, bool FULL>
__device__ __forceinline__ void gemm_lds_body(const GemmParams& p, uint8_t* lds, const Tile tile,
                                              const int nt) {
  static_assert(PB >= 1 && PB <= 3 && AD >= 2 && AD <= 4, "prefetch distances");
  constexpr int NB = (PB == 1) ? 2 : 4;  // weight register sets (prefetch distance PB)
  constexpr int AS = (AD == 2) ? 2 : 4;  // A staging register sets (prefetch distance AD)

  static_assert(scaled_fp4(V) || V == kInt4Fp8, "E4M3 or E2M1 activations only");
  static_assert(!FC1 || WN % 2 == 0, "FC1 pairs gate/up tiles");
  constexpr int NT = kWave * NW;           // threads per block
  constexpr int WAVES_N = NW / WAVES_M;
  constexpr int BM = 16 * WM * WAVES_M;
  static_assert(BM % 32 == 0, "BM must be a multiple of 32");
  constexpr bool MX = scaled_fp4(V);
  constexpr bool MXA = a_blockscaled(V);
  constexpr bool A4 = a_fp4(V);
  constexpr int AF = a_fmt(V);             // MFMA format code of A (a constant expression)
  constexpr int CPR = A4 ? 4 : 8;          // 16-byte chunks per A row and K step
  constexpr int NF = A4 ? 1 : 2;           // 1 KB operand fragments per 16 rows
  static_assert((BM * CPR) % NT == 0, "A stage must split evenly over the threads");
  constexpr int ABUF = BM * 16 * CPR;      // bytes of one A stage
  constexpr int NCH = BM * CPR / NT;       // 16-byte chunks per thread per stage

  // wave-uniform values are made scalar so that branches on them are scalar
  // branches (exec-masked branches make the compiler drain every outstanding
  // load at each join, which would serialise the prefetch)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = lane_id();
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int row_end = tile.row0 + tile.nrows;
  const int row_base = tile.row0 + 16 * WM * wm;
  const int nvalid = __builtin_amdgcn_readfirstlane(max(0, min(WM, (row_end - row_base + 15) / 16)));

  const int K = p.K;
  const int KS = K / kKStep, KS4 = (KS + 3) / 4;
  const int64_t e = tile.expert;
  const uint8_t* wbase = p.w + e * p.w_expert_stride;
  const uint8_t* sbase = p.s + e * p.s_expert_stride;
  const int64_t nb0 = (int64_t)nt * (WAVES_N * WN) + wn * WN;
  // N is a multiple of 128 and 16*WN divides 128, so a wave's columns are all
  // inside N or all past it (a wave with no rows or columns still stages A
  // and joins every barrier)
  static_assert(128 % (16 * WN) == 0, "wave columns must tile 128");
  const bool cols = __builtin_amdgcn_readfirstlane((int)(nb0 * 16 < p.N)) != 0;
  const int jvalid = cols ? WN : 0;

  // this thread's A chunks: tile row r, 16-byte column chunk c; source pointer
  // and LDS destination (fragment (r/16, h), lane (r%16) + 16*g; E2M1 rows
  // have one fragment per 16 rows, chunk c = the 32 elements of lane group c)
  const uint8_t* asrc[NCH];
  int adst[NCH];
#pragma unroll
  for (int u = 0; u < NCH; ++u) {
    const int q = threadIdx.x + NT * u;
    const int r = q / CPR, c = q % CPR;
    const int rr = min(tile.row0 + r, row_end - 1);
    const int64_t src = FC1 ? (int64_t)p.row_token[rr] : (int64_t)rr;
    asrc[u] = p.a + src * p.a_stride + 16 * c;
    int g, h;
    if (A4) { g = c; h = 0; }                        // k = 32g + [0,32)
    else if (MX) { g = c & 3; h = c >> 2; }          // k = 64h + 16g + [0,16)
    else { g = c >> 1; h = c & 1; }                  // k = 32g + 16h + [0,16)
    const int rho = r & 15;
    adst[u] = ((r >> 4) * NF + h) * 1024 + (16 * g + (rho ^ ((2 * g + h) | ((rho & 1) << 3)))) * 16;
  }
  // this lane's read offsets inside a fragment of half h = 0 / 1
  const int rho_l = lane & 15, g_l = lane >> 4;
  const int rd0 = (16 * g_l + (rho_l ^ ((2 * g_l) | ((rho_l & 1) << 3)))) * 16;
  const int rd1 = 1024 + (16 * g_l + (rho_l ^ ((2 * g_l + 1) | ((rho_l & 1) << 3)))) * 16;
  // MXFP8: this lane's A scale dwords (row of subtile i, k-block lane/16),
  // one per four steps like the weights' scale words
  const uint8_t* ascl[WM];
#pragma unroll
  for (int i = 0; i < WM; ++i) {
    if constexpr (MXA) {
      const int r = min(row_base + 16 * i + rho_l, row_end - 1);
      const int64_t src = FC1 ? (int64_t)p.row_token[r] : (int64_t)r;
      ascl[i] = p.a_scale + src * p.a_scale_stride + 4 * g_l;
    }
  }

  v4f acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  // per-token E4M3: row scales loaded before the K loop (their latency is
  // then not paid between the last MFMA and the first output store).  MXFP4
  // weights: transposed accumulators (weights as the MFMA's A operand), one
  // row scale per subtile; INT4: row-per-register accumulators, four
  constexpr bool TR = MX;
  float sc[WM][4];
  float sct[WM];
  if constexpr (V == kInt4Fp8) load_row_scales<FC1, WM>(p, row_base, row_end, lane, sc);
  if constexpr (V == kMxfp4Fp8) load_row_scales_t<FC1, WM>(p, row_base, row_end, lane, sct);
  if constexpr (TR && V != kMxfp4Fp8) {
#pragma unroll
    for (int i = 0; i < WM; ++i) sct[i] = 1.0f;
  }

  v4u ast[AS][NCH];
  uint4 bq[NB][WN];
  // MXFP4: E8M0 scale words of this / the next 4 steps.  INT4: lane L holds
  // the float32 group scale of column L%16 at step 4g + L/16 of this / the
  // next 4-step group g (the layout keeps those 64 floats contiguous); an
  // MFMA lane takes its column's scale for step S from lane L%16 + 16 S.
  uint32_t sx[WN], sx_next[WN];
  uint32_t ax[WM], ax_next[WM];  // MXFP8 A scale dwords of this / the next 4 steps

  auto load_a = [&](int ks, v4u (&dst)[NCH]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NCH; ++u) dst[u] = *reinterpret_cast<const v4u*>(asrc[u] + ks * (16 * CPR));
  };
  auto store_a = [&](int buf, const v4u (&src)[NCH]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NCH; ++u) *reinterpret_cast<v4u*>(lds + buf * ABUF + adst[u]) = src[u];
  };
  // Weight loads are unconditional: a wave past the end of N reloads the last
  // column block (never used).  A branch around them would make the
  // compiler's wait counts assume they may be missing and drain the prefetch.
  const int64_t nb_last = p.N / 16 - 1;
  auto load_b = [&](int ks, uint4 (&b)[WN]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int64_t nb = min(nb0 + j, nb_last);
      b[j] = *reinterpret_cast<const uint4*>(wbase + ((nb * KS + ks) * 64 + lane) * 16);
    }
  };
  auto load_sx = [&](int ks, uint32_t (&sc)[WN]) __attribute__((always_inline)) {
    // INT4: step 4g + L/16 of the group, clamped to the last step (unused)
    const int64_t gstep = min(((ks >> 2) << 2) + (lane >> 4), KS - 1);
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int64_t nb = min(nb0 + j, nb_last);
      if constexpr (MX)
        sc[j] = *reinterpret_cast<const uint32_t*>(sbase + ((nb * KS4 + (ks >> 2)) * 64 + lane) * 4);
      else
        sc[j] = *reinterpret_cast<const uint32_t*>(sbase + ((nb * KS + gstep) * 16 + (lane & 15)) * 4);
    }
    if constexpr (MXA) {
#pragma unroll
      for (int i = 0; i < WM; ++i)
        ax_next[i] = *reinterpret_cast<const uint32_t*>(ascl[i] + 16 * (ks >> 2));
    }
  };

  // K step ks with S = ks % 4 (E8M0 byte select and register-set index).
  // Prefetch loads are unconditional (their step index is clamped to the
  // last step) so that the steady-state loop has no branches around memory
  // operations and the compiler's wait counts stay exact.
  auto step = [&](auto s_c, int ks) __attribute__((always_inline)) {
    constexpr int S = decltype(s_c)::value;
    // the scale words of steps ks..ks+3 were loaded PB steps ago
    if constexpr (S == 0) {
#pragma unroll
      for (int j = 0; j < WN; ++j) sx[j] = sx_next[j];
      if constexpr (MXA) {
#pragma unroll
        for (int i = 0; i < WM; ++i) ax[i] = ax_next[i];
      }
    }
    load_a(min(ks + AD, KS - 1), ast[(S + AD) % AS]);
    load_b(min(ks + PB, KS - 1), bq[(S + PB) % NB]);
    constexpr bool LOAD_SX = (S + PB) % 4 == 0;
    if constexpr (LOAD_SX) load_sx(min(ks + PB, KS - 1), sx_next);
    const uint8_t* abuf = lds + (S & 1) * ABUF + (WM * wm) * (NF * 1024);
    v8i bop[WN];
    float gs[WN];  // INT4: this step's group scale of the lane's column
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      bop[j] = MX ? fp4_operand(bq[S % NB][j]) : int4_operand(bq[S % NB][j]);
      if constexpr (!MX)
        gs[j] = __uint_as_float(__builtin_amdgcn_ds_bpermute(((lane & 15) + 16 * S) << 2, (int)sx[j]));
    }
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      if (FULL || (cols && i < nvalid)) {
        const uint4 lo = *reinterpret_cast<const uint4*>(abuf + (NF * i) * 1024 + rd0);
        v8i aop;
        if constexpr (A4) {
          aop = fp4_operand(lo);
        } else {
          const uint4 hi = *reinterpret_cast<const uint4*>(abuf + (NF * i) * 1024 + rd1);
          aop = as_v8i(lo, hi);
        }
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          if constexpr (MX) {
            acc[i][j] = mfma_wt<AF, S, MXA ? S : 0>(bop[j], aop, acc[i][j], (int)sx[j],
                                                   MXA ? (int)ax[i] : 127);
          } else {
            const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                aop, bop[j], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[i][j][v] += part[v] * gs[j];
          }
        }
      }
    }
    // issue order inside the step: the wave's global loads and LDS reads are
    // spread between its MFMAs so they issue while the matrix pipe is busy
    if (FULL) interleave_schedule<WM * WN, (LOAD_SX ? 2 : 1) * WN + NCH + (LOAD_SX && MXA ? WM : 0), NF * WM>();
    __builtin_amdgcn_sched_barrier(0);
    // A of step ks+1 (a harmless copy of the last step once past the end)
    store_a((S + 1) & 1, ast[(S + 1) % AS]);
    __syncthreads();
  };

  // Prologue loads in step order.  The fences keep the scheduler from sinking
  // the first step's weight loads behind later ones: the wait counts at the
  // loop head are the minimum over the entry and back-edge paths, so a late
  // load here would tighten every iteration's waits.
  load_a(0, ast[0]);
  load_b(0, bq[0]);
  load_sx(0, sx_next);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 1; i < AD; ++i) {
    load_a(min(i, KS - 1), ast[i]);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int i = 1; i < PB; ++i) {
    load_b(min(i, KS - 1), bq[i]);
    __builtin_amdgcn_sched_barrier(0);
  }
  store_a(0, ast[0]);
  __syncthreads();
  int ks = 0;
  for (; ks + 4 <= KS; ks += 4) {
    step(std::integral_constant<int, 0>{}, ks);
    step(std::integral_constant<int, 1>{}, ks + 1);
    step(std::integral_constant<int, 2>{}, ks + 2);
    step(std::integral_constant<int, 3>{}, ks + 3);
  }
  if (ks < KS) step(std::integral_constant<int, 0>{}, ks);
  if (ks + 1 < KS) step(std::integral_constant<int, 1>{}, ks + 1);
  if (ks + 2 < KS) step(std::integral_constant<int, 2>{}, ks + 2);
  if constexpr (TR)
    finish_tile_t<V, FC1, WM, WN>(p, acc, sct, row_base, row_end, nvalid, nb0, jvalid, lane);
  else
    epilogue_sc<FC1, WM, WN>(p, acc, sc, row_base, row_end, nvalid, nb0, jvalid, lane);
}

template <int V, bool FC1, int NW, int WAVES_M, int WM, int WN, int MINB = 2, int PB = 2,
          int AD = 2>
__global__ __launch_bounds__(kWave * NW, MINB) void k_gemm_lds(GemmParams p) {
  constexpr int BM = 16 * WM * WAVES_M;
  constexpr int BN = 16 * WN * (NW / WAVES_M);
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * BM * kKStep];
  Tile tile;
  int nt;
  if (!work_item(p.tiles, p.num_tiles, p.n_tiles, p.pair_m, &tile, &nt)) return;
  const bool full = tile.nrows == BM && (int64_t)(nt + 1) * BN <= p.N;
  if (full) gemm_lds_body<V, FC1, NW, WAVES_M, WM, WN, PB, AD, true>(p, lds, tile, nt);
  else gemm_lds_body<V, FC1, NW, WAVES_M, WM, WN, PB, AD, false>(p, lds, tile, nt);
}

// Scheduling hint for one K step of the two-operand LDS kernel: the step's
// weight fragments and first activation fragment are read first, then the
// MFMAs with the remaining LDS reads and the global loads spread between them.
template <int NMFMA, int NVMEM, int NDS_FIRST, int NDS_REST>
__device__ __forceinline__ void interleave_schedule_ab() {
  __builtin_amdgcn_sched_group_barrier(0x100, NDS_FIRST, 0);  // DS read
#pragma unroll
  for (int m = 0; m < NMFMA; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    if (m < NVMEM) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
    if (m + 1 < NMFMA && (m + 1) * NDS_REST / NMFMA != m * NDS_REST / NMFMA)
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
}

// ----------------------------------------------------------------------------
// Grouped GEMM with both operands staged through LDS (INT4 weights x E4M3
// activations, 128-row tiles).
// Block = NW waves, WAVES_M x WAVES_N, each wave 16*WM rows x 16*WN device
// columns; block tile BM x BN.  A per-thread global load carries at most one
// 16-byte chunk of the step's A tile or weight tile, so every weight byte
// reaches the CU once per block instead of once per wave row, which halves
// the global-load bytes per MFMA against register-direct weights (the vector
// memory path, not HBM, bounds the prefill GEMMs).  Per 128-wide K step and
// LDS stage: A in the swizzled fragment order of gemm_lds_body, then the
// block's weight fragments in their device order (16-column block b at
// b * 1 KB, lane l's 16 bytes at l * 16: reads and writes are conflict-free).
// Two stages, one barrier per step; global loads run two steps ahead through
// two register staging sets.  The group scales go straight to registers.
template <int V, bool FC1, int NW, int WAVES_M, int WM, int WN, bool FULL>
__device__ __forceinline__ void gemm_ab_body(const GemmParams& p, uint8_t* lds, const Tile tile,
                                             const int nt) {
  static_assert(V == kInt4Fp8, "INT4 weights x E4M3 activations");
  static_assert(!FC1 || WN % 2 == 0, "FC1 pairs gate/up tiles");
  constexpr int NT = kWave * NW;
  constexpr int WAVES_N = NW / WAVES_M;
  constexpr int BM = 16 * WM * WAVES_M;
  constexpr int BNB = WAVES_N * WN;        // 16-column blocks per block tile
  constexpr int ABUF = BM * kKStep;        // A bytes of one stage
  constexpr int SBUF = ABUF + BNB * 1024;  // bytes of one stage
  constexpr int NCA = BM * 8 / NT;         // A chunks per thread per step
  constexpr int NCB = BNB * 64 / NT;       // weight chunks per thread per step
  static_assert(NCA * NT == BM * 8 && NCB * NT == BNB * 64, "chunks must split evenly");
  static_assert(128 % (16 * WN) == 0, "wave columns must tile 128");

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = lane_id();
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int row_end = tile.row0 + tile.nrows;
  const int row_base = tile.row0 + 16 * WM * wm;
  const int nvalid = __builtin_amdgcn_readfirstlane(max(0, min(WM, (row_end - row_base + 15) / 16)));

  const int K = p.K;
  const int KS = K / kKStep;
  const int64_t e = tile.expert;
  const uint8_t* wbase = p.w + e * p.w_expert_stride;
  const uint8_t* sbase = p.s + e * p.s_expert_stride;
  const int64_t nbb = (int64_t)nt * BNB;   // first 16-column block of the tile
  const int64_t nb0 = nbb + wn * WN;       // first 16-column block of this wave
  const bool cols = __builtin_amdgcn_readfirstlane((int)(nb0 * 16 < p.N)) != 0;
  const int jvalid = cols ? WN : 0;
  const int64_t nb_last = p.N / 16 - 1;

  // A chunks: tile row r, 16-byte column chunk c (as in gemm_lds_body)
  const uint8_t* asrc[NCA];
  int adst[NCA];
#pragma unroll
  for (int u = 0; u < NCA; ++u) {
    const int q = threadIdx.x + NT * u;
    const int r = q >> 3, c = q & 7;
    const int rr = min(tile.row0 + r, row_end - 1);
    const int64_t src = FC1 ? (int64_t)p.row_token[rr] : (int64_t)rr;
    asrc[u] = p.a + src * p.a_stride + 16 * c;
    const int g = c >> 1, h = c & 1;  // k = 32g + 16h + [0,16)
    const int rho = r & 15;
    adst[u] = ((r >> 4) * 2 + h) * 1024 + (16 * g + (rho ^ ((2 * g + h) | ((rho & 1) << 3)))) * 16;
  }
  // weight chunks: chunk q is lane slot q % 64 of local 16-column block q / 64
  // (blocks past N reload the last block; their columns are never used)
  const uint8_t* bsrc[NCB];
#pragma unroll
  for (int u = 0; u < NCB; ++u) {
    const int q = threadIdx.x + NT * u;
    const int64_t nb = min(nbb + (q >> 6), nb_last);
    bsrc[u] = wbase + (nb * KS * 64 + (q & 63)) * 16;
  }
  const int rho_l = lane & 15, g_l = lane >> 4;
  const int rd0 = (16 * g_l + (rho_l ^ ((2 * g_l) | ((rho_l & 1) << 3)))) * 16;
  const int rd1 = 1024 + (16 * g_l + (rho_l ^ ((2 * g_l + 1) | ((rho_l & 1) << 3)))) * 16;
  const int rdb = ABUF + wn * WN * 1024 + lane * 16;

  v4f acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  v4u ast[2][NCA], bst[2][NCB];
  uint32_t sq[4][WN];  // group scales of steps ks .. ks+3 (mod 4)

  auto load_ab = [&](int ks, v4u (&da)[NCA], v4u (&db)[NCB]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NCA; ++u) da[u] = *reinterpret_cast<const v4u*>(asrc[u] + ks * kKStep);
#pragma unroll
    for (int u = 0; u < NCB; ++u) db[u] = *reinterpret_cast<const v4u*>(bsrc[u] + ks * 1024);
  };
  auto store_ab = [&](int buf, const v4u (&sa)[NCA], const v4u (&sb)[NCB]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NCA; ++u) *reinterpret_cast<v4u*>(lds + buf * SBUF + adst[u]) = sa[u];
#pragma unroll
    for (int u = 0; u < NCB; ++u)
      *reinterpret_cast<v4u*>(lds + buf * SBUF + ABUF + (threadIdx.x + NT * u) * 16) = sb[u];
  };
  auto load_sq = [&](int ks, uint32_t (&sc)[WN]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int64_t nb = min(nb0 + j, nb_last);
      sc[j] = *reinterpret_cast<const uint32_t*>(sbase + ((nb * KS + ks) * 16 + (lane & 15)) * 4);
    }
  };
  auto step = [&](auto s_c, int ks) __attribute__((always_inline)) {
    constexpr int S = decltype(s_c)::value;
    const int kp = min(ks + 2, KS - 1);
    load_ab(kp, ast[S & 1], bst[S & 1]);
    load_sq(kp, sq[(S + 2) % 4]);
    const uint8_t* sbuf = lds + (S & 1) * SBUF;
    v8i bop[WN];
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const uint4 b = *reinterpret_cast<const uint4*>(sbuf + rdb + j * 1024);
      bop[j] = int4_operand(b);
    }
    const uint8_t* abuf = sbuf + (WM * wm) * 2048;
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      if (FULL || (cols && i < nvalid)) {
        const uint4 lo = *reinterpret_cast<const uint4*>(abuf + (2 * i) * 1024 + rd0);
        const uint4 hi = *reinterpret_cast<const uint4*>(abuf + (2 * i) * 1024 + rd1);
        const v8i aop = as_v8i(lo, hi);
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              aop, bop[j], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
          const float gs = __uint_as_float(sq[S][j]);
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[i][j][v] += part[v] * gs;
        }
      }
    }
    if (FULL) interleave_schedule_ab<WM * WN, NCA + NCB + WN, WN + 2, 2 * WM - 2>();
    __builtin_amdgcn_sched_barrier(0);
    // operands of step ks+1 (harmless copies of the last step once past the end)
    store_ab((S + 1) & 1, ast[(S + 1) & 1], bst[(S + 1) & 1]);
    __syncthreads();
  };

  // prologue loads in step order (fenced: see gemm_lds_body)
  load_ab(0, ast[0], bst[0]);
  load_sq(0, sq[0]);
  __builtin_amdgcn_sched_barrier(0);
  load_ab(min(1, KS - 1), ast[1], bst[1]);
  load_sq(min(1, KS - 1), sq[1]);
  __builtin_amdgcn_sched_barrier(0);
  store_ab(0, ast[0], bst[0]);
  __syncthreads();
  int ks = 0;
  for (; ks + 4 <= KS; ks += 4) {
    step(std::integral_constant<int, 0>{}, ks);
    step(std::integral_constant<int, 1>{}, ks + 1);
    step(std::integral_constant<int, 2>{}, ks + 2);
    step(std::integral_constant<int, 3>{}, ks + 3);
  }
  if (ks < KS) step(std::integral_constant<int, 0>{}, ks);
  if (ks + 1 < KS) step(std::integral_constant<int, 1>{}, ks + 1);
  if (ks + 2 < KS) step(std::integral_constant<int, 2>{}, ks + 2);
  finish_tile<V, FC1, WM, WN>(p, acc, row_base, row_end, nvalid, nb0, jvalid, lane);
}

template <int V, bool FC1, int NW, int WAVES_M, int WM, int WN, int MINB = 1>
__global__ __launch_bounds__(kWave * NW, MINB) void k_gemm_ab(GemmParams p) {
  constexpr int BM = 16 * WM * WAVES_M;
  constexpr int BN = 16 * WN * (NW / WAVES_M);
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * (BM * kKStep + BN * 64)];
  Tile tile;
  int nt;
  if (!work_item(p.tiles, p.num_tiles, p.n_tiles, p.pair_m, &tile, &nt)) return;
  const bool full = tile.nrows == BM && (int64_t)(nt + 1) * BN <= p.N;
  if (full) gemm_ab_body<V, FC1, NW, WAVES_M, WM, WN, true>(p, lds, tile, nt);
  else gemm_ab_body<V, FC1, NW, WAVES_M, WM, WN, false>(p, lds, tile, nt);
}

// ----------------------------------------------------------------------------
// Direct-to-LDS grouped GEMM for MXFP4 weights, 160 x 512 block tiles (WM = 5).
// 8 waves (2 x 4), each 80 rows (every second 16-row group of the tile) x
// 128 device columns (5 x 8 MFMA tiles), so
// one K step reads 18 KB of operands from LDS per 40 MFMAs per wave (40%
// less LDS traffic per MFMA than 64 x 64 wave tiles).  160-row tiles
// let one tile hold an expert of up to 160 rows: a tile costs about the same
// whether full or not (its weight stream dominates), so fewer tiles per
// expert is what counts.  With MXFP8 activations the waves also hold
// activation scales; that variant reads each subtile's A fragment and scale
// just before its MFMAs (two live at a time instead of five), which keeps
// the 5 x 8 wave tile within 256 registers.
// Operands reach LDS by global_load_lds (16 bytes per lane, lane L of a wave
// instruction lands at M0 + 16 L; an SALU write of M0 needs one wait state
// before the load reads it), so no staging registers are needed:
//   A       2 stages x 20 KB  16-row group g at 2g KB: E4M3 rows 0-7 in its
//                             first KB, rows 8-15 in the second, each KB
//                             8 rows x 128 bytes chunk-major (chunk c of
//                             row r at 16 (8c + r)), so one load moves
//                             whole 128-byte lines; E2M1 (64 bytes per row
//                             and step): 1 KB per group, lane L's piece at
//                             16 L
//   weights 3 stages x 32 KB  16-column block b at b KB, in device order
//   scales  2 slots x 8 KB (one 4-step group of E8M0 words each), block b
//           at 256 b
//   MXFP8 activation scales  2 slots x 3 KB (one 4-step group each): tile row
//           r's 16 bytes at 16 r, loaded by waves 0-2 (64 rows each)
// Step ks issues A of ks+1, weights of ks+2 and, at the
// start of a 4-step group, the next group's MXFP4 scale words (and, before
// the A loads, the next group's activation scales); the wave then
// waits until its loads of step ks+1 have landed (the vector memory counter
// counts these loads in issue order) and joins the block barrier.  Every
// load's step index is clamped to the last step, so the number of loads per
// step, and with it every wait count, is fixed.  The loads are inline
// assembly: the compiler does not track them, which keeps its conservative
// full drains out of the loop; the kernel drains them itself before the
// epilogue (an LDS write landing after the block exits would corrupt the next
// block's LDS): at the start of the peeled last step when K is a multiple of
// 512, else after the last step.
namespace dma {
constexpr int kNW = 8, kWN = 8, kWavesN = 4;
constexpr int kBNB = kWavesN * kWN;     // 16-column blocks per tile
constexpr int kBPW = kBNB / kNW;        // weight blocks loaded per wave
static_assert(kBPW * kNW == kBNB, "weight blocks per wave");
constexpr int kBBuf = kBNB * 1024, kSxSlot = kBNB * 256;
// LDS map of a tile whose waves own WM 16-row subtiles each (MXA: with the
// activation-scale slots; A4: E2M1 activations, 64 bytes per row and step)
template <int WM, bool MXA, bool A4>
struct Map {
  static constexpr int kBM = 2 * 16 * WM;   // tile rows
  static constexpr int kRG = kBM / 16;      // 16-row groups (wave w loads w and w + 8)
  static_assert(kRG >= kNW && kRG <= 2 * kNW, "row groups per wave");
  static constexpr int kNF = A4 ? 1 : 2;    // 1 KB operand fragments per 16 rows
  static constexpr int kABuf = kBM * 16 * 4 * kNF;
  static constexpr int kAOff = 0, kBOff = 2 * kABuf, kSOff = kBOff + 3 * kBBuf;
  static constexpr int kAsDma = (kBM + 63) / 64;  // activation-scale loads per group (waves 0..)
  static constexpr int kAsSlot = kAsDma * 1024, kAsOff = kSOff + 2 * kSxSlot;
  static constexpr int kBytes = kAsOff + (MXA ? 2 * kAsSlot : 0);
  static_assert(kBytes <= 160 * 1024, "LDS of one CU");
};
}  // namespace dma

__device__ __forceinline__ void lds_dma16(const void* gaddr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(gaddr), "s"(lds_addr) : "memory", "m0");
}
__device__ __forceinline__ void lds_dma16_s(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds_addr) : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4_s(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds_addr) : "memory", "m0");
}
// Wait until at most N of this wave's loads are outstanding, then block barrier.
template <int N>
__device__ __forceinline__ void wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(N) : "memory");
}

// One code path for full and partial tiles: the per-subtile checks are scalar
// branches, which also keep the compiler from hoisting every fragment read of
// a step (a branch-free full-tile path needed more than 256 registers here).
template <int V, bool FC1, int WM, bool PEEL>
__device__ __forceinline__ void gemm_dma_body(const GemmParams& p, uint8_t* lds, const Tile tile,
                                              const int nt) {
  using namespace dma;
  static_assert(scaled_fp4(V), "MXFP4 weights x E4M3 or E2M1 activations only");
  constexpr bool MXA = a_blockscaled(V);
  constexpr bool A4 = a_fp4(V);
  constexpr int AF = a_fmt(V);
  constexpr int WN = kWN;
  using L = Map<WM, MXA, A4>;
  constexpr int NF = L::kNF;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = lane_id();
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  // Wave row wm owns the tile's 16-row groups 2i + wm (i < WM), so a partly
  // filled tile splits its groups evenly between the two waves of a SIMD
  // (an expert of 128 rows in a 160-row tile: 4 + 4 subtiles, not 5 + 3)
  constexpr int RS = 32;                   // rows between a wave's subtiles
  constexpr int kSub = 2 * NF * 1024;      // LDS bytes between a wave's A subtiles
  constexpr int kSaSub = 2 * 16 * 16;      // the same for the MXFP8 A scales
  const int row_end = tile.row0 + tile.nrows;
  const int row_base = tile.row0 + 16 * wm;
  const int ngroups = (tile.nrows + 15) / 16;
  const int nvalid = __builtin_amdgcn_readfirstlane(max(0, min(WM, (ngroups - wm + 1) / 2)));
  const int K = p.K;
  const int KS = K / kKStep, KS4 = (KS + 3) / 4;
  const int64_t e = tile.expert;
  const uint8_t* wbase = p.w + e * p.w_expert_stride;
  const uint8_t* sbase = p.s + e * p.s_expert_stride;
  const int64_t nbb = (int64_t)nt * kBNB;
  const int64_t nb0 = nbb + wn * WN;
  const bool cols = __builtin_amdgcn_readfirstlane((int)(nb0 * 16 < p.N)) != 0;
  const int jvalid = cols ? WN : 0;
  const int64_t nb_last = p.N / 16 - 1;
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;

  // A: this wave loads fragments (g, 0) and (g, 1) of row groups g = wave and
  // (waves below L::kRG - 8) g = wave + 8: row 16 g + L%16 of the tile (the
  // last row repeated past the end), operand piece L/16
  const bool two_rg = wave < L::kRG - kNW;  // compile-time false when L::kRG == kNW
  // E4M3 A: one load covers 8 rows x 128 bytes (lane L: row L % 8, 16-byte
  // chunk L / 8), two loads a 16-row group, so each load fetches whole
  // 128-byte lines (with 16 rows x 64 bytes, the layout the MFMA lanes read,
  // every load touched 16 half lines: same-box, DeepSeek-V4-Pro GEMM2
  // 2.115 -> 2.085 ms, DeepSeek-V3 prefill GEMM1 0.865 -> 0.855 ms);
  // E2M1 A: 16 rows x 64 bytes
  const int kofs = A4 ? 16 * (lane >> 4) : 16 * (lane >> 3);
  const int rl = A4 ? (lane & 15) : (lane & 7);
  auto arow = [&](int r) __attribute__((always_inline)) {
    const int rr = min(r, row_end - 1);
    return p.a + (FC1 ? (int64_t)p.row_token[rr] : (int64_t)rr) * p.a_stride + kofs;
  };
  const uint8_t* arow0 = arow(tile.row0 + 16 * wave + rl);
  const uint8_t* arow1 = arow(tile.row0 + 16 * (wave + kNW) + rl);
  const uint8_t* arow0h = A4 ? arow0 : arow(tile.row0 + 16 * wave + 8 + rl);
  const uint8_t* arow1h = A4 ? arow1 : arow(tile.row0 + 16 * (wave + kNW) + 8 + rl);
  // weights: this wave loads 16-column blocks kBPW wave + u (clamped to N)
  const uint8_t* wcol[kBPW];
#pragma unroll
  for (int u = 0; u < kBPW; ++u) wcol[u] = wbase + min(nbb + kBPW * wave + u, nb_last) * KS * 1024;

  auto issue_a = [&](int ks, int stage) __attribute__((always_inline)) {
    const uint32_t dst = lds0 + L::kAOff + stage * L::kABuf + wave * (NF * 1024);
    if constexpr (A4) {  // one fragment per 16 rows: k = 32 (L/16) + [0, 32)
      lds_dma16(arow0 + ks * (kKStep / 2), dst);
      if (two_rg) lds_dma16(arow1 + ks * (kKStep / 2), dst + kNW * 1024);
    } else {
      lds_dma16(arow0 + ks * kKStep, dst);
      lds_dma16(arow0h + ks * kKStep, dst + 1024);
      if (two_rg) {
        lds_dma16(arow1 + ks * kKStep, dst + kNW * 2048);
        lds_dma16(arow1h + ks * kKStep, dst + kNW * 2048 + 1024);
      }
    }
  };
  auto issue_b = [&](int ks, int stage) __attribute__((always_inline)) {
    const uint32_t dst = lds0 + L::kBOff + stage * kBBuf + wave * kBPW * 1024;
#pragma unroll
    for (int u = 0; u < kBPW; ++u) lds_dma16_s(wcol[u] + ks * 1024, lane * 16, dst + u * 1024);
  };
  // half h (0 or 1) of issue_b's loads
  auto issue_b_part = [&](int ks, int stage, int h) __attribute__((always_inline)) {
    const uint32_t dst = lds0 + L::kBOff + stage * kBBuf + wave * kBPW * 1024;
#pragma unroll
    for (int u = h * (kBPW / 2); u < (h + 1) * (kBPW / 2); ++u)
      lds_dma16_s(wcol[u] + ks * 1024, lane * 16, dst + u * 1024);
  };
  // MXFP8: wave w < L::kAsDma loads the activation-scale group of tile rows
  // 64 w + L (the last row repeated past the end); a 32-bit offset from the
  // scale array (its size is checked on the host) saves a register pair
  uint32_t asoff = 0;
  if constexpr (MXA) {
    const int r = min(tile.row0 + 64 * min(wave, L::kAsDma - 1) + lane, row_end - 1);
    asoff = (uint32_t)((FC1 ? (int64_t)p.row_token[r] : (int64_t)r) * p.a_scale_stride);
  }
  auto issue_as = [&](int grp, int slot) __attribute__((always_inline)) {
    if (MXA && wave < L::kAsDma)
      lds_dma16_s(p.a_scale, asoff + 16 * grp, lds0 + L::kAsOff + slot * L::kAsSlot + wave * 1024);
  };
  auto issue_sx = [&](int grp, int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kBPW; ++u) {
      const uint8_t* src = sbase + (min(nbb + kBPW * wave + u, nb_last) * KS4 + grp) * 256;
      lds_dma4_s(src, lane * 4, lds0 + L::kSOff + slot * kSxSlot + (wave * kBPW + u) * 256);
    }
  };

  v4f acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  // per-token E4M3: the row scales are loaded before the K loop, so their
  // latency (two dependent loads through row_token for GEMM1) is not paid
  // between the last MFMA and the first output store; with the transposed
  // accumulators a lane holds one row per subtile, so one scale each
  float sc[WM];
  if constexpr (!MXA) load_row_scales_t<FC1, WM, RS>(p, row_base, row_end, lane, sc);
  else {
#pragma unroll
    for (int i = 0; i < WM; ++i) sc[i] = 1.0f;
  }
  uint32_t sx[WN];
  uint4 alo[2], ahi[2];  // A fragment halves, two subtiles in flight
  int axr[2];            // MXFP8: the A scale dwords of those subtiles

  // LDS addresses of this lane's fragments: weights of B stage bst, A of
  // A stage ast, weight scale words and MXFP8 A scales of step ksx's group
  auto b_at = [&](int bst) __attribute__((always_inline)) {
    return lds + L::kBOff + bst * kBBuf + (wn * WN) * 1024 + lane * 16;
  };
  // MFMA lane (r, g) = (lane % 16, lane / 16): its low operand piece (k =
  // 16 g + [0, 16)) is chunk g of row r, at byte ((r / 8) * 64 + 8 g + r % 8) * 16
  // of the group; the high piece (k = 64 + 16 g + [0, 16)) 512 bytes later
  const int aoff = A4 ? lane * 16 : (((lane >> 3) & 1) * 64 + 8 * (lane >> 4) + (lane & 7)) * 16;
  auto a_at = [&](int ast) __attribute__((always_inline)) {
    return lds + L::kAOff + ast * L::kABuf + wm * (NF * 1024) + aoff;
  };
  auto sx_at = [&](int ksx) __attribute__((always_inline)) {
    return lds + L::kSOff + ((ksx >> 2) & 1) * kSxSlot + (wn * WN) * 256 + lane * 4;
  };
  // MXFP8: A scale dword of subtile i is at + kSaSub i (row lane%16, k-block lane/16)
  auto sa_at = [&](int ksx) __attribute__((always_inline)) {
    return lds + L::kAsOff + ((ksx >> 2) & 1) * L::kAsSlot + (16 * wm + (lane & 15)) * 16 +
           4 * (lane >> 4);
  };
  auto read_a = [&](const uint8_t* as, const uint8_t* sa, int i, int buf)
                    __attribute__((always_inline)) {
    alo[buf] = *reinterpret_cast<const uint4*>(as + i * kSub);
    if constexpr (!A4) ahi[buf] = *reinterpret_cast<const uint4*>(as + i * kSub + 512);
    if constexpr (MXA) axr[buf] = *reinterpret_cast<const int*>(sa + i * kSaSub);
  };

  // loads per step after the A loads (which come first, 2 or 4 per wave):
  // weights (kBPW) and, at the start of a group, the scale words (kBPW)
  auto step = [&](auto s_c, int ks, int bstage) __attribute__((always_inline)) {
    constexpr int S = decltype(s_c)::value;
    // The step's direct-to-LDS loads are issued in four parts between the
    // MFMA groups of subtiles 0-3, in the order activation scales, A,
    // weights, scale words (the wait below relies on it).  Issued all at the
    // top of the step, the eight waves' ~100 loads per CU queued in the
    // address unit, and each wave's fragment reads and MFMAs waited behind
    // its own loads (1,100-2,000 cycles per step, measured with s_memtime).
    const int bnext = bstage == 0 ? 2 : bstage - 1;
    auto issue_part = [&](int part) __attribute__((always_inline)) {
      if (part == 0) {
        if constexpr (MXA && S == 0) issue_as(min((ks >> 2) + 1, KS4 - 1), ((ks >> 2) + 1) & 1);
        issue_a(min(ks + 1, KS - 1), (S + 1) & 1);
      } else if (part == 1) {
        issue_b_part(min(ks + 2, KS - 1), bnext, 0);
      } else if (part == 2) {
        issue_b_part(min(ks + 2, KS - 1), bnext, 1);
      } else if (part == 3) {
        if constexpr (S == 0) issue_sx(min((ks >> 2) + 1, KS4 - 1), ((ks >> 2) + 1) & 1);
      }
    };
    // all of the step's weight fragments are read after the barrier that
    // ends the previous step
    const uint8_t* bs = b_at(bstage);
    if constexpr (S == 0) {
      const uint8_t* ss = sx_at(ks);
#pragma unroll
      for (int j = 0; j < WN; ++j) sx[j] = *reinterpret_cast<const uint32_t*>(ss + j * 256);
    }
    const uint8_t* sa = sa_at(ks);
    const uint8_t* as = a_at(S & 1);
    v8i bop[WN];
    if constexpr (!A4) {
      // E4M3 codes (per-token or MXFP8), both GEMMs: LDS reads in MFMA
      // order, the A fragment (and MXFP8 scale) of subtile 0 and the weight
      // fragments first, then those of subtile i + 1 while the MFMAs of
      // subtile i run, so a subtile's MFMAs do not wait for its own reads.
      // Only two A fragments are live at a time (the MXFP8 activation
      // scales fit in the 160-row tile).  The reads are unconditional
      // (subtiles past the tile end hold copies of its last row); only the
      // MFMAs of such subtiles are skipped.  For per-token E4M3 this order
      // was 2-4 % slower than the compiler's own while the row-per-register
      // epilogue's scales took 20 registers; with transposed accumulators
      // (5 scales) it is faster on both GEMMs (same box, DeepSeek-V4-Pro
      // GEMM1 3.38 -> 3.29 ms; GEMM2 2.198 -> 2.113 ms against an order that
      // moved the barrier before the last subtile and read the next step's
      // weight fragments between its MFMAs, which is also 2-3 % slower on
      // the MXFP8 GEMM2 now and was removed).
      read_a(as, sa, 0, 0);
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const uint4 b = *reinterpret_cast<const uint4*>(bs + j * 1024);
        bop[j] = fp4_operand(b);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        if (i + 1 < WM) read_a(as, sa, i + 1, (i + 1) & 1);
        if (cols && i < nvalid) {
          const v8i aop = as_v8i(alo[i & 1], ahi[i & 1]);
#pragma unroll
          for (int j = 0; j < WN; ++j)
            acc[i][j] = mfma_wt<AF, S, MXA ? S : 0>(bop[j], aop, acc[i][j], (int)sx[j],
                                                   MXA ? axr[i & 1] : 127);
        }
        __builtin_amdgcn_sched_barrier(0);
        issue_part(i);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // E2M1 (W4A4) activations: the compiler's own order (all of the
      // step's fragments read before the first MFMA); the order above
      // measured 2-3 % slower here, and equal since the transposed
      // accumulators
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const uint4 b = *reinterpret_cast<const uint4*>(bs + j * 1024);
        bop[j] = fp4_operand(b);
      }
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        if (cols && i < nvalid) {
          const v8i aop = fp4_operand(*reinterpret_cast<const uint4*>(as + i * kSub));
          const int ax = *reinterpret_cast<const int*>(sa + i * kSaSub);
#pragma unroll
          for (int j = 0; j < WN; ++j)
            acc[i][j] = mfma_wt<AF, S, MXA ? S : 0>(bop[j], aop, acc[i][j], (int)sx[j], ax);
        }
        __builtin_amdgcn_sched_barrier(0);
        issue_part(i);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // subtiles fewer than the four load parts
#pragma unroll
    for (int part = WM; part < 4; ++part) issue_part(part);
    // the loads of step ks+1 (A issued above, weights one step earlier) have
    // landed once only the loads issued after this step's A loads remain
    wait_barrier<(S == 0 ? 2 * kBPW : kBPW)>();
  };

  // The last K step issues no loads and overlaps the epilogue with its
  // MFMAs: subtile i - 1's outputs are written while subtile i's MFMAs run.
  auto last_step = [&](auto s_c, int ks, int bstage) __attribute__((always_inline)) {
    constexpr int S = decltype(s_c)::value;
    // the only loads still in flight are copies of earlier steps' data
    // issued one step ago (their step index is clamped); drain them
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const uint8_t* bs = b_at(bstage);
    if constexpr (S == 0) {
      const uint8_t* ss = sx_at(ks);
#pragma unroll
      for (int j = 0; j < WN; ++j) sx[j] = *reinterpret_cast<const uint32_t*>(ss + j * 256);
    }
    const uint8_t* sa = sa_at(ks);
    const uint8_t* as = a_at(S & 1);
    v8i bop[WN];
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const uint4 b = *reinterpret_cast<const uint4*>(bs + j * 1024);
      bop[j] = fp4_operand(b);
    }
    if constexpr (!A4) read_a(as, sa, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      if constexpr (!A4) {
        if (i + 1 < WM) read_a(as, sa, i + 1, (i + 1) & 1);
        if (cols && i < nvalid) {
          const v8i aop = as_v8i(alo[i & 1], ahi[i & 1]);
#pragma unroll
          for (int j = 0; j < WN; ++j)
            acc[i][j] = mfma_wt<AF, S, MXA ? S : 0>(bop[j], aop, acc[i][j], (int)sx[j],
                                                   MXA ? axr[i & 1] : 127);
        }
      } else {
        if (cols && i < nvalid) {
          const v8i aop = fp4_operand(*reinterpret_cast<const uint4*>(as + i * kSub));
          const int ax = *reinterpret_cast<const int*>(sa + i * kSaSub);
#pragma unroll
          for (int j = 0; j < WN; ++j)
            acc[i][j] = mfma_wt<AF, S, MXA ? S : 0>(bop[j], aop, acc[i][j], (int)sx[j], ax);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (i > 0)
        finish_tile_t<V, FC1, WM, WN, RS>(p, acc, sc, row_base, row_end, nvalid, nb0, jvalid,
                                          lane, i - 1, i);
      __builtin_amdgcn_sched_barrier(0);
    }
    finish_tile_t<V, FC1, WM, WN, RS>(p, acc, sc, row_base, row_end, nvalid, nb0, jvalid, lane,
                                      WM - 1, WM);
  };

  // prologue: A and weights (and scales) of step 0, weights of step 1
  issue_as(0, 0);
  issue_a(0, 0);
  issue_b(0, 0);
  issue_sx(0, 0);
  issue_b(min(1, KS - 1), 1);
  wait_barrier<kBPW>();
  int ks = 0, bstage = 0;
  if constexpr (PEEL) {
    // K a multiple of 512 (whole 4-step groups): the last step, S = 3, is
    // peeled so its MFMAs overlap the epilogue (a kernel of its own: with the
    // remainder steps and a peeled step of every S in one body the compiler
    // spilled 200+ bytes per lane)
    for (; ks + 4 < KS; ks += 4) {
      step(std::integral_constant<int, 0>{}, ks, bstage);
      bstage = bstage == 2 ? 0 : bstage + 1;
      step(std::integral_constant<int, 1>{}, ks + 1, bstage);
      bstage = bstage == 2 ? 0 : bstage + 1;
      step(std::integral_constant<int, 2>{}, ks + 2, bstage);
      bstage = bstage == 2 ? 0 : bstage + 1;
      step(std::integral_constant<int, 3>{}, ks + 3, bstage);
      bstage = bstage == 2 ? 0 : bstage + 1;
    }
    step(std::integral_constant<int, 0>{}, ks, bstage);
    bstage = bstage == 2 ? 0 : bstage + 1;
    step(std::integral_constant<int, 1>{}, ks + 1, bstage);
    bstage = bstage == 2 ? 0 : bstage + 1;
    step(std::integral_constant<int, 2>{}, ks + 2, bstage);
    bstage = bstage == 2 ? 0 : bstage + 1;
    last_step(std::integral_constant<int, 3>{}, ks + 3, bstage);
  } else {
    for (; ks + 4 <= KS; ks += 4) {
      step(std::integral_constant<int, 0>{}, ks, bstage);
      bstage = bstage == 2 ? 0 : bstage + 1;
      step(std::integral_constant<int, 1>{}, ks + 1, bstage);
      bstage = bstage == 2 ? 0 : bstage + 1;
      step(std::integral_constant<int, 2>{}, ks + 2, bstage);
      bstage = bstage == 2 ? 0 : bstage + 1;
      step(std::integral_constant<int, 3>{}, ks + 3, bstage);
      bstage = bstage == 2 ? 0 : bstage + 1;
    }
    if (ks < KS) { step(std::integral_constant<int, 0>{}, ks, bstage); bstage = bstage == 2 ? 0 : bstage + 1; }
    if (ks + 1 < KS) { step(std::integral_constant<int, 1>{}, ks + 1, bstage); bstage = bstage == 2 ? 0 : bstage + 1; }
    if (ks + 2 < KS) step(std::integral_constant<int, 2>{}, ks + 2, bstage);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    finish_tile_t<V, FC1, WM, WN, RS>(p, acc, sc, row_base, row_end, nvalid, nb0, jvalid, lane);
  }
}

template <int V, bool FC1, int WM, bool PEEL>
__global__ __launch_bounds__(dma::kNW * kWave, 1) void k_gemm_dma(GemmParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[dma::Map<WM, a_blockscaled(V), a_fp4(V)>::kBytes];
  Tile tile;
  int nt;
  if (!work_item(p.tiles, p.num_tiles, p.n_tiles, p.pair_m, &tile, &nt)) return;
  gemm_dma_body<V, FC1, WM, PEEL>(p, lds, tile, nt);
}

template <int V, bool FC1>
static hipError_t launch_v(int cfg, const GemmParams& p, int64_t blocks, hipStream_t st) {
  if (cfg == 1) {
    // INT4: 8 waves side by side over 512 columns, so each staged A tile
    // serves twice the columns (GEMM1 10 % faster than 4 waves over 256)
    if constexpr (V == kInt4Fp8) k_gemm_lds<V, FC1, 8, 1, 4, 4, 1><<<(unsigned)blocks, 512, 0, st>>>(p);
    else k_gemm_lds<V, FC1, 4, 1, 4, 4><<<(unsigned)blocks, 256, 0, st>>>(p);
  }
  else if constexpr (scaled_fp4(V)) {  // 160 x 512
    if (p.K % (4 * kKStep) == 0)  // whole 4-step groups: peeled last step
      k_gemm_dma<V, FC1, 5, true><<<(unsigned)blocks, dma::kNW * kWave, 0, st>>>(p);
    else
      k_gemm_dma<V, FC1, 5, false><<<(unsigned)blocks, dma::kNW * kWave, 0, st>>>(p);
  }
  else k_gemm_ab<V, FC1, 8, 2, 4, 4><<<(unsigned)blocks, 512, 0, st>>>(p);
  return hipGetLastError();
}

hipError_t launch_gemm_lds(int variant, bool fc1, int cfg, const GemmParams& p,
                           int64_t max_tiles, hipStream_t st) {
  const int64_t blocks = gemm_blocks(max_tiles, p.n_tiles);
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  switch (variant) {
    case kMxfp4Fp8: return fc1 ? launch_v<kMxfp4Fp8, true>(cfg, p, blocks, st)
                               : launch_v<kMxfp4Fp8, false>(cfg, p, blocks, st);
    case kMxfp4Mxfp8: return fc1 ? launch_v<kMxfp4Mxfp8, true>(cfg, p, blocks, st)
                                 : launch_v<kMxfp4Mxfp8, false>(cfg, p, blocks, st);
    case kMxfp4Mxfp4: return fc1 ? launch_v<kMxfp4Mxfp4, true>(cfg, p, blocks, st)
                                 : launch_v<kMxfp4Mxfp4, false>(cfg, p, blocks, st);
    case kInt4Fp8: return fc1 ? launch_v<kInt4Fp8, true>(cfg, p, blocks, st)
                              : launch_v<kInt4Fp8, false>(cfg, p, blocks, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
