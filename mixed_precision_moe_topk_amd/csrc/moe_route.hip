// Top-k router, routing index (expert-grouped row permutation) and the
// grouped-GEMM work map.
//
// Router: the expert ids and their final weights are what flashinfer PR #4793
// ("Unify MoE CuTe DSL dispatch to be dtype agnostic") passes to its fused MoE
// (token_selected_experts / token_final_scales).  Here they are computed on
// the device: per token the k largest float32 logits, equal logits ordered by
// the smaller expert index, then a softmax over the k selected logits.
//
// Work map: flashinfer PR #3738 ("perf: optimize MXFP4xBF16 & INT4xFP8 and add
// MXFP4xFP8 CUTLASS MoE backend for SM90"), Implementation Notes, builds the
// grouped-GEMM schedule before the GEMM so that no tile lookup happens in the
// main loop; its review (scheduler thread) requires 64-bit linear work indices
// and that an empty routed batch is a no-op.  The map here is a list of
// (expert, first row, row count) tiles written by one small kernel; the GEMM
// grid indexes it with a 64-bit linear block index.
#include "moe_common.h"

namespace moe {

// One wave per token.  Lane j holds logits j, j+64, ... (E <= 1024).
__global__ __launch_bounds__(256) void k_router(RouteParams p) {
  const int lane = lane_id();
  const int64_t t = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= p.tokens) return;
  const int E = p.experts;
  const float* row = p.logits + t * E;
  constexpr int kPer = kMaxExperts / kWave;  // 16
  float v[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = lane + i * kWave;
    v[i] = (e < E) ? row[e] : 0.0f;
  }
  uint32_t taken = 0;  // bit i: value i of this lane already selected
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (lane + i * kWave >= E) taken |= 1u << i;

  float sel_v[kMaxTopK];
  int sel_e[kMaxTopK];
  const int K = p.top_k;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    sel_v[j] = 0.0f;
    sel_e[j] = 0;
    if (j >= K) continue;
    // lane-local best: larger value, then smaller expert index
    float bv = 0.0f;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (taken & (1u << i)) continue;
      const int e = lane + i * kWave;
      if (be == 0x7FFFFFFF || v[i] > bv) {  // indices grow with i: ties keep the first
        bv = v[i];
        be = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o);
      const int oe = __shfl_xor(be, o);
      const bool better = (oe != 0x7FFFFFFF) &&
                          (be == 0x7FFFFFFF || ov > bv || (ov == bv && oe < be));
      if (better) {
        bv = ov;
        be = oe;
      }
    }
    sel_v[j] = bv;
    sel_e[j] = be;
    if ((be & (kWave - 1)) == lane) taken |= 1u << (be / kWave);
  }
  // softmax over the selected logits (sel_v[0] is the largest)
  float sum = 0.0f;
  float pr[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    pr[j] = (j < K) ? expf(sel_v[j] - sel_v[0]) : 0.0f;
    sum += pr[j];
  }
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j < K && lane == j) {
      p.ids[t * K + j] = sel_e[j];
      p.weights[t * K + j] = __fdiv_rn(pr[j], sum);
    }
  }
}

// Per chunk of kRouteChunk (token, slot) pairs: expert histogram.
__global__ __launch_bounds__(256) void k_route_count(RouteParams p) {
  __shared__ int32_t cnt[kMaxExperts];
  const int64_t total = p.tokens * p.top_k;
  const int64_t base = (int64_t)blockIdx.x * kRouteChunk;
  for (int e = threadIdx.x; e < p.experts; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < kRouteChunk; i += blockDim.x) {
    const int64_t f = base + i;
    if (f < total) atomicAdd(&cnt[p.ids[f]], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < p.experts; e += blockDim.x)
    p.chunk_counts[(int64_t)blockIdx.x * p.experts + e] = cnt[e];
}

// Single block: per-expert totals, chunk bases, expert offsets, tile list.
__global__ __launch_bounds__(1024) void k_route_scan(RouteParams p) {
  __shared__ int32_t tot[kMaxExperts];
  __shared__ int32_t ntl[kMaxExperts];
  const int E = p.experts;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int32_t run = 0;
    for (int c = 0; c < p.nchunks; ++c) {
      const int64_t idx = (int64_t)c * E + e;
      const int32_t v = p.chunk_counts[idx];
      p.chunk_counts[idx] = run;  // rows of this expert in earlier chunks
      run += v;
    }
    tot[e] = run;
    ntl[e] = (run + p.tile_m - 1) / p.tile_m;
  }
  __syncthreads();
  // exclusive scans over experts (E <= 1024: one thread does the short serial
  // scan; it is a few hundred adds)
  if (threadIdx.x == 0) {
    int32_t r = 0, tl = 0;
    for (int e = 0; e < E; ++e) {
      const int32_t c = tot[e], n = ntl[e];
      p.offsets[e] = r;
      tot[e] = r;
      ntl[e] = tl;
      r += c;
      tl += n;
    }
    p.offsets[E] = r;
    *p.num_tiles = tl;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int32_t start = tot[e];
    const int32_t cnt = p.offsets[e + 1] - start;
    int32_t ti = ntl[e];
    for (int32_t r = 0; r < cnt; r += p.tile_m, ++ti) {
      Tile tl;
      tl.expert = e;
      tl.row0 = start + r;
      tl.nrows = min(p.tile_m, cnt - r);
      tl.pad = 0;
      p.tiles[ti] = tl;
    }
  }
}

// One wave per chunk: stable placement of each (token, slot) pair into its
// expert's rows in ascending (token, slot) order.
__global__ __launch_bounds__(64) void k_route_scatter(RouteParams p) {
  __shared__ int32_t cursor[kMaxExperts];
  const int lane = lane_id();
  const int64_t total = p.tokens * p.top_k;
  const int64_t base = (int64_t)blockIdx.x * kRouteChunk;
  for (int e = lane; e < p.experts; e += kWave)
    cursor[e] = p.offsets[e] + p.chunk_counts[(int64_t)blockIdx.x * p.experts + e];
  __syncthreads();
  for (int it = 0; it < kRouteChunk; it += kWave) {
    const int64_t f = base + it + lane;
    const bool valid = f < total;
    const int e = valid ? p.ids[f] : -1;
    uint64_t rem = __ballot(valid);
    int pos = 0;
    while (rem) {
      const int leader = __ffsll((unsigned long long)rem) - 1;
      const int el = __shfl(e, leader);
      const bool mine = valid && e == el;
      const uint64_t m = __ballot(mine) & rem;
      if (mine) pos = cursor[el] + __popcll(m & ((1ull << lane) - 1ull));
      __builtin_amdgcn_wave_barrier();
      if (lane == leader) cursor[el] += __popcll(m);
      __builtin_amdgcn_wave_barrier();
      rem &= ~m;
    }
    if (valid) {
      p.row_token[pos] = (int32_t)(f / p.top_k);
      p.slot_row[f] = pos;
    }
  }
}

hipError_t launch_route(const RouteParams& p, hipStream_t st) {
  if (p.tokens == 0) return hipSuccess;
  const int wpb = 4;
  k_router<<<(unsigned)((p.tokens + wpb - 1) / wpb), wpb * kWave, 0, st>>>(p);
  k_route_count<<<p.nchunks, 256, 0, st>>>(p);
  k_route_scan<<<1, 1024, 0, st>>>(p);
  k_route_scatter<<<p.nchunks, 64, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace moe
