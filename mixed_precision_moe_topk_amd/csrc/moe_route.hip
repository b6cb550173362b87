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

// Wave-wide reductions of the ROCm device library (results in every lane).
extern "C" __device__ __attribute__((const)) float __ockl_wfred_max_f32(float);
extern "C" __device__ __attribute__((const)) int __ockl_wfred_min_i32(int);

namespace moe {

// Top-k and softmax of token t, by one wave.  Lane j holds logits j, j+64,
// ..., PER of them (E <= 64 PER).  Each of the k rounds takes every lane's
// best remaining logit (larger value, then smaller expert index), the wave
// maximum of those by a reduction, and the lanes that hold the maximum by a
// ballot; if more than one lane holds it (an exact tie, or -0.0 against
// +0.0), the smallest expert index among them wins, by a second reduction.
// A round is thus a chain of two or three wave reductions instead of a
// six-step shuffle of value and index.
template <int PER>
__device__ __forceinline__ void route_token(const RouteParams& p, const int64_t t) {
  const int lane = lane_id();
  const int E = p.experts;
  const float* row = p.logits + t * E;
  float v[PER];
  uint32_t taken = 0;  // bit i: value i of this lane already selected (or absent)
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + i * kWave;
    const float x = (e < E) ? row[e] : 0.0f;
    // a NaN logit ranks as -inf: every round then has a holder of the
    // maximum (-inf at worst), so every id is a valid expert index
    v[i] = x == x ? x : -INFINITY;
    if (e >= E) taken |= 1u << i;
  }

  float sel_v[kMaxTopK];
  int sel_e[kMaxTopK];
  const int K = p.top_k;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    sel_v[j] = 0.0f;
    sel_e[j] = 0;
    if (j >= K) continue;
    // lane-local best: larger value, then smaller expert index
    float bv = -INFINITY;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (taken & (1u << i)) continue;
      if (be == 0x7FFFFFFF || v[i] > bv) {  // indices grow with i: ties keep the first
        bv = v[i];
        be = lane + i * kWave;
      }
    }
    const float vmax = __ockl_wfred_max_f32(bv);
    const bool hold = be != 0x7FFFFFFF && bv == vmax;
    const uint64_t holders = __ballot(hold);
    int win;
    if (__popcll(holders) == 1)
      win = __builtin_amdgcn_readlane(be, __ffsll((unsigned long long)holders) - 1);
    else
      win = __ockl_wfred_min_i32(hold ? be : 0x7FFFFFFF);
    sel_v[j] = vmax;
    sel_e[j] = win;
    if ((win & (kWave - 1)) == lane) taken |= 1u << (win / kWave);
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

// One wave per token.
template <int PER>
__global__ __launch_bounds__(256) void k_router(RouteParams p) {
  const int64_t t = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t < p.tokens) route_token<PER>(p, t);
}

// Routing index over chunks of kChunkTokens tokens (one wave per chunk).  For
// every expert a 64-bit mask of the chunk's tokens that selected it is built
// with atomic ORs in LDS (order-independent, so deterministic); the rank of
// token t among the chunk's rows of expert e is popcount(mask[e] & lanes < t).
// Rows of one expert thus come in ascending (token, slot) order.
constexpr int kChunkTokens = kRouteChunkTokens;

__device__ __forceinline__ void build_masks(const RouteParams& p, uint64_t* mask, int64_t t0) {
  const int lane = lane_id();
  for (int e = lane; e < p.experts; e += kWave) mask[e] = 0;
  __syncthreads();
  const int64_t t = t0 + lane;
  if (t < p.tokens) {
    for (int j = 0; j < p.top_k; ++j)
      atomicOr(reinterpret_cast<unsigned long long*>(&mask[p.ids[t * p.top_k + j]]),
               1ull << lane);
  }
  __syncthreads();
}

__global__ __launch_bounds__(64) void k_route_count(RouteParams p) {
  __shared__ uint64_t mask[kMaxExperts];
  build_masks(p, mask, (int64_t)blockIdx.x * kChunkTokens);
  for (int e = lane_id(); e < p.experts; e += kWave)
    p.chunk_counts[(int64_t)blockIdx.x * p.experts + e] = __popcll(mask[e]);
}

// Single block: per-expert totals, chunk bases, expert offsets, tile list.
// Thread e (blockDim.x == 1024 >= E) holds `run`, the rows of expert e.
// Block-wide exclusive scans of the rows and of the tiles per expert (wave
// scans + wave totals) give the expert offsets and the work map; returns the
// first row of expert e.
__device__ int32_t scan_experts(const RouteParams& p, const int32_t run, int32_t (*wsum)[16]) {
  const int E = p.experts;
  const int e = threadIdx.x;
  const int32_t nt = (run + p.tile_m - 1) / p.tile_m;
  const int lane = lane_id(), w = threadIdx.x / kWave;
  int32_t a = run, b = nt;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int32_t ya = __shfl_up(a, o), yb = __shfl_up(b, o);
    if (lane >= o) { a += ya; b += yb; }
  }
  if (lane == kWave - 1) { wsum[0][w] = a; wsum[1][w] = b; }
  __syncthreads();
  int32_t pa = 0, pb = 0;
  for (int i = 0; i < w; ++i) { pa += wsum[0][i]; pb += wsum[1][i]; }
  const int32_t ex_a = pa + a - run, ex_b = pb + b - nt;
  if (e == E - 1) {
    p.offsets[E] = ex_a + run;
    *p.num_tiles = ex_b + nt;
  }
  if (e < E) {
    p.offsets[e] = ex_a;
    int32_t ti = ex_b;
    for (int32_t r = 0; r < run; r += p.tile_m, ++ti) {
      Tile tl;
      tl.expert = e;
      tl.row0 = ex_a + r;
      tl.nrows = min(p.tile_m, run - r);
      tl.pad = 0;
      p.tiles[ti] = tl;
    }
  }
  return ex_a;
}

__global__ __launch_bounds__(1024) void k_route_scan(RouteParams p) {
  __shared__ int32_t wsum[2][16];
  const int E = p.experts;
  const int e = threadIdx.x;  // blockDim.x == 1024 >= E
  int32_t run = 0;
  if (e < E) {
    // exclusive prefix over chunks, 16 independent loads at a time (a chain
    // of dependent loads would cost one memory latency per chunk)
    constexpr int kB = 16;
    for (int c0 = 0; c0 < p.nchunks; c0 += kB) {
      int32_t v[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u)
        v[u] = c0 + u < p.nchunks ? p.chunk_counts[(int64_t)(c0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        if (c0 + u < p.nchunks) p.chunk_counts[(int64_t)(c0 + u) * E + e] = run;  // rows in earlier chunks
        run += v[u];
      }
    }
  }
  scan_experts(p, run, wsum);
}

__global__ __launch_bounds__(64) void k_route_scatter(RouteParams p) {
  __shared__ uint64_t mask[kMaxExperts];
  const int64_t t0 = (int64_t)blockIdx.x * kChunkTokens;
  build_masks(p, mask, t0);
  const int lane = lane_id();
  const int64_t t = t0 + lane;
  if (t >= p.tokens) return;
  const uint64_t below = (1ull << lane) - 1ull;
  for (int j = 0; j < p.top_k; ++j) {
    const int64_t f = t * p.top_k + j;
    const int e = p.ids[f];
    const int pos = p.offsets[e] + p.chunk_counts[(int64_t)blockIdx.x * p.experts + e] +
                    __popcll(mask[e] & below);
    p.row_token[pos] = (int32_t)t;
    p.slot_row[f] = pos;
  }
}

// Routing index of a batch of at most one chunk (64 tokens) in one block of
// 1024 threads: the same masks, scan and ranks as the chunked kernels (so the
// same results) in one launch instead of three.
__global__ __launch_bounds__(1024) void k_route_small(RouteParams p) {
  __shared__ uint64_t mask[kMaxExperts];
  __shared__ int32_t offs[kMaxExperts];
  __shared__ int32_t wsum[2][16];
  const int E = p.experts, K = p.top_k;
  const int tid = threadIdx.x;
  if (tid < E) mask[tid] = 0;
  __syncthreads();
  if (tid < p.tokens) {
    for (int j = 0; j < K; ++j)
      atomicOr(reinterpret_cast<unsigned long long*>(&mask[p.ids[tid * K + j]]), 1ull << tid);
  }
  __syncthreads();
  const int32_t run = tid < E ? __popcll(mask[tid]) : 0;
  const int32_t first = scan_experts(p, run, wsum);
  if (tid < E) offs[tid] = first;
  __syncthreads();
  if (tid < p.tokens) {
    const uint64_t below = (1ull << tid) - 1ull;
    for (int j = 0; j < K; ++j) {
      const int64_t f = (int64_t)tid * K + j;
      const int e = p.ids[f];
      const int pos = offs[e] + __popcll(mask[e] & below);
      p.row_token[pos] = tid;
      p.slot_row[f] = pos;
    }
  }
}

hipError_t launch_route(const RouteParams& p, hipStream_t st) {
  if (p.tokens == 0) return hipSuccess;
  const int wpb = 4;
  const dim3 grid((unsigned)((p.tokens + wpb - 1) / wpb)), block(wpb * kWave);
  // logits per lane: the fewest that hold all experts
  if (p.experts <= 64) k_router<1><<<grid, block, 0, st>>>(p);
  else if (p.experts <= 128) k_router<2><<<grid, block, 0, st>>>(p);
  else if (p.experts <= 256) k_router<4><<<grid, block, 0, st>>>(p);
  else if (p.experts <= 512) k_router<8><<<grid, block, 0, st>>>(p);
  else k_router<16><<<grid, block, 0, st>>>(p);
  if (p.tokens <= kChunkTokens) {
    k_route_small<<<1, 1024, 0, st>>>(p);
    return hipGetLastError();
  }
  k_route_count<<<p.nchunks, 64, 0, st>>>(p);
  k_route_scan<<<1, 1024, 0, st>>>(p);
  k_route_scatter<<<p.nchunks, 64, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace moe
