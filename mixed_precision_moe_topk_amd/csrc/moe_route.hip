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
#include "moe_router.h"

namespace moe {

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

// The count kernel takes kGroupChunks chunks per block (one wave each), so
// the single-block scan runs over groups of chunks (16 groups for 16384
// tokens instead of 256 chunks: the scan's chain of dependent loads shrinks
// accordingly).  Per expert it writes, for each chunk, the rows in earlier
// chunks of its group (chunk_counts) and the group's total (group counts,
// stored after the chunk counts).
constexpr int kGroupChunks = kRouteGroupChunks;
static_assert(kGroupChunks * kWave == 1024 && kMaxExperts <= 1024,
              "one count-kernel thread per expert (its scan for a single group)");

// One block of 1024 threads: expert offsets and the tile list.  Thread e
// (blockDim.x == 1024 >= E) holds `run`, the rows of expert e.
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

// A batch of one group (at most 1024 tokens) also runs the scan here, so its
// routing index takes two launches instead of three.
__global__ __launch_bounds__(kGroupChunks * kWave) void k_route_count(RouteParams p) {
  __shared__ uint64_t gmask[kGroupChunks][kMaxExperts];
  __shared__ int32_t wsum[2][16];
  const int w = threadIdx.x / kWave;
  const int64_t c0 = (int64_t)blockIdx.x * kGroupChunks;
  build_masks(p, gmask[w], (c0 + w) * kChunkTokens);
  const int E = p.experts;
  const int e = threadIdx.x;  // blockDim.x == 1024 >= E
  const bool single = gridDim.x == 1;
  int32_t* group_counts = p.chunk_counts + (int64_t)p.nchunks * E;
  int32_t run = 0;
  if (e < E) {
#pragma unroll
    for (int u = 0; u < kGroupChunks; ++u) {
      if (c0 + u < p.nchunks) p.chunk_counts[(c0 + u) * E + e] = run;
      run += __popcll(gmask[u][e]);
    }
    // one group: its prefix (rows in earlier groups) is 0
    group_counts[(int64_t)blockIdx.x * E + e] = single ? 0 : run;
  }
  if (single) scan_experts(p, run, wsum);
}

__global__ __launch_bounds__(1024) void k_route_scan(RouteParams p) {
  __shared__ int32_t wsum[2][16];
  const int E = p.experts;
  const int e = threadIdx.x;  // blockDim.x == 1024 >= E
  const int64_t ng = (p.nchunks + kGroupChunks - 1) / kGroupChunks;
  int32_t* group_counts = p.chunk_counts + (int64_t)p.nchunks * E;
  int32_t run = 0;
  if (e < E) {
    // exclusive prefix over groups, 16 independent loads at a time (a chain
    // of dependent loads would cost one memory latency per group)
    constexpr int kB = 16;
    for (int64_t g0 = 0; g0 < ng; g0 += kB) {
      int32_t v[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) v[u] = g0 + u < ng ? group_counts[(g0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        if (g0 + u < ng) group_counts[(g0 + u) * E + e] = run;  // rows in earlier groups
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
    const int pos = p.offsets[e] +
                    p.chunk_counts[((int64_t)p.nchunks + blockIdx.x / kGroupChunks) * p.experts + e] +
                    p.chunk_counts[(int64_t)blockIdx.x * p.experts + e] + __popcll(mask[e] & below);
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

hipError_t launch_route_index(const RouteParams& p, hipStream_t st) {
  if (p.tokens == 0) return hipSuccess;
  if (p.tokens <= kChunkTokens) {
    k_route_small<<<1, 1024, 0, st>>>(p);
    return hipGetLastError();
  }
  const int ngroups = (p.nchunks + kGroupChunks - 1) / kGroupChunks;
  k_route_count<<<ngroups, kGroupChunks * kWave, 0, st>>>(p);
  if (ngroups > 1) k_route_scan<<<1, 1024, 0, st>>>(p);
  k_route_scatter<<<p.nchunks, 64, 0, st>>>(p);
  return hipGetLastError();
}

hipError_t launch_route(const RouteParams& p, hipStream_t st) {
  if (p.tokens == 0) return hipSuccess;
  const int wpb = kRouterWaves;
  const dim3 grid((unsigned)((p.tokens + wpb - 1) / wpb)), block(wpb * kWave);
  switch (router_per(p.experts)) {
    case 1: k_router<1><<<grid, block, 0, st>>>(p); break;
    case 2: k_router<2><<<grid, block, 0, st>>>(p); break;
    case 3: k_router<3><<<grid, block, 0, st>>>(p); break;
    case 4: k_router<4><<<grid, block, 0, st>>>(p); break;
    case 6: k_router<6><<<grid, block, 0, st>>>(p); break;
    case 8: k_router<8><<<grid, block, 0, st>>>(p); break;
    case 12: k_router<12><<<grid, block, 0, st>>>(p); break;
    default: k_router<16><<<grid, block, 0, st>>>(p); break;
  }
  const hipError_t e = hipGetLastError();
  return e != hipSuccess ? e : launch_route_index(p, st);
}

}  // namespace moe
