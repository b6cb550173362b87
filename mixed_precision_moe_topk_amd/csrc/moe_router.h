// Top-k router of one token per wave (device code shared by the routing
// kernels and the launch that runs the router next to the token quantiser).
//
// The expert ids and their final weights are what flashinfer PR #4793 ("Unify
// MoE CuTe DSL dispatch to be dtype agnostic") passes to its fused MoE
// (token_selected_experts / token_final_scales): per token the k largest
// float32 logits, equal logits ordered by the smaller expert index, then a
// softmax over the k selected logits.
#pragma once
#include "moe_common.h"

// Wave-wide reduction of the ROCm device library (result in every lane).
extern "C" __device__ __attribute__((const)) uint32_t __ockl_wfred_max_u32(uint32_t);

namespace moe {

// Waves (tokens) per router block, and logits per lane: the fewest of 1, 2,
// 3, 4, 6, 8, 12, 16 that hold all experts (E <= 1024).
constexpr int kRouterWaves = 4;
inline int router_per(int experts) {
  return experts <= 64 ? 1 : experts <= 128 ? 2 : experts <= 192 ? 3 : experts <= 256 ? 4
       : experts <= 384 ? 6 : experts <= 512 ? 8 : experts <= 768 ? 12 : 16;
}

// Order-preserving code of a logit: the larger code is the larger logit.
// NaN codes as -inf and -0.0 as +0.0, so equal logits (either zero) tie and
// the expert index decides.  Every logit codes to at least 0x007FFFFF (-inf),
// so code 0 marks an empty slot.
__device__ __forceinline__ uint32_t logit_code(float x) {
  const uint32_t u = __float_as_uint(x == x ? x + 0.0f : -INFINITY);
  return (u >> 31) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float code_logit(uint32_t c) {
  return __uint_as_float((c >> 31) ? (c & 0x7FFFFFFFu) : ~c);
}

// Lanes set in m take b, the others a (two v_cndmask; written as asm so that
// a chain of them over an array stays a chain of selects instead of being
// rewritten into a data-dependent index with a select tree per element).
__device__ __forceinline__ uint64_t pick64(uint64_t a, uint64_t b, uint64_t m) {
  uint32_t lo, hi;
  asm("v_cndmask_b32_e64 %0, %1, %2, %3"
      : "=v"(lo) : "v"((uint32_t)a), "v"((uint32_t)b), "s"(m));
  asm("v_cndmask_b32_e64 %0, %1, %2, %3"
      : "=v"(hi) : "v"((uint32_t)(a >> 32)), "v"((uint32_t)(b >> 32)), "s"(m));
  return ((uint64_t)hi << 32) | lo;
}

// Batcher's merge-exchange sorting network for N keys (Knuth, TAOCP vol. 3,
// 5.2.2 Algorithm M), valid for any N: 12 comparators for 6 keys, 19 for 8.
template <int N>
struct MergeExchange {
  int a[N * N + 1], b[N * N + 1];
  int n;
  constexpr MergeExchange() : a(), b(), n(0) {
    int t = 0;
    while ((1 << t) < N) ++t;
    for (int p = t > 0 ? 1 << (t - 1) : 0; p > 0; p >>= 1) {
      int q = 1 << (t - 1), r = 0, d = p;
      for (;;) {
        for (int i = 0; i + d < N; ++i)
          if ((i & p) == r) {
            a[n] = i;
            b[n] = i + d;
            ++n;
          }
        if (q == p) break;
        d = q - p;
        q >>= 1;
        r = p;
      }
    }
  }
};

// Top-k and softmax of token t, by one wave.  Lane j holds logits j, j+64,
// ..., PER of them (E <= 64 PER), as 64-bit keys (code << 32 | ~expert: the
// larger key is the larger logit, then the smaller expert index), sorted in
// descending order once.  Each of the k rounds then takes the wave maximum
// of the lanes' first codes by one integer reduction; the lane that holds it
// (by a ballot; on an exact tie, the one with the smaller expert index, by a
// second reduction) gives up its first key.
template <int PER>
__device__ __forceinline__ void route_token(const RouteParams& p, const int64_t t) {
  const int lane = lane_id();
  const int E = p.experts;
  const float* row = p.logits + t * E;
  uint64_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + i * kWave;
    key[i] = e < E ? ((uint64_t)logit_code(row[e]) << 32) | (uint32_t)~e : 0;
  }
  constexpr MergeExchange<PER> net{};
#pragma unroll
  for (int c = 0; c < net.n; ++c) {
    const uint64_t x = key[net.a[c]], y = key[net.b[c]];
    const bool s = y > x;
    key[net.a[c]] = s ? y : x;
    key[net.b[c]] = s ? x : y;
  }

  float sel_v[kMaxTopK];
  int sel_e[kMaxTopK];
  const int K = p.top_k;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    sel_v[j] = 0.0f;
    sel_e[j] = 0;
    if (j >= K) continue;
    // at least E - j >= 1 logits remain, so cmax is a logit's code (> 0)
    const uint32_t hc = (uint32_t)(key[0] >> 32);
    const uint32_t cmax = __ockl_wfred_max_u32(hc);
    const bool hold = hc == cmax;
    const uint64_t holders = __ballot(hold);
    int wl;
    if (__popcll(holders) == 1) {
      wl = __ffsll((unsigned long long)holders) - 1;
    } else {  // equal logits: the largest ~expert, i.e. the smallest expert
      const uint32_t lo = __ockl_wfred_max_u32(hold ? (uint32_t)key[0] : 0u);
      wl = __ffsll((unsigned long long)__ballot(hold && (uint32_t)key[0] == lo)) - 1;
    }
    sel_v[j] = code_logit(cmax);
    sel_e[j] = (int)~(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)key[0], wl);
    const uint64_t w = 1ull << wl;  // the winning lane shifts its keys up by one
#pragma unroll
    for (int i = 0; i + 1 < PER; ++i) key[i] = pick64(key[i], key[i + 1], w);
    key[PER - 1] = pick64(key[PER - 1], 0, w);
  }
  // softmax over the selected logits (sel_v[0] is the largest): lane j < k
  // takes slot j's exponential; the sum runs over the slots in order
  float lv = 0.0f;
  int le = 0;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j)
    if (lane == j) {
      lv = sel_v[j];
      le = sel_e[j];
    }
  const float pj = lane < K ? expf(lv - sel_v[0]) : 0.0f;
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j)
    sum += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pj), j));
  if (lane < K) {
    p.ids[t * K + lane] = le;
    p.weights[t * K + lane] = __fdiv_rn(pj, sum);
  }
}

}  // namespace moe
