// Memory-bound steps of the fused MoE: per-token FP8 activation quantisation,
// FC2-input requantisation and the router-weighted finalize.
//
// flashinfer PR #3738 ("perf: optimize MXFP4xBF16 & INT4xFP8 and add MXFP4xFP8
// CUTLASS MoE backend for SM90"), Implementation Notes: FP8 activations are
// quantised at run time with one scale per token (here s = amax/448, E4M3
// codes of x/s with IEEE division, round to nearest even, saturating at 448);
// its runner threads per-token FP8 scales through expansion, activation and
// both GEMMs (Walkthrough, "Runner and per-token FP8 execution"), so the
// SwiGLU output is requantised the same way per expanded row before FC2.
// PR #4793 ("Unify MoE CuTe DSL dispatch to be dtype agnostic") fuses the
// router-weighted sum of the k expert outputs into a finalize step.
#include "moe_router.h"

namespace moe {

// Block-wide max of non-negative floats (256 threads).
__device__ __forceinline__ float block_max256(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x / kWave;
  if (lane_id() == 0) red[w] = v;
  __syncthreads();
  v = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return v;
}

__device__ __forceinline__ float bf16x8_amax(const uint4& u, float amax) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    amax = fmaxf(amax, fabsf(__uint_as_float(w[j] << 16)));
    amax = fmaxf(amax, fabsf(__uint_as_float(w[j] & 0xFFFF0000u)));
  }
  return amax;
}

// E4M3 codes of fl32(x / s) for eight bf16 values (|x| <= amax, so the
// quotients stay within 448 * (1 + 2^-23)); inv = fl32(1 / s).
__device__ __forceinline__ uint2 bf16x8_to_e4m3(const uint4& u, float s, float inv) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  uint32_t c[2] = {0, 0};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float lo = div_for_e4m3(__uint_as_float(w[j] << 16), s, inv);
    const float hi = div_for_e4m3(__uint_as_float(w[j] & 0xFFFF0000u), s, inv);
    c[j / 2] |= e4m3_pk(lo, hi) << (16 * (j & 1));
  }
  return make_uint2(c[0], c[1]);
}

// One block per token row: x bf16 [T, H] -> codes E4M3 [T, H], scales [T].
// H % 8 == 0.  Rows of up to 8192 elements are read once and kept in
// registers between the amax and the quantisation; longer rows are read twice.
__device__ __forceinline__ void quant_token_row(const uint16_t* __restrict__ x, int32_t H,
                                                uint8_t* __restrict__ codes,
                                                float* __restrict__ scales, const int64_t t,
                                                float* red) {
  constexpr int kR = 4;  // uint4 (8 bf16) per thread kept in registers
  const uint4* row = reinterpret_cast<const uint4*>(x + t * H);
  uint2* out = reinterpret_cast<uint2*>(codes + t * H);
  const int nv = H / 8;
  float amax = 0.0f;
  if (nv <= kR * 256) {
    uint4 u[kR];
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      const int i = threadIdx.x + 256 * r;
      u[r] = i < nv ? row[i] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < kR; ++r) amax = bf16x8_amax(u[r], amax);
    amax = block_max256(amax, red);
    const float s = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
    const float inv = __fdiv_rn(1.0f, s);
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      const int i = threadIdx.x + 256 * r;
      if (i < nv) out[i] = bf16x8_to_e4m3(u[r], s, inv);
    }
    if (threadIdx.x == 0) scales[t] = s;
    return;
  }
  for (int i = threadIdx.x; i < nv; i += blockDim.x) amax = bf16x8_amax(row[i], amax);
  amax = block_max256(amax, red);
  const float s = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
  const float inv = __fdiv_rn(1.0f, s);
  for (int i = threadIdx.x; i < nv; i += blockDim.x) out[i] = bf16x8_to_e4m3(row[i], s, inv);
  if (threadIdx.x == 0) scales[t] = s;
}

__global__ __launch_bounds__(256) void k_quant_tokens(const uint16_t* __restrict__ x, int32_t H,
                                                      uint8_t* __restrict__ codes,
                                                      float* __restrict__ scales) {
  __shared__ float red[4];
  quant_token_row(x, H, codes, scales, blockIdx.x, red);
}

// One block per expanded row: h f32 [rows, I] -> FC2 input.
//   FP8:  per-row E4M3 codes [rows, I] + scales [rows]
//   BF16: bf16 bits [rows, I] (scale 1, written as 1.0f)
// I % 4 == 0.
__global__ __launch_bounds__(256) void k_requant(const float* __restrict__ h, int32_t I,
                                                 int bf16_out, uint8_t* __restrict__ codes,
                                                 float* __restrict__ scales) {
  __shared__ float red[4];
  const int64_t r = blockIdx.x;
  const float4* row = reinterpret_cast<const float4*>(h + r * I);
  const int nv = I / 4;
  if (bf16_out) {
    uint2* out = reinterpret_cast<uint2*>(codes + r * I * 2);
    for (int i = threadIdx.x; i < nv; i += blockDim.x) {
      const float4 v = load_stream(row + i);
      out[i] = make_uint2(bf16_bits(v.x) | (bf16_bits(v.y) << 16),
                          bf16_bits(v.z) | (bf16_bits(v.w) << 16));
    }
    if (threadIdx.x == 0) scales[r] = 1.0f;
    return;
  }
  auto f4_amax = [](const float4& v, float a) {
    return fmaxf(fmaxf(a, fabsf(v.x)), fmaxf(fabsf(v.y), fmaxf(fabsf(v.z), fabsf(v.w))));
  };
  auto f4_e4m3 = [](const float4& v, float s, float inv) {
    return e4m3_pk(div_for_e4m3(v.x, s, inv), div_for_e4m3(v.y, s, inv)) |
           (e4m3_pk(div_for_e4m3(v.z, s, inv), div_for_e4m3(v.w, s, inv)) << 16);
  };
  uint32_t* out = reinterpret_cast<uint32_t*>(codes + r * I);
  float amax = 0.0f;
  constexpr int kR = 4;  // float4 per thread kept in registers (rows up to 4096)
  if (nv <= kR * 256) {
    float4 v[kR];
#pragma unroll
    for (int q = 0; q < kR; ++q) {
      const int i = threadIdx.x + 256 * q;
      v[q] = i < nv ? load_stream(row + i) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int q = 0; q < kR; ++q) amax = f4_amax(v[q], amax);
    amax = block_max256(amax, red);
    const float s = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
    const float inv = __fdiv_rn(1.0f, s);
#pragma unroll
    for (int q = 0; q < kR; ++q) {
      const int i = threadIdx.x + 256 * q;
      if (i < nv) out[i] = f4_e4m3(v[q], s, inv);
    }
    if (threadIdx.x == 0) scales[r] = s;
    return;
  }
  for (int i = threadIdx.x; i < nv; i += blockDim.x) amax = f4_amax(row[i], amax);
  amax = block_max256(amax, red);
  const float s = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
  const float inv = __fdiv_rn(1.0f, s);
  for (int i = threadIdx.x; i < nv; i += blockDim.x) out[i] = f4_e4m3(row[i], s, inv);
  if (threadIdx.x == 0) scales[r] = s;
}

// ---------------------------------------------------------------- MXFP8 / MXFP4
// OCP MX conversion: per 32 consecutive elements X = floor(log2 amax) - emax
// (emax 8 for E4M3 elements, 2 for E2M1; clamped to [-127, 127]; amax = 0 ->
// X = 0, code 127), elements E4M3 / E2M1 of v * 2^-X rounded to nearest even
// and saturated (448 / 6).  v * 2^-X is exact in float32 unless the product
// is below 2^-126, where the code is +-0 either way.  (MXFP8 inputs of
// flashinfer PR #4793, "Unify MoE CuTe DSL dispatch to be dtype agnostic",
// and PR #3614's MXFP8xMXFP8; the MXFP4 activation pack of PR #4793's w4a4
// mode, quantised like the weights.)

// Eight consecutive elements per thread, four threads (consecutive lanes) per
// 32-element block.  `valid`: the group's block lies inside the row (rows are
// a multiple of 32 long, so a group is wholly inside or outside).  Returns
// the eight codes (E4M3: 8 bytes; E2M1: one dword, element i in bits 4i..4i+3,
// i.e. element 2j in the low nibble of byte j); *code = the block's E8M0 code.
template <bool E2M1>
__device__ __forceinline__ uint2 mx_quant8(const float (&v)[8], bool valid, uint32_t* code) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  if (!valid) amax = 0.0f;
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  const int x = mx_exponent<E2M1 ? 2 : 8>(amax);
  *code = (uint32_t)(x + 127);
  const float inv = __uint_as_float((uint32_t)(127 - x) << 23);  // 2^-X, a normal float
  uint32_t c[2] = {0, 0};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (E2M1)
      c[0] |= (e2m1_magnitude_code(fabsf(v[i]) * inv) | ((__float_as_uint(v[i]) >> 31) << 3))
              << (4 * i);
  }
  if (!E2M1) {  // v * 2^-X is below 512 in magnitude; saturate at 448 as the encoder does
#pragma unroll
    for (int i = 0; i < 8; i += 2)
      c[i / 4] |= e4m3_pk(fminf(fmaxf(v[i] * inv, -448.0f), 448.0f),
                          fminf(fmaxf(v[i + 1] * inv, -448.0f), 448.0f)) << (8 * (i & 3));
  }
  return make_uint2(c[0], c[1]);
}

// One block (256 threads) per row of C elements (C % 32 == 0), 2048 elements
// per pass: bf16 (SRC_BF16) or float32 input -> E4M3 codes [C] (E2M1: packed
// codes [C/2]) + E8M0 codes in the block-scaled MFMA's scale order
// (mx_scale_offset); the row's float scale is written as 1.0.
template <bool SRC_BF16, bool E2M1>
__device__ __forceinline__ void quant_mx_row(const void* __restrict__ src, int32_t C,
                                             uint8_t* __restrict__ codes,
                                             uint8_t* __restrict__ bscales,
                                             float* __restrict__ scales, const int64_t r) {
  for (int i = threadIdx.x; 8 * (i - (int)(threadIdx.x & 3)) < C; i += 256) {
    const bool valid = 8 * i < C;
    float v[8];
    if (SRC_BF16) {
      const uint4 u = valid ? reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + r * C)[i]
                            : make_uint4(0, 0, 0, 0);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = __uint_as_float(w[j] << 16);
        v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      }
    } else {
      const float4* row = reinterpret_cast<const float4*>(static_cast<const float*>(src) + r * C);
      const float4 a = valid ? row[2 * i] : make_float4(0.f, 0.f, 0.f, 0.f);
      const float4 b = valid ? row[2 * i + 1] : make_float4(0.f, 0.f, 0.f, 0.f);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    uint32_t code;
    const uint2 q = mx_quant8<E2M1>(v, valid, &code);
    if (valid) {
      if (E2M1) reinterpret_cast<uint32_t*>(codes + r * (C / 2))[i] = q.x;
      else reinterpret_cast<uint2*>(codes + r * C)[i] = q;
      if ((i & 3) == 0) bscales[r * mx_scale_row_bytes(C) + mx_scale_offset(i / 4)] = (uint8_t)code;
    }
  }
  if (threadIdx.x == 0) scales[r] = 1.0f;
}

template <bool SRC_BF16, bool E2M1>
__global__ __launch_bounds__(256) void k_quant_mx(const void* __restrict__ src, int32_t C,
                                                  uint8_t* __restrict__ codes,
                                                  uint8_t* __restrict__ bscales,
                                                  float* __restrict__ scales) {
  quant_mx_row<SRC_BF16, E2M1>(src, C, codes, bscales, scales, blockIdx.x);
}

// The router and the token quantiser in one launch: they read different
// inputs (logits, hidden states) and the routing index waits only for the
// router, so the first ceil(T / 4) blocks route four tokens each and the
// next T blocks quantise one token each (QM 0: per-token E4M3, 1: MXFP8, 2:
// MXFP4).  The two kernels back to back cost the router's time on top of the
// quantiser's.
template <int PER, int QM>
__global__ __launch_bounds__(256) void k_router_quant(RouteParams p, const uint16_t* __restrict__ x,
                                                      int32_t H, uint8_t* __restrict__ codes,
                                                      float* __restrict__ scales,
                                                      uint8_t* __restrict__ bscales,
                                                      int64_t router_blocks) {
  __shared__ float red[4];
  if ((int64_t)blockIdx.x < router_blocks) {
    const int64_t t = (int64_t)blockIdx.x * kRouterWaves + threadIdx.x / kWave;
    if (t < p.tokens) route_token<PER>(p, t);
    return;
  }
  const int64_t t = (int64_t)blockIdx.x - router_blocks;
  if constexpr (QM == 0) quant_token_row(x, H, codes, scales, t, red);
  else quant_mx_row<true, QM == 2>(x, H, codes, bscales, scales, t);
}

template <int QM>
static void launch_rq(const RouteParams& p, const uint16_t* x, int32_t H, uint8_t* codes,
                      float* scales, uint8_t* bscales, hipStream_t st) {
  const int64_t rb = (p.tokens + kRouterWaves - 1) / kRouterWaves;
  const unsigned grid = (unsigned)(rb + p.tokens);
  switch (router_per(p.experts)) {
    case 1: k_router_quant<1, QM><<<grid, 256, 0, st>>>(p, x, H, codes, scales, bscales, rb); break;
    case 2: k_router_quant<2, QM><<<grid, 256, 0, st>>>(p, x, H, codes, scales, bscales, rb); break;
    case 3: k_router_quant<3, QM><<<grid, 256, 0, st>>>(p, x, H, codes, scales, bscales, rb); break;
    case 4: k_router_quant<4, QM><<<grid, 256, 0, st>>>(p, x, H, codes, scales, bscales, rb); break;
    case 6: k_router_quant<6, QM><<<grid, 256, 0, st>>>(p, x, H, codes, scales, bscales, rb); break;
    case 8: k_router_quant<8, QM><<<grid, 256, 0, st>>>(p, x, H, codes, scales, bscales, rb); break;
    case 12: k_router_quant<12, QM><<<grid, 256, 0, st>>>(p, x, H, codes, scales, bscales, rb); break;
    default: k_router_quant<16, QM><<<grid, 256, 0, st>>>(p, x, H, codes, scales, bscales, rb); break;
  }
}

hipError_t launch_router_quant(const RouteParams& p, const uint16_t* x, int32_t H, int mode,
                               uint8_t* codes, float* scales, uint8_t* bscales, hipStream_t st) {
  if (p.tokens == 0) return hipSuccess;
  static_assert(kRouterWaves * kWave == 256, "router blocks are quantiser-sized");
  if (mode == kQuantMxfp8) launch_rq<1>(p, x, H, codes, scales, bscales, st);
  else if (mode == kQuantMxfp4) launch_rq<2>(p, x, H, codes, scales, bscales, st);
  else launch_rq<0>(p, x, H, codes, scales, bscales, st);
  const hipError_t e = hipGetLastError();
  return e != hipSuccess ? e : launch_route_index(p, st);
}

// Blocks (t, y): out[t] = bf16(sum_j fl32(w[t,j] * y2[row(t,j)])), the float32
// sum taken in slot order, over the float4 columns y, y + gridDim.y, ... (in
// units of the block size).  H % 4 == 0.  A block walks its k rows from start
// to end, so each row is read as one sequential stream.  KC > 0: top-k known
// at compile time, so the k row loads of a column group are issued together
// (one load in flight per thread would leave the kernel latency-bound).
template <int KC, int NTHR>
__global__ __launch_bounds__(NTHR) void k_finalize(const float* __restrict__ y2,
                                                  const float* __restrict__ weights,
                                                  const int32_t* __restrict__ slot_row,
                                                  int32_t k_rt, int32_t H,
                                                  uint16_t* __restrict__ out) {
  // each product is rounded to float32 before it is added: no fused
  // multiply-add (by default the compiler contracts w * y + acc into one)
#pragma clang fp contract(off)
  const int64_t t = blockIdx.x;
  const int k = KC > 0 ? KC : k_rt;
  const int nv = H / 4;
  // blockIdx.y splits the token's columns when there are few tokens
  for (int i = blockIdx.y * blockDim.x + threadIdx.x; i < nv; i += gridDim.y * blockDim.x) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (KC > 0) {
      float4 y[KC];
#pragma unroll
      for (int j = 0; j < KC; ++j)
        y[j] = load_stream(reinterpret_cast<const float4*>(y2 + (int64_t)slot_row[t * KC + j] * H) + i);
#pragma unroll
      for (int j = 0; j < KC; ++j) {
        const float w = weights[t * KC + j];
        acc.x = acc.x + w * y[j].x;
        acc.y = acc.y + w * y[j].y;
        acc.z = acc.z + w * y[j].z;
        acc.w = acc.w + w * y[j].w;
      }
    } else {
      for (int j = 0; j < k; ++j) {
        const float w = weights[t * k + j];
        const float4 y = load_stream(reinterpret_cast<const float4*>(y2 + (int64_t)slot_row[t * k + j] * H) + i);
        acc.x = acc.x + w * y.x;
        acc.y = acc.y + w * y.y;
        acc.z = acc.z + w * y.z;
        acc.w = acc.w + w * y.w;
      }
    }
    reinterpret_cast<uint2*>(out + t * H)[i] =
        make_uint2(bf16_bits(acc.x) | (bf16_bits(acc.y) << 16),
                   bf16_bits(acc.z) | (bf16_bits(acc.w) << 16));
  }
}

hipError_t launch_quant_tokens(const uint16_t* x, int64_t T, int32_t H, int mode,
                               uint8_t* codes, float* scales, uint8_t* bscales, hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (mode == kQuantMxfp8) k_quant_mx<true, false><<<(unsigned)T, 256, 0, st>>>(x, H, codes, bscales, scales);
  else if (mode == kQuantMxfp4) k_quant_mx<true, true><<<(unsigned)T, 256, 0, st>>>(x, H, codes, bscales, scales);
  else k_quant_tokens<<<(unsigned)T, 256, 0, st>>>(x, H, codes, scales);
  return hipGetLastError();
}

hipError_t launch_requant(const float* h, int64_t rows, int32_t I, int mode, uint8_t* codes,
                          float* scales, uint8_t* bscales, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  if (mode == kQuantMxfp8)
    k_quant_mx<false, false><<<(unsigned)rows, 256, 0, st>>>(h, I, codes, bscales, scales);
  else if (mode == kQuantMxfp4)
    k_quant_mx<false, true><<<(unsigned)rows, 256, 0, st>>>(h, I, codes, bscales, scales);
  else
    k_requant<<<(unsigned)rows, 256, 0, st>>>(h, I, mode == kQuantBf16 ? 1 : 0, codes, scales);
  return hipGetLastError();
}

hipError_t launch_finalize(const float* y2, const float* weights, const int32_t* slot_row,
                           int64_t T, int32_t k, int32_t H, uint16_t* out, hipStream_t st) {
  if (T == 0) return hipSuccess;
  // Many tokens: a block of 1024 threads per token (3 % faster than 256 on
  // 16384 tokens x 7168 columns; the output stores, not the y2 reads, set the
  // pace: without them the kernel reads at a plain read's 7.1 TB/s).  Few
  // tokens: 256 threads, with a token's columns split over up to 2048 / T
  // blocks so that a small batch still fills the GPU (64 tokens, H = 7168: 7
  // blocks each).
  if (T >= 2048) {
    const dim3 grid((unsigned)T, 1);
    switch (k) {
      case 2: k_finalize<2, 1024><<<grid, 1024, 0, st>>>(y2, weights, slot_row, k, H, out); break;
      case 4: k_finalize<4, 1024><<<grid, 1024, 0, st>>>(y2, weights, slot_row, k, H, out); break;
      case 6: k_finalize<6, 1024><<<grid, 1024, 0, st>>>(y2, weights, slot_row, k, H, out); break;
      case 8: k_finalize<8, 1024><<<grid, 1024, 0, st>>>(y2, weights, slot_row, k, H, out); break;
      default: k_finalize<0, 1024><<<grid, 1024, 0, st>>>(y2, weights, slot_row, k, H, out); break;
    }
    return hipGetLastError();
  }
  const int64_t nchunk = (H / 4 + 255) / 256;
  const int64_t split = std::max<int64_t>(1, std::min<int64_t>(nchunk, 2048 / std::max<int64_t>(T, 1)));
  const dim3 grid((unsigned)T, (unsigned)split);
  switch (k) {
    case 2: k_finalize<2, 256><<<grid, 256, 0, st>>>(y2, weights, slot_row, k, H, out); break;
    case 4: k_finalize<4, 256><<<grid, 256, 0, st>>>(y2, weights, slot_row, k, H, out); break;
    case 6: k_finalize<6, 256><<<grid, 256, 0, st>>>(y2, weights, slot_row, k, H, out); break;
    case 8: k_finalize<8, 256><<<grid, 256, 0, st>>>(y2, weights, slot_row, k, H, out); break;
    default: k_finalize<0, 256><<<grid, 256, 0, st>>>(y2, weights, slot_row, k, H, out); break;
  }
  return hipGetLastError();
}

}  // namespace moe
