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
#include "moe_common.h"

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

// One block per token row: x bf16 [T, H] -> codes E4M3 [T, H], scales [T].
// H % 8 == 0.
__global__ __launch_bounds__(256) void k_quant_tokens(const uint16_t* __restrict__ x, int32_t H,
                                                      uint8_t* __restrict__ codes,
                                                      float* __restrict__ scales) {
  __shared__ float red[4];
  const int64_t t = blockIdx.x;
  const uint4* row = reinterpret_cast<const uint4*>(x + t * H);
  const int nv = H / 8;
  float amax = 0.0f;
  for (int i = threadIdx.x; i < nv; i += blockDim.x) {
    const uint4 u = row[i];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      amax = fmaxf(amax, fabsf(__uint_as_float(w[j] << 16)));
      amax = fmaxf(amax, fabsf(__uint_as_float(w[j] & 0xFFFF0000u)));
    }
  }
  amax = block_max256(amax, red);
  const float s = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
  uint2* out = reinterpret_cast<uint2*>(codes + t * H);
  for (int i = threadIdx.x; i < nv; i += blockDim.x) {
    const uint4 u = row[i];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    uint32_t c[2] = {0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = e4m3_encode(__fdiv_rn(__uint_as_float(w[j] << 16), s));
      const uint32_t hi = e4m3_encode(__fdiv_rn(__uint_as_float(w[j] & 0xFFFF0000u), s));
      c[j / 2] |= (lo | (hi << 8)) << (16 * (j & 1));
    }
    out[i] = make_uint2(c[0], c[1]);
  }
  if (threadIdx.x == 0) scales[t] = s;
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
      const float4 v = row[i];
      out[i] = make_uint2(bf16_bits(v.x) | (bf16_bits(v.y) << 16),
                          bf16_bits(v.z) | (bf16_bits(v.w) << 16));
    }
    if (threadIdx.x == 0) scales[r] = 1.0f;
    return;
  }
  float amax = 0.0f;
  for (int i = threadIdx.x; i < nv; i += blockDim.x) {
    const float4 v = row[i];
    amax = fmaxf(fmaxf(amax, fabsf(v.x)), fmaxf(fabsf(v.y), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
  amax = block_max256(amax, red);
  const float s = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
  uint32_t* out = reinterpret_cast<uint32_t*>(codes + r * I);
  for (int i = threadIdx.x; i < nv; i += blockDim.x) {
    const float4 v = row[i];
    out[i] = e4m3_encode(__fdiv_rn(v.x, s)) | (e4m3_encode(__fdiv_rn(v.y, s)) << 8) |
             (e4m3_encode(__fdiv_rn(v.z, s)) << 16) | (e4m3_encode(__fdiv_rn(v.w, s)) << 24);
  }
  if (threadIdx.x == 0) scales[r] = s;
}

// One block per token: out[t] = bf16(sum_j fl32(w[t,j] * y2[row(t,j)])), the
// float32 sum taken in slot order.  H % 4 == 0.
__global__ __launch_bounds__(256) void k_finalize(const float* __restrict__ y2,
                                                  const float* __restrict__ weights,
                                                  const int32_t* __restrict__ slot_row,
                                                  int32_t k, int32_t H,
                                                  uint16_t* __restrict__ out) {
  const int64_t t = blockIdx.x;
  const int nv = H / 4;
  for (int i = blockIdx.y * blockDim.x + threadIdx.x; i < nv; i += gridDim.y * blockDim.x) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const float w = weights[t * k + j];
      const float4 y = reinterpret_cast<const float4*>(y2 + (int64_t)slot_row[t * k + j] * H)[i];
      acc.x = __fadd_rn(acc.x, __fmul_rn(w, y.x));
      acc.y = __fadd_rn(acc.y, __fmul_rn(w, y.y));
      acc.z = __fadd_rn(acc.z, __fmul_rn(w, y.z));
      acc.w = __fadd_rn(acc.w, __fmul_rn(w, y.w));
    }
    reinterpret_cast<uint2*>(out + t * H)[i] =
        make_uint2(bf16_bits(acc.x) | (bf16_bits(acc.y) << 16),
                   bf16_bits(acc.z) | (bf16_bits(acc.w) << 16));
  }
}

hipError_t launch_quant_tokens(const uint16_t* x, int64_t T, int32_t H, uint8_t* codes,
                               float* scales, hipStream_t st) {
  if (T == 0) return hipSuccess;
  k_quant_tokens<<<(unsigned)T, 256, 0, st>>>(x, H, codes, scales);
  return hipGetLastError();
}

hipError_t launch_requant(const float* h, int64_t rows, int32_t I, int afmt_bf16,
                          uint8_t* codes, float* scales, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  k_requant<<<(unsigned)rows, 256, 0, st>>>(h, I, afmt_bf16, codes, scales);
  return hipGetLastError();
}

hipError_t launch_finalize(const float* y2, const float* weights, const int32_t* slot_row,
                           int64_t T, int32_t k, int32_t H, uint16_t* out, hipStream_t st) {
  if (T == 0) return hipSuccess;
  // one block per (token, 1024 columns)
  dim3 grid((unsigned)T, (unsigned)((H / 4 + 255) / 256));
  k_finalize<<<grid, 256, 0, st>>>(y2, weights, slot_row, k, H, out);
  return hipGetLastError();
}

}  // namespace moe
