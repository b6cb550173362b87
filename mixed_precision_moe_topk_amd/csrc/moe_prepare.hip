// Weight preparation: float32 expert masters -> MXFP4 or INT4 codes and
// scales in the device layout the GEMMs read, and the inverse (device layout
// -> canonical row-major codes) used to check the codes bit for bit.
//
// Formats (flashinfer PR #3738, "perf: optimize MXFP4xBF16 & INT4xFP8 and add
// MXFP4xFP8 CUTLASS MoE backend for SM90", Description):
//   MXFP4: E2M1 elements, one E8M0 scale per 32 elements along K; the shared
//          exponent is floor(log2(block amax)) - 2 (OCP MX v1.0 conversion:
//          emax of E2M1 is 2), clamped to the E8M0 range, elements rounded to
//          nearest even on the E2M1 grid and clamped to +-6.
//   INT4:  symmetric codes with one float32 scale per 128 elements along K,
//          s = amax/7, q = round-half-even(w/s) (the quantiser never yields -8).
// Device layout ("folded" scales: the same packed layout serves every K tile,
// Implementation Notes of the same page):
//   codes  [N/16][K/128][64 lanes][16 bytes]; lane l = (row % 16) + 16*g holds
//          the 32 elements k = 128*ks + 32*g + [0, 32) of row 16*nb + l%16 --
//          exactly the per-lane operand of a 16x16x128 MFMA.
//   MXFP4: natural nibble order (element 2i low nibble); scales
//          [N/16][ceil(K/512)][64 lanes][4 bytes], byte j = E8M0 code of
//          (row, 32-block 4*(4*kk+j) + g); unused bytes are 0x7F.
//   INT4:  sign-magnitude nibbles (bit 3 sign), and inside every 32-bit word
//          the element at offset o (0..7) sits in nibble position 2o (o < 4) or
//          2(o-4)+1 (o >= 4), so that masking even/odd nibbles yields four
//          consecutive elements per byte lane; scales [N/16][K/128][16] fp32.
//   W1 rows are stored as alternating 16-row blocks gate0, up0, gate1, up1, ...
//   (canonical rows [0, I) are gate, [I, 2I) up) so that one wave's output
//   tile holds matching gate and up columns for the fused SwiGLU.
#include "moe_common.h"

namespace moe {

__device__ __forceinline__ int64_t canon_row(int64_t dn, int32_t N, bool inter) {
  if (!inter) return dn;
  const int64_t db = dn >> 4, r = dn & 15;
  return (db & 1) * (N / 2) + (db >> 1) * 16 + r;
}


// thread per (device row, 32-block)
__global__ __launch_bounds__(256) void k_prepare_mxfp4(const float* __restrict__ w, int32_t N,
                                                       int32_t K, int inter,
                                                       uint8_t* __restrict__ codes,
                                                       int64_t codes_stride,
                                                       uint8_t* __restrict__ scales,
                                                       int64_t scales_stride) {
  const int e = blockIdx.y;
  const int nb32 = K / 32;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)N * nb32) return;
  const int64_t dn = idx / nb32;
  const int b = (int)(idx % nb32);
  const int64_t cn = canon_row(dn, N, inter != 0);
  const float4* src = reinterpret_cast<const float4*>(w + ((int64_t)e * N + cn) * K + 32 * b);
  float v[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 f = src[i];
    v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  int X = 0;
  uint32_t scode = 127;
  if (amax > 0.0f) {
    const uint32_t ab = __float_as_uint(amax);
    const int e2 = (ab >= 0x00800000u) ? (int)(ab >> 23) - 127 : (31 - __clz(ab)) - 149;
    X = max(e2 - 2, -127);
    scode = (uint32_t)(X + 127);
  }
  const float inv = __uint_as_float((uint32_t)(127 - X) << 23);  // 2^-X, normal for X in [-127, 125]
  uint32_t out[4] = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t sgn = (__float_as_uint(v[i]) >> 31) << 3;
    const uint32_t c = e2m1_magnitude_code(fabsf(v[i]) * inv) | sgn;
    out[i / 8] |= c << (4 * (i % 8));
  }
  const int KS = K / kKStep, KS4 = (KS + 3) / 4;
  const int ks = b / 4, g = b % 4;
  const int lane = (int)(dn & 15) + 16 * g;
  const int64_t nb = dn >> 4;
  uint8_t* cbase = codes + e * codes_stride;
  *reinterpret_cast<uint4*>(cbase + ((nb * KS + ks) * 64 + lane) * 16) =
      make_uint4(out[0], out[1], out[2], out[3]);
  uint8_t* sbase = scales + e * scales_stride;
  sbase[((nb * KS4 + ks / 4) * 64 + lane) * 4 + (ks % 4)] = (uint8_t)scode;
}

// thread per (device row, 128-group)
__global__ __launch_bounds__(256) void k_prepare_int4(const float* __restrict__ w, int32_t N,
                                                      int32_t K, int inter,
                                                      uint8_t* __restrict__ codes,
                                                      int64_t codes_stride,
                                                      uint8_t* __restrict__ scales,
                                                      int64_t scales_stride) {
  const int e = blockIdx.y;
  const int KS = K / kKStep;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)N * KS) return;
  const int64_t dn = idx / KS;
  const int ks = (int)(idx % KS);
  const int64_t cn = canon_row(dn, N, inter != 0);
  const float4* src = reinterpret_cast<const float4*>(w + ((int64_t)e * N + cn) * K + kKStep * ks);
  float amax = 0.0f;
  for (int i = 0; i < 32; ++i) {
    const float4 f = src[i];
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(f.x), fabsf(f.y)), fmaxf(fabsf(f.z), fabsf(f.w))));
  }
  const float s = amax > 0.0f ? __fdiv_rn(amax, 7.0f) : 1.0f;
  const int64_t nb = dn >> 4;
  uint8_t* cbase = codes + e * codes_stride;
  for (int g = 0; g < 4; ++g) {
    uint32_t out[4] = {0, 0, 0, 0};
    for (int d = 0; d < 4; ++d) {
      const float4 lo = src[8 * g + 2 * d];
      const float4 hi = src[8 * g + 2 * d + 1];
      const float vals[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      uint32_t word = 0;
      for (int o = 0; o < 8; ++o) {
        float q = __builtin_rintf(__fdiv_rn(vals[o], s));
        q = fminf(fmaxf(q, -8.0f), 7.0f);
        const int qi = (int)q;
        const uint32_t nib = (uint32_t)(qi < 0 ? -qi : qi) | (qi < 0 ? 8u : 0u);
        const int pos = (o < 4) ? 2 * o : 2 * (o - 4) + 1;
        word |= nib << (4 * pos);
      }
      out[d] = word;
    }
    const int lane = (int)(dn & 15) + 16 * g;
    *reinterpret_cast<uint4*>(cbase + ((nb * KS + ks) * 64 + lane) * 16) =
        make_uint4(out[0], out[1], out[2], out[3]);
  }
  float* sbase = reinterpret_cast<float*>(scales + e * scales_stride);
  sbase[(nb * KS + ks) * 16 + (dn & 15)] = s;
}

// inverse: device layout -> canonical codes [N, K/2] and scales
__global__ __launch_bounds__(256) void k_unpack_mxfp4(const uint8_t* __restrict__ codes,
                                                      int64_t codes_stride,
                                                      const uint8_t* __restrict__ scales,
                                                      int64_t scales_stride, int32_t N, int32_t K,
                                                      int inter, uint8_t* __restrict__ oc,
                                                      uint8_t* __restrict__ os) {
  const int e = blockIdx.y;
  const int nb32 = K / 32;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)N * nb32) return;
  const int64_t dn = idx / nb32;
  const int b = (int)(idx % nb32);
  const int64_t cn = canon_row(dn, N, inter != 0);
  const int KS = K / kKStep, KS4 = (KS + 3) / 4;
  const int ks = b / 4, g = b % 4;
  const int lane = (int)(dn & 15) + 16 * g;
  const int64_t nb = dn >> 4;
  const uint4 c = *reinterpret_cast<const uint4*>(codes + e * codes_stride +
                                                  ((nb * KS + ks) * 64 + lane) * 16);
  *reinterpret_cast<uint4*>(oc + ((int64_t)e * N + cn) * (K / 2) + 16 * b) = c;
  os[((int64_t)e * N + cn) * nb32 + b] =
      scales[e * scales_stride + ((nb * KS4 + ks / 4) * 64 + lane) * 4 + (ks % 4)];
}

__global__ __launch_bounds__(256) void k_unpack_int4(const uint8_t* __restrict__ codes,
                                                     int64_t codes_stride,
                                                     const uint8_t* __restrict__ scales,
                                                     int64_t scales_stride, int32_t N, int32_t K,
                                                     int inter, uint8_t* __restrict__ oc,
                                                     uint8_t* __restrict__ os) {
  const int e = blockIdx.y;
  const int KS = K / kKStep;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)N * KS) return;
  const int64_t dn = idx / KS;
  const int ks = (int)(idx % KS);
  const int64_t cn = canon_row(dn, N, inter != 0);
  const int64_t nb = dn >> 4;
  uint8_t* dst = oc + ((int64_t)e * N + cn) * (K / 2) + 64 * ks;
  for (int g = 0; g < 4; ++g) {
    const int lane = (int)(dn & 15) + 16 * g;
    const uint4 c = *reinterpret_cast<const uint4*>(codes + e * codes_stride +
                                                    ((nb * KS + ks) * 64 + lane) * 16);
    const uint32_t words[4] = {c.x, c.y, c.z, c.w};
    uint32_t outw[4];
    for (int d = 0; d < 4; ++d) {
      uint32_t o32 = 0;
      for (int o = 0; o < 8; ++o) {
        const int pos = (o < 4) ? 2 * o : 2 * (o - 4) + 1;
        const uint32_t nib = (words[d] >> (4 * pos)) & 0xF;
        const int mag = nib & 7;
        const int q = (nib & 8) ? -mag : mag;
        o32 |= ((uint32_t)q & 0xF) << (4 * o);
      }
      outw[d] = o32;
    }
    *reinterpret_cast<uint4*>(dst + 16 * g) = make_uint4(outw[0], outw[1], outw[2], outw[3]);
  }
  reinterpret_cast<float*>(os)[((int64_t)e * N + cn) * KS + ks] =
      reinterpret_cast<const float*>(scales + e * scales_stride)[(nb * KS + ks) * 16 + (dn & 15)];
}

hipError_t launch_prepare(int wfmt_int4, const float* w, int32_t n_experts, int32_t N,
                          int32_t K, bool interleave_gate_up, uint8_t* codes,
                          int64_t codes_stride, uint8_t* scales, int64_t scales_stride,
                          hipStream_t st) {
  if (n_experts == 0) return hipSuccess;
  const int64_t items = wfmt_int4 ? (int64_t)N * (K / kKStep) : (int64_t)N * (K / 32);
  dim3 grid((unsigned)((items + 255) / 256), (unsigned)n_experts);
  if (wfmt_int4)
    k_prepare_int4<<<grid, 256, 0, st>>>(w, N, K, interleave_gate_up, codes, codes_stride,
                                         scales, scales_stride);
  else
    k_prepare_mxfp4<<<grid, 256, 0, st>>>(w, N, K, interleave_gate_up, codes, codes_stride,
                                          scales, scales_stride);
  return hipGetLastError();
}

hipError_t launch_unpack(int wfmt_int4, const uint8_t* codes, int64_t codes_stride,
                         const uint8_t* scales, int64_t scales_stride, int32_t n_experts,
                         int32_t N, int32_t K, bool interleave_gate_up, uint8_t* out_codes,
                         uint8_t* out_scales, hipStream_t st) {
  if (n_experts == 0) return hipSuccess;
  const int64_t items = wfmt_int4 ? (int64_t)N * (K / kKStep) : (int64_t)N * (K / 32);
  dim3 grid((unsigned)((items + 255) / 256), (unsigned)n_experts);
  if (wfmt_int4)
    k_unpack_int4<<<grid, 256, 0, st>>>(codes, codes_stride, scales, scales_stride, N, K,
                                        interleave_gate_up, out_codes, out_scales);
  else
    k_unpack_mxfp4<<<grid, 256, 0, st>>>(codes, codes_stride, scales, scales_stride, N, K,
                                         interleave_gate_up, out_codes, out_scales);
  return hipGetLastError();
}

}  // namespace moe
