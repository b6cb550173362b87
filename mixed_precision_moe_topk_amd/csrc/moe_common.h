// Shared device helpers and launch-parameter structs of the fused MoE library
// (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------- constants
constexpr int kWave = 64;
constexpr int kKStep = 128;        // K consumed by one 16x16x128 MFMA
constexpr int kMxBlock = 32;       // elements per E8M0 scale (OCP MX block)
constexpr int kInt4Group = 128;    // elements per INT4 group scale
constexpr int kRouteChunkTokens = 64;  // tokens per routing chunk (one wave)
constexpr int kRouteGroupChunks = 16;  // chunks per block of the routing count kernel
constexpr int kMaxTopK = 16;
constexpr int kMaxExperts = 1024;

enum Variant : int {
  kMxfp4Fp8 = 0,   // E2M1 weights (E8M0 / 32) x per-token E4M3 activations
  kMxfp4Bf16 = 1,  // E2M1 weights (E8M0 / 32) x bf16 activations
  kInt4Fp8 = 2,    // INT4 weights (fp32 / 128) x per-token E4M3 activations
  kMxfp4Mxfp8 = 3, // E2M1 weights (E8M0 / 32) x E4M3 activations (E8M0 / 32)
  kMxfp4Mxfp4 = 4, // E2M1 weights (E8M0 / 32) x E2M1 activations (E8M0 / 32), W4A4
};

// Weights and activations both carry E8M0 block scales, applied by the MFMA.
constexpr bool a_blockscaled(int v) { return v == kMxfp4Mxfp8 || v == kMxfp4Mxfp4; }
// E2M1 weights on the block-scaled MFMA (E4M3 or E2M1 activations).
constexpr bool scaled_fp4(int v) { return v == kMxfp4Fp8 || v == kMxfp4Mxfp8 || v == kMxfp4Mxfp4; }
// E2M1 activations: the A operand is 4 registers of 32 consecutive k per lane
// (64 bytes per row and 128-wide K step) and the MFMA runs at the FP4 rate.
constexpr bool a_fp4(int v) { return v == kMxfp4Mxfp4; }
// MFMA format code of the A operand (0 E4M3, 4 E2M1).
constexpr int a_fmt(int v) { return a_fp4(v) ? 4 : 0; }

// Work-map entry of the grouped GEMMs: rows [row0, row0 + nrows) of expert
// `expert` (entries are grouped by expert, in expert order).
struct Tile {
  int32_t expert;
  int32_t row0;
  int32_t nrows;
  int32_t pad;
};

// Block -> (tile, N-tile) map shared by the GEMM kernels.  Block b runs on
// XCD b % 8 (each XCD has its own L2); q = b / 8, x = b % 8.
//   pair = 0: M-tile m = 8 (q / n_tiles) + x, N-tile q % n_tiles: one M-tile's
//     N-tiles run back to back on one XCD and share its activation rows in
//     that L2, while neighbouring M-tiles run at the same time on the other
//     XCDs (4 % faster than the plain order b -> (b / n_tiles, b % n_tiles) on
//     the 4096-token prefill GEMM1; an XCD-contiguous remap of whole item
//     ranges was slower).
//   pair = 1: the adjacent M-tiles 16 g + 2 x and 16 g + 2 x + 1 (g = q /
//     (2 n_tiles)) run N-tile major on XCD x, so the two blocks that read one
//     weight slice start back to back on one L2.  Chosen by the host when the
//     rows average at least one tile per expert, so that adjacent M-tiles are
//     mostly one expert's (16384-token prefill, ~5 M-tiles per active expert,
//     same-box pairs on three boxes: layer -0.5 to -1.7 %, GEMM2 -2 to -3 %,
//     GEMM1 -2 to +0.6 %; on the shapes whose experts fill one tile it was
//     0.2-1.3 % slower).
// The grid is rounded up to a multiple of 16 * n_tiles blocks (gemm_blocks)
// so either map covers every item; blocks past the last M-tile return false.
__device__ __forceinline__ bool work_item(const Tile* tiles, const int32_t* num_tiles,
                                          int32_t n_tiles, int32_t pair, Tile* tile, int* nt) {
  const int64_t b = blockIdx.x, q = b >> 3, x = b & 7;
  int64_t m;
  if (pair) {
    const int64_t g = q / (2 * n_tiles), r = q % (2 * n_tiles);
    m = 16 * g + 2 * x + (r & 1);
    *nt = (int)(r >> 1);
  } else {
    m = (q / n_tiles) * 8 + x;
    *nt = (int)(q % n_tiles);
  }
  if (m >= *num_tiles) return false;
  *tile = tiles[m];
  return true;
}
// Grid size of a GEMM launch covering max_tiles M-tiles (see work_item).
inline int64_t gemm_blocks(int64_t max_tiles, int32_t n_tiles) {
  return ((max_tiles + 15) / 16) * 16 * n_tiles;
}

// ---------------------------------------------------------------- vectors
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v2s __attribute__((ext_vector_type(2)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- numerics
// Nearest E2M1 magnitude code (0, 0.5, 1, 1.5, 2, 3, 4, 6 -> 0..7) of a
// non-negative value, ties to the even code, saturating at 6.
__device__ __forceinline__ uint32_t e2m1_magnitude_code(float v_abs) {
  return (v_abs > 0.25f) + (v_abs >= 0.75f) + (v_abs > 1.25f) + (v_abs >= 1.75f) +
         (v_abs > 2.5f) + (v_abs >= 3.5f) + (v_abs > 5.0f);
}

// Streaming (non-temporal) 16-byte load, for data read exactly once: h by the
// FC2 quantiser and y2 by the finalize (8-10 % faster than cached loads on
// the prefill finalize).
__device__ __forceinline__ float4 load_stream(const float4* p) {
  const v4f q = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
  return make_float4(q[0], q[1], q[2], q[3]);
}

// OCP MX shared exponent of a 32-element block: floor(log2 amax) - EMAX
// (EMAX 8 for E4M3 elements, 2 for E2M1), clamped to [-127, 127]; 0 for an
// all-zero block (E8M0 code 127).
template <int EMAX>
__device__ __forceinline__ int mx_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  const uint32_t b = __float_as_uint(amax);
  const int e = (int)((b >> 23) & 0xFFu);
  const int fl = e ? e - 127 : (31 - __clz(b & 0x7FFFFFu)) - 149;  // floor(log2 amax)
  return min(max(fl - EMAX, -127), 127);
}

// E4M3 codes of two floats of magnitude at most 448, as bytes 0 and 1:
// gfx950's v_cvt_pk_fp8_f32 (OCP E4M3 "FN": bias 7, round to nearest even,
// sign kept when the magnitude rounds to zero, 2^-9-spaced codes below 2^-6).
// On the device it gave the same code as a bit-manipulation encoder of that
// definition for every float32 of magnitude <= 464, of either sign; callers
// clamp larger magnitudes to 448 first (saturation).
__device__ __forceinline__ uint32_t e4m3_pk(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// fl32(v / s) as far as its E4M3 code goes, with inv = fl32(1 / s): the
// product v * inv is within 2 ulp of the IEEE quotient fl32(v / s) (each of
// the two roundings contributes at most 2^-24 relative error), so both lie on
// the same side of every E4M3 rounding midpoint, and encode alike, unless
// the product is within 2 ulp of a midpoint (the 20 bits below the E4M3
// mantissa equal 0x80000 +- 2) or below 2^-6, where the E4M3 grid is
// uniform and midpoints sit at other bit positions; those rare values take
// the exact quotient, as do non-finite products (a tiny s whose reciprocal
// overflows).  Saves the ~10-instruction IEEE division per element.
__device__ __forceinline__ float div_for_e4m3(float v, float s, float inv) {
  const float q = v * inv;
  const uint32_t a = __float_as_uint(q) & 0x7FFFFFFFu;
  const bool exact = a < 0x3C800000u || a >= 0x7F800000u || ((a & 0xFFFFFu) - 0x7FFFEu) <= 4u;
  return exact ? __fdiv_rn(v, s) : q;
}

// float32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_bits(float v) {
  uint32_t b = __float_as_uint(v);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return b >> 16;
}

__device__ __forceinline__ float e8m0_to_float(uint32_t c) {
  // 2^(c-127); c = 0 is the float32 subnormal 2^-127
  return __uint_as_float(c ? (c << 23) : 0x00400000u);
}

// E4M3 codes of the magnitudes 0..7 (byte j of the 8-byte table {hi:lo}):
//   0:00 1:38 2:40 3:44 4:48 5:4A 6:4C 7:4E.  Every INT4 value is exact in
// E4M3; the sign is bit 7 of the code.
constexpr uint32_t kI4MagLo = 0x44403800u, kI4MagHi = 0x4E4C4A48u;

// Four sign-magnitude INT4 nibbles, one per byte (bits 0-2 magnitude, bit 3
// sign, bits 4-7 zero) -> four E4M3 codes.
__device__ __forceinline__ uint32_t int4sm_to_e4m3(uint32_t nib4) {
  const uint32_t mag = __builtin_amdgcn_perm(kI4MagHi, kI4MagLo, nib4 & 0x07070707u);
  return mag | ((nib4 & 0x08080808u) << 4);
}

// ---------------------------------------------------------------- wave ops
__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// ---------------------------------------------------------------- params
struct RouteParams {
  const float* logits;     // [T, E]
  int64_t tokens;
  int32_t experts;
  int32_t top_k;
  int32_t* ids;            // [T, k]
  float* weights;          // [T, k]
  int32_t* chunk_counts;   // [nchunks, E] then the group counts [ngroups, E]
  int32_t nchunks;         // ceil(T / kRouteChunkTokens)
  int32_t* offsets;        // [E + 1]
  int32_t* row_token;      // [T*k]
  int32_t* slot_row;       // [T*k]
  Tile* tiles;             // [max_tiles]
  int32_t* num_tiles;      // [1]
  int32_t tile_m;
};

struct GemmParams {
  const uint8_t* a;            // FC1: token rows (E4M3 or bf16); FC2: expanded rows
  int64_t a_stride;            // bytes per A row
  const int32_t* row_token;    // FC1 gather map (expanded row -> token); null for FC2
  const float* row_scale;      // FC1: per-token scale; FC2: per-row scale; null for bf16 and MXFP8
  const uint8_t* a_scale;      // MXFP8: E8M0 scales of A in MFMA scale order (FC1 rows gathered); else null
  int64_t a_scale_stride;      // bytes per A row of a_scale (mx_scale_row_bytes(K))
  const uint8_t* w;            // packed weights of expert 0 of this matrix
  int64_t w_expert_stride;     // bytes between experts
  const uint8_t* s;            // scales of expert 0 of this matrix
  int64_t s_expert_stride;
  const Tile* tiles;
  const int32_t* num_tiles;
  int32_t n_tiles;             // N / BN
  int32_t pair_m;              // block map: 1 pairs adjacent M-tiles per XCD (see work_item)
  int32_t K;
  int32_t N;                   // device columns (FC1: 2I interleaved gate/up; FC2: H)
  float* out;                  // FC1: h [rows, N/2]; FC2: y2 [rows, N]
  int64_t out_stride;          // floats per output row
  // FC1 with MX activations and tiles whose waves hold whole 32-column
  // blocks of h: when q_out is set, the epilogue writes the FC2 input (E4M3 or
  // packed E2M1 codes + E8M0 codes in MFMA scale order) instead of h
  uint8_t* q_out;
  int64_t q_stride;            // bytes per q_out row
  uint8_t* q_bscales;
  int64_t q_bstride;           // bytes per q_bscales row (mx_scale_row_bytes(N/2))
};

// E8M0 block scales of MXFP8 activations, stored in the order the block-scaled
// MFMA takes them: per row, one 16-byte group per four 128-wide K steps; in a
// group, the dword of k-block g (elements [32g, 32g + 32) of a step) holds
// the scales of the four steps in bytes 0..3.  Lane l of an MFMA then loads
// the dword of its row and of k-block l/16 once per four steps and selects
// the step's byte with the MFMA's scale byte select, as for the weights.
__host__ __device__ constexpr int64_t mx_scale_row_bytes(int64_t cols) {
  return 16 * ((cols + 511) / 512);
}
__host__ __device__ constexpr int64_t mx_scale_offset(int64_t kb) {  // kb = col / 32
  return 16 * (kb >> 4) + 4 * (kb & 3) + ((kb >> 2) & 3);
}

// ---------------------------------------------------------------- launchers
hipError_t launch_route(const RouteParams& p, hipStream_t st);
// The routing index alone (the kernels after the router): count / scan /
// scatter, or the single-block kernel for at most 64 tokens.
hipError_t launch_route_index(const RouteParams& p, hipStream_t st);
// Activation quantisation modes of the token and FC2-input quantisers.
enum QuantMode : int { kQuantFp8Row = 0, kQuantBf16 = 1, kQuantMxfp8 = 2, kQuantMxfp4 = 3 };
// FP8 rows: codes + one float scale per row; MXFP8 / MXFP4: E4M3 codes [C] /
// packed E2M1 codes [C/2] + E8M0 per 32 (bscales [rows][mx_scale_row_bytes(C)]
// in MFMA scale order, row scales written as 1.0); BF16: bits, scale 1.
hipError_t launch_quant_tokens(const uint16_t* x, int64_t T, int32_t H, int mode,
                               uint8_t* codes, float* scales, uint8_t* bscales, hipStream_t st);
// The router and the token quantiser (mode kQuantFp8Row / kQuantMxfp8 /
// kQuantMxfp4) in one launch, then the routing index: the same outputs as
// launch_route followed by launch_quant_tokens.
hipError_t launch_router_quant(const RouteParams& p, const uint16_t* x, int32_t H, int mode,
                               uint8_t* codes, float* scales, uint8_t* bscales, hipStream_t st);
hipError_t launch_requant(const float* h, int64_t rows, int32_t I, int mode, uint8_t* codes,
                          float* scales, uint8_t* bscales, hipStream_t st);
hipError_t launch_finalize(const float* y2, const float* weights, const int32_t* slot_row,
                           int64_t T, int32_t k, int32_t H, uint16_t* out, hipStream_t st);
hipError_t launch_gemm(int variant, bool fc1, int cfg, const GemmParams& p, int64_t max_tiles,
                       hipStream_t st);
hipError_t launch_prepare(int wfmt_int4, const float* w, int32_t n_experts, int32_t N,
                          int32_t K, bool interleave_gate_up, uint8_t* codes,
                          int64_t codes_stride, uint8_t* scales, int64_t scales_stride,
                          hipStream_t st);
hipError_t launch_unpack(int wfmt_int4, const uint8_t* codes, int64_t codes_stride,
                         const uint8_t* scales, int64_t scales_stride, int32_t n_experts,
                         int32_t N, int32_t K, bool interleave_gate_up, uint8_t* out_codes,
                         uint8_t* out_scales, hipStream_t st);

// GEMM tile configurations (rows x device columns per block tile), chosen by
// the mean rows per expert.  BF16 activations keep the register-direct kernel;
// E4M3 activations use the LDS-staged kernels for the two larger shapes: A in
// LDS for 64 x 256; for the largest shape both operands in LDS with 8 waves,
// filled by direct-to-LDS loads for MXFP4 (160 x 512) and through registers
// for INT4 (128 x 256, whose E4M3 expansion of the weights needs the
// registers the larger tile would take).
struct GemmCfg {
  int nw, waves_m, wm, wn;  // waves per block, wave rows, 16x16 tiles per wave (M, N)
  int bm() const { return 16 * waves_m * wm; }
  int bn() const { return 16 * (nw / waves_m) * wn; }
};
constexpr int kNumGemmCfg = 3;
inline GemmCfg gemm_cfg(int i, int variant) {
  switch (i) {
    case 0: return GemmCfg{4, 1, 1, 4};                                        // 16 x 256
    case 1: return variant == kMxfp4Bf16 ? GemmCfg{4, 1, 3, 2}    // 48 x 128
             : variant == kInt4Fp8 ? GemmCfg{8, 1, 4, 4}     // 64 x 512
                                   : GemmCfg{4, 1, 4, 4};  // 64 x 256
    default:
      return variant == kMxfp4Bf16 ? GemmCfg{4, 2, 4, 4}    // 128 x 128
             : variant == kMxfp4Mxfp8 ? GemmCfg{8, 2, 5, 8}  // 160 x 512
             : variant == kMxfp4Mxfp4 ? GemmCfg{8, 2, 5, 8}  // 160 x 512
             : variant == kMxfp4Fp8 ? GemmCfg{8, 2, 5, 8}    // 160 x 512
                                  : GemmCfg{8, 2, 4, 4};   // 128 x 256
  }
}

}  // namespace moe
