/*
 * C ABI of the MI355X (gfx950) fused mixed-precision Mixture-of-Experts layer.
 *
 * The layer (flashinfer PR #3738, "perf: optimize MXFP4xBF16 & INT4xFP8 and add
 * MXFP4xFP8 CUTLASS MoE backend for SM90", Description and Implementation
 * Notes; flashinfer PR #4793, "Unify MoE CuTe DSL dispatch to be dtype
 * agnostic", for the routing outputs and the finalize fusion):
 *
 *   1. top-k routing on float32 logits: the k largest logits per token (equal
 *      logits ordered by the smaller expert index), weights = softmax over the
 *      k selected logits;
 *   2. FP8 activations: per-token E4M3 quantisation, s = amax/448, codes of
 *      x/s rounded to nearest even and saturated at 448; MXFP8 / MXFP4
 *      activations: per 32 elements the OCP MX exponent X = floor(log2 amax)
 *      - 8 / - 2 and E4M3 / E2M1 codes of x * 2^-X (flashinfer PR #4793,
 *      Walkthrough: MXFP8 dispatch packing, MXFP4 activation pack); BF16
 *      activations are used as they are;
 *   3. grouped GEMM1 (gate+up) over the routed rows of each expert, times the
 *      token scale, then h = silu(gate) * up in float32;
 *   4. FC2 input: the activation format's quantiser applied to each row of h
 *      (per-row E4M3, MXFP8 or MXFP4); BF16 activations -> bf16(h);
 *   5. grouped GEMM2, times the row scale (float32 y2; block scales of the MX
 *      formats are applied inside the matrix product);
 *   6. out[t] = bf16(sum over the k slots of weight * y2), float32 sum.
 *
 * Weight formats: MXFP4 (E2M1 codes, one E8M0 scale per 32 elements along K)
 * or INT4 (symmetric codes, one float32 scale per 128 elements along K).
 * Supported combinations: MXFP4 x FP8, MXFP4 x BF16, INT4 x FP8, and with
 * block-scaled activations MXFP4 x MXFP8 and MXFP4 x MXFP4 (W4A4).
 *
 * Conventions
 *   - All tensors are dense row-major; "device" pointers are HIP device
 *     memory on the current device; the caller owns every buffer.
 *   - Every call is asynchronous on `stream` unless stated; no call
 *     synchronises the stream or allocates, except moe_run and moe_autotune
 *     (see below).
 *   - Errors are returned as moe_status; moe_last_error() gives a message
 *     for the calling thread.  Nothing is printed and nothing aborts.
 *   - Asynchronous device faults surface at the caller's next
 *     synchronisation.  With the environment variable MOE_SYNC_CHECK=1 every
 *     call synchronises and checks each kernel, so a fault names its kernel.
 *   - Pointers must be 16-byte aligned; hidden and inter must be multiples of
 *     128; 1 <= num_experts <= 1024; 1 <= top_k <= min(num_experts, 16).
 *   - Only gfx950 devices are supported (MOE_ERR_UNSUPPORTED otherwise).
 */
#ifndef MOE_AMD_MOE_H_
#define MOE_AMD_MOE_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 7

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* bad dims, pointers, alignment or ranges */
  MOE_ERR_UNSUPPORTED = 2, /* format combination or device not supported */
  MOE_ERR_WORKSPACE = 3,   /* caller workspace smaller than moe_workspace_query */
  MOE_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed */
  MOE_ERR_INTERNAL = 5
} moe_status;

typedef enum { MOE_W_MXFP4 = 0, MOE_W_INT4_G128 = 1 } moe_wfmt;
/* Activations: FP8_TOKEN = E4M3 with one float32 scale per token (and per FC2
 * input row); MXFP8 = E4M3 with one E8M0 scale per 32 consecutive elements of
 * a token (and of an FC2 input row), applied inside the block-scaled MFMA
 * (MXFP4 weights only); MXFP4 (W4A4) = E2M1 with one E8M0 scale per 32, the
 * weights' own quantiser, at the MFMA's FP4 rate (MXFP4 weights only); BF16 =
 * the activations as given. */
typedef enum { MOE_A_FP8_TOKEN = 0, MOE_A_BF16 = 1, MOE_A_MXFP8 = 2, MOE_A_MXFP4 = 3 } moe_afmt;

/* Shape and formats of one MoE layer.  W1 is [2*inter, hidden] per expert
 * (rows [0, inter) gate, [inter, 2*inter) up); W2 is [hidden, inter]. */
typedef struct {
  int32_t num_experts;
  int32_t hidden;
  int32_t inter;
  int32_t wfmt; /* moe_wfmt */
  int32_t afmt; /* moe_afmt */
} moe_dims;

/* Byte offsets of the intermediates inside a moe_run_ws workspace (for
 * inspection by tests; all regions are 256-byte aligned).
 *   ids         int32  [T, k]   selected experts, descending logit
 *   topk_w      float  [T, k]   routing weights
 *   offsets     int32  [E + 1]  first expanded row of each expert
 *   row_token   int32  [T*k]    token of each expanded row (expert-major,
 *                               then token, then slot)
 *   slot_row    int32  [T, k]   expanded row of each (token, slot)
 *   tok_codes   uint8  [T, H]   E4M3 token codes (FP8 and MXFP8 activations);
 *                      [T, H/2] E2M1 codes, element 2i in the low nibble (MXFP4)
 *   tok_scales  float  [T]      token scales (FP8 activations; 1.0 for MX formats)
 *   h           float  [T*k, I] SwiGLU output per expanded row (an empty
 *                               region, never written, when fc2_fused)
 *   fc2_codes   uint8  [T*k, I] E4M3 (FP8, MXFP8), [T*k, I/2] E2M1 (MXFP4) or
 *                               bf16 bits ([T*k, I] uint16)
 *   fc2_scales  float  [T*k]    per-row FC2 input scale (FP8; not written for
 *                               the MX formats and BF16)
 *   tok_bscales uint8  [T, 16*ceil(H/512)]   E8M0 block scales of the token
 *                                  codes (MXFP8, MXFP4), in matrix-core order:
 *                                  the scale of elements [32b, 32b + 32) of a
 *                                  row sits at byte 16*(b/16) + 4*(b%4) + (b/4)%4
 *   fc2_bscales uint8  [T*k, 16*ceil(I/512)] same for the FC2 codes (MXFP8, MXFP4)
 *   y2          float  [T*k, H] GEMM2 output per expanded row
 *   num_tiles   int32  [1]      GEMM work-map length; tile_m rows per tile
 * gemm_cfg is the tile configuration the call uses (tuned or default, see
 * moe_tune_set), max_tiles the bound on its work-map length.  fc2_fused = 1:
 * GEMM1 writes the FC2 input itself (MX activation formats: codes and block
 * scales; BF16: bf16(h)), so h is not written and fc2_scales are not set. */
typedef struct {
  size_t total;
  size_t ids, topk_w, chunk_counts, offsets, row_token, slot_row, tiles, num_tiles;
  size_t tok_codes, tok_scales, h, fc2_codes, fc2_scales, y2;
  int32_t tile_m;
  int32_t gemm_cfg;
  int64_t max_tiles;
  size_t tok_bscales, fc2_bscales;
  int32_t fc2_fused;
} moe_ws_layout;

/* Version of this ABI (MOE_ABI_VERSION of the header the library was built
 * with); a binding compares it with its own before any other call. */
int32_t moe_abi_version(void);

/* Message of the last failed call on this thread ("" if none).  Errors are
 * reported, never raised or printed: flashinfer PR #3614 ("fix: make the
 * cutlass MoE gemm profiler MXFP8-aware ...", Description) traces an
 * autotune crash to an assertion deep inside a kernel launcher; here a bad
 * argument is a status code and a message before any launch. */
const char* moe_last_error(void);

/* Bytes of the packed weights and of the scales for all experts (pure host
 * arithmetic; flashinfer PR #3738, Implementation Notes: one folded
 * weight-scale layout serves every K tile, so the sizes depend on the shape
 * and formats only, never on the tile configuration).  Per expert: codes (2*I*H + H*I)/2 bytes; scales
 * 2*I*ceil(H/512)*16 + H*ceil(I/512)*16 bytes (MXFP4) or
 * 4*(2*I*H + H*I)/128 bytes (INT4). */
moe_status moe_weights_query(const moe_dims* dims, size_t* weight_bytes, size_t* scale_bytes);

/* Quantises float32 master weights of experts [expert_begin, expert_begin +
 * expert_count) into the device layout (flashinfer PR #3738, Description:
 * MXFP4 weights with one E8M0 scale per 32 elements along K, INT4 weights
 * with group scales; Implementation Notes: weight preprocessing into a
 * folded weight-scale layout independent of the GEMM's K tile — here the
 * matrix-core operand order, with one 16-byte scale group per four K steps).
 *   w1: device float [expert_count, 2*inter, hidden]
 *   w2: device float [expert_count, hidden, inter]
 *   weights, scales: device buffers of moe_weights_query's sizes (all experts);
 *   only the slice of the given experts is written.
 * Quantisation (MXFP4: shared exponent floor(log2(block amax)) - 2, elements
 * rounded to nearest even on the E2M1 grid and clamped to +-6; INT4: scale
 * amax/7, codes round-half-even(w/s)) is deterministic and stream-ordered.
 * Call it repeatedly over expert chunks so that the float32 masters never
 * need to be resident at once. */
moe_status moe_prepare_weights(const moe_dims* dims, const float* w1, const float* w2,
                               int32_t expert_begin, int32_t expert_count, void* weights,
                               void* scales, hipStream_t stream);

/* Inverse of the device layout (moe_prepare_weights; flashinfer PR #3738,
 * Implementation Notes, folded weight-scale layout), for checking codes bit
 * for bit: writes the
 * canonical row-major codes and scales of experts [expert_begin,
 * expert_begin + expert_count) into device buffers
 *   w1q uint8 [n, 2*inter, hidden/2]   (element 2i in the low nibble;
 *                                        INT4 as two's complement)
 *   w1s uint8 [n, 2*inter, hidden/32]  (MXFP4 E8M0) or float [n, 2*inter, hidden/128] (INT4)
 *   w2q uint8 [n, hidden, inter/2]
 *   w2s uint8 [n, hidden, inter/32]    or float [n, hidden, inter/128]. */
moe_status moe_unpack_weights(const moe_dims* dims, const void* weights, const void* scales,
                              int32_t expert_begin, int32_t expert_count, void* w1q, void* w1s,
                              void* w2q, void* w2s, hipStream_t stream);

/* Workspace bytes moe_run_ws needs for num_tokens tokens and top_k (the
 * caller-owned workspace and its size query that flashinfer's fused MoE
 * keeps: PR #4411 page, "revert(moe): revert #3738 ...", Conflict
 * resolution, cutlass_fused_moe_workspace_size / workspace_buffer).  Errors:
 * MOE_ERR_INVALID_ARG for bad dims, num_tokens < 0 or > 2^26, top_k outside
 * [1, min(num_experts, 16)] or a null output pointer. */
moe_status moe_workspace_query(const moe_dims* dims, int64_t num_tokens, int32_t top_k,
                               size_t* bytes);

/* Offsets of the intermediates inside that workspace (same page and section
 * as moe_workspace_query; the tests read the routing maps, token codes and
 * GEMM outputs at these offsets).  Errors as moe_workspace_query. */
moe_status moe_workspace_layout(const moe_dims* dims, int64_t num_tokens, int32_t top_k,
                                moe_ws_layout* layout);

/* Runs the layer with a caller-owned workspace (flashinfer PR #3738,
 * Description: routing, expansion with runtime per-token FP8 quantisation,
 * grouped GEMM1 over MXFP4 / INT4 weights with the activation, grouped GEMM2
 * and the weighted top-k reduction; the caller-owned workspace as kept by
 * the PR #4411 page, Conflict resolution).
 *   hidden:        device bf16 bits [num_tokens, hidden]
 *   router_logits: device float [num_tokens, num_experts]; a NaN logit ranks
 *                  as -inf, so every selected id is a valid expert index; a
 *                  token whose largest selected logit is infinite (or whose
 *                  logits are all NaN) gets NaN weights and a NaN output row
 *   weights, scales: prepared by moe_prepare_weights for all experts
 *   out:           device bf16 bits [num_tokens, hidden], fully overwritten
 *   workspace:     device buffer of at least moe_workspace_query bytes
 * num_tokens = 0 returns MOE_OK without launching.  No allocation, no host
 * synchronisation (unless MOE_SYNC_CHECK=1) and no memset: the call can be
 * captured into a HIP graph (with stage timing off); the workspace needs no
 * initialisation. */
moe_status moe_run_ws(const moe_dims* dims, const void* hidden, int64_t num_tokens,
                      const float* router_logits, const void* weights, const void* scales,
                      int32_t top_k, void* out, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* Same as moe_run_ws (flashinfer PR #3738, Description), with a workspace the
 * library keeps per (device, stream) and grows stream-ordered
 * (hipMallocAsync) when a call needs more: the library-managed workspace the
 * fused MoE uses when the caller passes none (PR #4411 page, Conflict
 * resolution).  Calls on different streams use different workspaces; an
 * arena lives until moe_release_arenas or the end of the process.  Errors
 * as moe_run_ws, plus MOE_ERR_HIP when the arena cannot grow. */
moe_status moe_run(const moe_dims* dims, const void* hidden, int64_t num_tokens,
                   const float* router_logits, const void* weights, const void* scales,
                   int32_t top_k, void* out, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * layer, kernels and results as moe_run_ws, with the workspace taken from a
 * static device array of MOE_NOALLOC_SCRATCH_BYTES bytes that the library
 * holds on every device it runs on until the process ends.  The call
 * allocates nothing (no hipMalloc / hipFree, no allocating library routine)
 * and records no stage-trace events.  Every call on one device shares that
 * device's array, so calls that overlap in time on one device (different
 * streams or threads without ordering between them) race and corrupt each
 * other's intermediates; calls ordered on one stream are fine.  The array
 * needs no clearing: every region is written before it is read within a call.
 * Arguments as moe_run_ws.  Errors: as moe_run_ws; MOE_ERR_WORKSPACE (nothing
 * launched) when moe_workspace_query for these dims, num_tokens and top_k
 * exceeds MOE_NOALLOC_SCRATCH_BYTES — e.g. DeepSeek-V3 shapes (hidden 7168,
 * inter 2048, top-8) fit up to about 150 tokens; MOE_ERR_HIP if the device
 * address of the array cannot be looked up. */
#define MOE_NOALLOC_SCRATCH_BYTES (64ull << 20)
moe_status moe_run_noalloc(const moe_dims* dims, const void* hidden, int64_t num_tokens,
                           const float* router_logits, const void* weights, const void* scales,
                           int32_t top_k, void* out, hipStream_t stream);

/* Frees every workspace moe_run holds (all devices and streams).  Waits for
 * each device that holds one (hipDeviceSynchronize), so no call may be in
 * flight on another thread.  The next moe_run allocates again.  Errors:
 * MOE_ERR_HIP if a device call fails (the remaining arenas are still freed). */
moe_status moe_release_arenas(void);

/* Test hook for the FC2 input of the fused epilogues (flashinfer PR #3738,
 * Implementation Notes: tactics are checked for correctness against a
 * reference path).  enable = 1 (the default): GEMM1 writes the FC2 input
 * itself where the format and tile allow it (MX activation formats, BF16), so
 * float32 h is never stored.  enable = 0: GEMM1 stores h and the separate FC2
 * quantiser runs for every format; moe_workspace_layout then reports
 * fc2_fused = 0 and reserves h.  Both give the same FC2 bytes (the fused
 * epilogue applies the same quantiser to the same h values), which the
 * tests check bit for bit.  Process-wide; it changes the workspace size, so
 * set it only while no call is in flight.  Errors: MOE_ERR_INVALID_ARG unless
 * enable is 0 or 1. */
moe_status moe_set_fc2_fused(int32_t enable);

/* The routing step of the run calls alone, same kernels (flashinfer PR #4793,
 * Walkthrough: the fused MoE consumes the router's selected experts and final
 * scales; flashinfer PR #3738, Implementation Notes: the grouped GEMM's
 * per-expert work map is computed on the device before the GEMMs).
 *   router_logits:  device float [num_tokens, num_experts]; NaN ranks as
 *                   -inf (see moe_run_ws)
 *   ids:            device int32 [num_tokens, top_k] out: the k largest logits
 *                   per token in descending order, equal logits by the smaller
 *                   expert index
 *   weights:        device float [num_tokens, top_k] out: softmax over the k
 *                   selected logits, in the order of ids
 *   expert_offsets: device int32 [num_experts + 1] out: first expanded row of
 *                   each expert; expert_offsets[num_experts] = num_tokens*top_k
 *   row_token:      device int32 [num_tokens*top_k] out: token of each
 *                   expanded row (expert-major, then token, then slot)
 *   slot_row:       device int32 [num_tokens, top_k] out: expanded row of each
 *                   (token, slot)
 *   workspace:      device buffer of at least moe_workspace_query bytes for
 *                   the same dims, num_tokens and top_k; the routing scratch
 *                   (per-chunk and per-group counts) and the GEMM work map
 *                   are written to its chunk_counts, tiles and num_tiles
 *                   regions (moe_ws_layout)
 * The outputs may lie inside the workspace at the offsets moe_workspace_layout
 * gives for them (where moe_run_ws puts them).  num_tokens = 0 returns MOE_OK
 * without launching.  Errors as moe_run_ws. */
moe_status moe_route(const moe_dims* dims, const float* router_logits, int64_t num_tokens,
                     int32_t top_k, int32_t* ids, float* weights, int32_t* expert_offsets,
                     int32_t* row_token, int32_t* slot_row, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);

/* The token quantisation step of the run calls alone, same kernels
 * (flashinfer PR #3738, Implementation Notes: per-token activation scales
 * computed while the routed rows are expanded; flashinfer PR #4793,
 * Walkthrough: MXFP8 dispatch packing and the MXFP4 activation pack of the
 * w4a4 mode).
 *   hidden:       device bf16 bits [num_tokens, hidden]
 *   codes:        device uint8 out: [num_tokens, hidden] E4M3 (FP8_TOKEN,
 *                 MXFP8) or [num_tokens, hidden/2] E2M1 with element 2i in the
 *                 low nibble (MXFP4)
 *   scales:       device float [num_tokens] out: amax/448 (1.0 for an
 *                 all-zero token) for FP8_TOKEN; 1.0 for the MX formats
 *   block_scales: device uint8 [num_tokens, 16*ceil(hidden/512)] out: E8M0
 *                 codes per 32 elements in the matrix-core order described
 *                 at moe_ws_layout.tok_bscales (MXFP8, MXFP4); must be null
 *                 for FP8_TOKEN
 * BF16 activations have no quantisation step: MOE_ERR_UNSUPPORTED.
 * num_tokens = 0 returns MOE_OK without launching. */
moe_status moe_quantize_tokens(const moe_dims* dims, const void* hidden, int64_t num_tokens,
                               void* codes, float* scales, void* block_scales,
                               hipStream_t stream);

/* Tile configurations of the grouped GEMMs.  A call picks one of
 * MOE_NUM_GEMM_CFG configurations (0: 16-row tiles, 1: 48/64-row tiles, 2:
 * 128/160-row tiles; the exact shapes depend on the formats and are reported
 * by moe_workspace_layout as tile_m).  By default the choice follows the mean
 * rows per expert (T*k/E: <= 16 -> 0, <= 48 -> 1, else 2).  A tuned choice
 * overrides it for one layer shape (moe_dims), top_k and token bucket
 * ceil(log2 num_tokens) for the rest of the process (flashinfer PR #3738,
 * Implementation Notes: the MoE autotuner tunes both GEMMs over the tactics
 * per shape, validates each tactic's results before timing it, and tunes on
 * representative routing).  The workspace size never depends on the choice.
 * All three functions are thread-safe; tuned choices are shared by all
 * devices and streams of the process. */
#define MOE_NUM_GEMM_CFG 3

/* Sets (gemm_cfg in [0, MOE_NUM_GEMM_CFG)) or removes (gemm_cfg = -1) the
 * tuned configuration of the bucket of num_tokens (>= 1).  Host only. */
moe_status moe_tune_set(const moe_dims* dims, int64_t num_tokens, int32_t top_k,
                        int32_t gemm_cfg);

/* Forgets every tuned configuration.  Host only. */
moe_status moe_tune_clear(void);

/* Tunes the tile configuration on the caller's inputs (same arguments as
 * moe_run_ws; num_tokens >= 1; use routing as skewed as the real workload).
 * First runs the default configuration as the reference, then for every
 * configuration: one run whose output must match the reference (relative L2
 * <= 1e-3, same non-finite positions; the default itself is checked too), and
 * only if it matches, `iters` (1..1000) timed runs between HIP events on
 * `stream`.  Stores the fastest matching configuration for the bucket of
 * num_tokens and returns it in *chosen; cfg_ms (optional, MOE_NUM_GEMM_CFG
 * floats) receives each configuration's mean milliseconds per call, -1 for a
 * rejected one.  Unlike the run calls it allocates (its own workspace and
 * output, hipMalloc, freed before returning) and synchronises `stream`; the
 * caller's out buffer is not touched.  MOE_ERR_INTERNAL if no configuration
 * matches. */
moe_status moe_autotune(const moe_dims* dims, const void* hidden, int64_t num_tokens,
                        const float* router_logits, const void* weights, const void* scales,
                        int32_t top_k, int32_t iters, int32_t* chosen, float* cfg_ms,
                        hipStream_t stream);

/* Stage timing.  With mode MOE_TRACE_ALL every moe_run_ws / moe_run call
 * records a HIP event on its stream before its first kernel and after each
 * stage below; with MOE_TRACE_GEMM1 only the two events around GEMM1 (each
 * event costs a few microseconds of stream time, which matters for a
 * decode-sized call of about a millisecond).  Events are created once and
 * reused; recording adds no synchronisation.  moe_trace_read waits for the
 * recorded events, writes the summed duration in milliseconds of each stage
 * over all recorded calls into stage_ms[0 .. nstages) (stages a call did not
 * time count as 0) and the number of calls into *calls, then forgets them.
 * At most 4096 calls are kept; later calls are not recorded.  An unknown
 * mode returns MOE_ERR_INVALID_ARG.  Not for use under HIP graph capture. */
typedef enum {
  MOE_STAGE_ROUTE = 0,    /* router, routing index, work map; for E4M3 and MX
                             activations also the token quantisation, which
                             shares the router's launch */
  MOE_STAGE_QUANT = 1,    /* nothing (the token quantisation runs in the
                             route stage; kept so stage indices stay fixed) */
  MOE_STAGE_GEMM1 = 2,    /* grouped GEMM1 + SwiGLU */
  MOE_STAGE_REQUANT = 3,  /* FC2 input (nothing when GEMM1 writes it, fc2_fused) */
  MOE_STAGE_GEMM2 = 4,    /* grouped GEMM2 */
  MOE_STAGE_FINALIZE = 5, /* router-weighted top-k sum */
  MOE_NUM_STAGES = 6
} moe_stage;

enum { MOE_TRACE_OFF = 0, MOE_TRACE_ALL = 1, MOE_TRACE_GEMM1 = 2 };
moe_status moe_trace_enable(int32_t mode);
moe_status moe_trace_read(float* stage_ms, int32_t nstages, int32_t* calls);

#ifdef __cplusplus
}
#endif

#endif /* MOE_AMD_MOE_H_ */
