/*
 * mxq.h -- C ABI of libmxq: block-scaled microscaling quantization and the
 * MXFP4 grouped GEMM, hand-written HIP for gfx950 (MI355X).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every data pointer is DEVICE memory owned by the caller.  The library
 *    never allocates or frees device memory and never synchronizes; each
 *    call enqueues its kernels on `stream` (a hipStream_t passed as void*;
 *    NULL = the null stream) and returns immediately.  The one exception is
 *    the debug check mxq_validate_offs, which copies into host memory of its
 *    own and waits for the stream.
 *  - Tensors are dense and row-major; leading dimensions are flattened into
 *    `rows` by the caller.  Any alignment is accepted (misaligned or oddly
 *    shaped tensors take a slower general kernel).
 *  - Zero-sized problems return MXQ_OK without launching anything.
 *  - Arguments are validated on the host before any HIP call; a failed check
 *    returns a negative mxq_status and enqueues nothing.  A launch failure
 *    returns MXQ_ERR_HIP.  Nothing is ever thrown across the ABI.
 *  - Values must be finite where the operation takes an amax (NaN/Inf inputs
 *    are outside the method's domain; the result for such a block is
 *    unspecified but the call is memory-safe).
 *
 * Sources (page title, then the section on it):
 *   [MX]  "nemo_automodel.components.quantization.mxfp4" (NeMo AutoModel API)
 *   [QC]  "nemo_automodel.components.models.deepseek_v41.quantization"
 *   [MO]  "NVIDIA Model Optimizer: from mtq.quantize to a 4.95-bit
 *          DeepSeek-R1", section "NVFP4 in the code: two scales and a nibble"
 */
#ifndef MXQ_H
#define MXQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MXQ_OK = 0,
  MXQ_ERR_NULL = -1,    /* a required pointer is NULL                          */
  MXQ_ERR_SHAPE = -2,   /* negative size, K % 32 != 0, or inconsistent sizes    */
  MXQ_ERR_DTYPE = -3,   /* dtype code not supported by this entry point        */
  MXQ_ERR_FORMAT = -4,  /* format code not one of mxq_format                   */
  MXQ_ERR_BLOCK = -5,   /* block_size <= 0 (or odd for packed fp4 storage)     */
  MXQ_ERR_ALIGN = -6,   /* grouped GEMM activation / packed weights / output not 16-B aligned */
  MXQ_ERR_ALIAS = -7,   /* output overlaps an input that must stay unmodified  */
  MXQ_ERR_HIP = -8,     /* a HIP launch reported an error                      */
  MXQ_ERR_OFFS = -9     /* mxq_validate_offs: offs breaks its precondition     */
} mxq_status;

typedef enum { MXQ_F32 = 0, MXQ_BF16 = 1, MXQ_F16 = 2 } mxq_dtype;
typedef enum { MXQ_FMT_FP8 = 0, MXQ_FMT_MXFP4 = 1, MXQ_FMT_NVFP4 = 2 } mxq_format;

/*
 * quantize_mxfp4 -- [MX] quantize_mxfp4.
 * Quantizes x [rows, k] (dtype xt: f32, bf16 or f16) along its last dim in
 * blocks of 32 columns ([MX] MXFP4_BLOCK_SIZE).  Per block: amax = max |x|;
 * scale exponent e = floor(log2(amax)) - 2, exact, clamped to [-127, 127],
 * with e = -127 for an all-zero block; every element is rounded to the e2m1
 * grid {0, .5, 1, 1.5, 2, 3, 4, 6} by the midpoints of [MX] _FP4_E2M1_MIDPOINTS,
 * ties to the even grid value ([MO]), saturating at 6; the sign bit is set for
 * x < 0.
 * Outputs: packed [rows, k/2] (two codes per byte, even column in the low
 * nibble, [MX] module docstring) and scales [rows, k/32] (E8M0 bytes e + 127).
 * Errors: MXQ_ERR_NULL, MXQ_ERR_SHAPE (rows < 0, k < 0 or k % 32 != 0),
 * MXQ_ERR_DTYPE, MXQ_ERR_ALIAS (outputs overlap x).
 */
int quantize_mxfp4(const void* x, int xt, int64_t rows, int64_t k,
                   int8_t* packed, uint8_t* scales, void* stream);

/*
 * dequantize_mxfp4 -- [MX] dequantize_mxfp4.
 * out[r, j] = TABLE[nibble(packed[r, j/2], j%2)] * 2^(scales[r, j/32] - 127),
 * computed exactly and rounded nearest-even to `ot` (f32, bf16 or f16).
 * TABLE is [MX] _FP4_E2M1_TABLE; code 8 decodes to +0.0.  Scale byte 0xFF
 * decodes to NaN (float8_e8m0fnu); results past the output range become inf.
 * packed [rows, k/2], scales [rows, k/32], out [rows, k].
 * Errors: MXQ_ERR_NULL, MXQ_ERR_SHAPE, MXQ_ERR_DTYPE, MXQ_ERR_ALIAS.
 */
int dequantize_mxfp4(const int8_t* packed, const uint8_t* scales, int64_t rows, int64_t k,
                     void* out, int ot, void* stream);

/*
 * quantize_cache -- [QC] quantize_cache / _CacheQuantization.forward.
 * Fake-quantizes x [rows, channels] (dtype t) into a new tensor out of the
 * same shape and dtype, in groups of `block_size` consecutive channels; a
 * final partial group is treated as zero-padded.  Per group: scale s =
 * power-of-two ceiling of max(fp32(amax / fmax), 2^-126) ([QC]
 * _power_of_two_ceiling), fmax = 6 for mxfp4/nvfp4 and 448 for fp8 ([MO]);
 * nvfp4 clamps s to the E4M3-representable powers 2^-9 .. 2^8.  Each element
 * becomes grid(x / s) * s rounded to t, where grid is the e2m1 cast (as in
 * quantize_mxfp4; code 8 gives +0.0) or nearest-even E4M3 (keeps the sign).
 * x is not modified; out must not overlap x.
 * Errors: MXQ_ERR_NULL, MXQ_ERR_SHAPE, MXQ_ERR_DTYPE, MXQ_ERR_FORMAT,
 * MXQ_ERR_BLOCK, MXQ_ERR_ALIAS.
 */
int quantize_cache(const void* x, void* out, int t, int64_t rows, int64_t channels,
                   int fmt, int32_t block_size, void* stream);

/*
 * quantize_cache_bwd -- [QC] _CacheQuantization.backward (straight-through).
 * grad_in = grad_out, bit for bit, numel elements of dtype t.  When the two
 * pointers are equal nothing is launched.  Partially overlapping buffers are
 * rejected with MXQ_ERR_ALIAS.
 */
int quantize_cache_bwd(const void* grad_out, void* grad_in, int t, int64_t numel, void* stream);

/*
 * quantize_cache_packed -- packed KV-cache storage: the codes and group scales
 * that quantize_cache ([QC] quantize_cache, with the scale rule and element
 * casts described there) rounds through, stored instead of multiplied back.
 * x [rows, channels] of dtype t, whole groups only (channels % block_size ==
 * 0; block_size even for mxfp4/nvfp4).  Writes
 *   codes: mxfp4/nvfp4 uint8 [rows, channels/2], e2m1 codes two per byte, the
 *          even channel in the low nibble, sign bit for x < 0 (-0.0 -> +0);
 *          fp8 uint8 [rows, channels], E4M3 (FN) bytes, sign kept;
 *   scales: uint8 [rows, channels/block_size], the group scale 2^k as an E8M0
 *          byte k + 127 (mxfp4, fp8) or as E4M3 bits (nvfp4, k in -9..8).
 * dequantize_cache_packed of the result equals quantize_cache of x bit for
 * bit.  Fast path: block_size a power of two in [8, 512], x 16-byte aligned,
 * codes 4-byte (fp4) or 8-byte (fp8) aligned; anything else runs one thread
 * per group.  Inputs must be finite.  Buffers are the caller's (device
 * memory); none may overlap.
 * Errors: MXQ_ERR_SHAPE (negative sizes, channels % block_size != 0),
 * MXQ_ERR_DTYPE, MXQ_ERR_FORMAT, MXQ_ERR_BLOCK (block_size <= 0, or odd for
 * the fp4 formats), MXQ_ERR_NULL, MXQ_ERR_ALIAS, MXQ_ERR_HIP.
 */
int quantize_cache_packed(const void* x, int t, int64_t rows, int64_t channels, int fmt, int32_t block_size,
                          uint8_t* codes, uint8_t* scales, void* stream);

/*
 * dequantize_cache_packed -- dequant-on-read of the packed form: out[i] =
 * code value (e2m1 table, code 8 -> +0.0; or E4M3) times the group's scale
 * (2^(b-127) for an E8M0 byte, the E4M3 value for nvfp4; NaN bytes give NaN),
 * rounded nearest-even to t, into out [rows, channels].  Same layouts, checks
 * and errors as quantize_cache_packed (fast path: out 16-byte aligned).
 */
int dequantize_cache_packed(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t channels, int fmt,
                            int32_t block_size, void* out, int t, void* stream);

/*
 * quantize_nvfp4 -- [MO] section "NVFP4 in the code: two scales and a
 * nibble": two-level NVFP4.  x [rows, k] of dtype xt (k % 16 == 0, any
 * alignment; 16-byte aligned x and 4-byte aligned packed take the fast path)
 * -> packed uint8 [rows, k/2] (two e2m1 codes per byte, even column in the
 * low nibble), block_scales uint8 [rows, k/16] (E4M3 bit patterns) and
 * *global_scale (one float in DEVICE memory, 4-byte aligned).  In fp32,
 * rounded nearest-even in this order: g = max|x| / 2688 (6 * 448) over the
 * whole tensor; per block of 16, s_b = E4M3(max|x_b| / fl(6 g)) with a zero
 * ratio set to 1.0 and then clamped to [2^-9, 448]; d_b = fl(s_b g); codes =
 * e2m1(fl(x / d_b)) by the midpoints, ties to the even code, saturating at 6,
 * sign bit for x < 0.  An all-zero tensor gives g = 0, scales 1.0, codes 0.
 * Inputs must be finite.  *global_scale is also the scratch word of the
 * tensor max while the call runs (all launches on `stream`).  rows * k == 0
 * returns MXQ_OK without a launch and leaves *global_scale alone.
 * Errors: MXQ_ERR_SHAPE (k % 16 != 0 or negative sizes), MXQ_ERR_DTYPE,
 * MXQ_ERR_NULL, MXQ_ERR_ALIGN (global_scale), MXQ_ERR_ALIAS (any two of the
 * four buffers overlap), MXQ_ERR_HIP.
 */
int quantize_nvfp4(const void* x, int xt, int64_t rows, int64_t k, uint8_t* packed, uint8_t* block_scales,
                   float* global_scale, void* stream);

/*
 * quantize_nvfp4_mse -- [MO] section "Where the scales come from" (NVFP4's
 * own rules, the `mse` rule): two-level NVFP4 as quantize_nvfp4 (same g,
 * layouts, zero-tensor rule, arguments and errors), except that each block's
 * scale is searched: every positive finite E4M3 value (codes 0x01 .. 0x7E, in
 * that order) is tried as s_b and the first with the least squared error is
 * kept.  The error of a candidate is computed in fp32, each operation rounded
 * nearest-even: d = fl(s_b g), codes of fl(x / d), e_i = x_i -
 * e2m1(code_i) d rounded once (a fused multiply-add), then fl(e_i e_i)
 * summed over i = 0 .. 15 in order, each sum rounded; a candidate whose d
 * underflows to 0 is skipped.  The codes stored
 * are those of fl(x / d) under the chosen scale, so dequantize_nvfp4 reads
 * the result.  One thread per block of 16 (126 candidates each): bound by
 * VALU throughput, not HBM.  Any alignment of x.
 */
int quantize_nvfp4_mse(const void* x, int xt, int64_t rows, int64_t k, uint8_t* packed, uint8_t* block_scales,
                       float* global_scale, void* stream);

/*
 * dequantize_nvfp4 -- the inverse of quantize_nvfp4 ([MO], same section):
 * out[i] = fl(e2m1(code_i) * fl(E4M3(s_b) * g)), rounded nearest-even to ot
 * (code 8 decodes to +0.0; an E4M3 NaN scale gives NaN).  global_scale is a
 * device pointer to g.  Errors as quantize_nvfp4 (out must not overlap the
 * inputs).
 */
int dequantize_nvfp4(const uint8_t* packed, const uint8_t* block_scales, const float* global_scale, int64_t rows,
                     int64_t k, void* out, int ot, void* stream);

/*
 * mxfp4_grouped_mm_fwd -- [MX] MXFP4GroupedMM.forward.
 * x bf16 [tokens, k] grouped contiguously by expert; packed [experts, n, k/2]
 * and scales [experts, n, k/32] (mxfp4 weights W_e [n, k], packed along k);
 * offs int32 [experts] DEVICE array of cumulative token counts: expert e owns
 * rows [offs[e-1], offs[e]) (offs[-1] = 0).  Computes y[rows_e] = x[rows_e] @
 * W_e^T into y bf16 [tokens, n]: weights are dequantized on the fly (never
 * written to memory), products accumulate in fp32, output rounds nearest-even.
 * Rows at or past offs[experts-1] are written as zeros.
 * offs should be non-decreasing with offs[experts-1] <= tokens; this is not
 * checked on the host (it would need a device sync).  The kernels clamp each
 * offset into [clamped previous offset, tokens], so out-of-range offsets never
 * cause an access past x or y; the result is then that of the clamped offsets.
 * x, packed and y must be 16-byte aligned; y must not overlap x.
 * Errors: MXQ_ERR_NULL, MXQ_ERR_SHAPE (negative sizes, k % 32 != 0 or
 * n % 8 != 0), MXQ_ERR_ALIGN, MXQ_ERR_ALIAS, MXQ_ERR_HIP (also when the
 * launch would pass 2^24 output tiles of 128 x 256, a hardware grid limit:
 * about tokens * n > 5.5e11).
 */
int mxfp4_grouped_mm_fwd(const void* x, int64_t tokens, int64_t k,
                         const int8_t* packed, const uint8_t* scales, int64_t experts, int64_t n,
                         const int32_t* offs, void* y, void* stream);

/*
 * mxfp4_grouped_mm_bwd_x -- [MX] MXFP4GroupedMM.backward.
 * grad_out bf16 [tokens, n]; weights and offs as in the forward.  Computes
 * grad_x[rows_e] = grad_out[rows_e] @ W_e into grad_x bf16 [tokens, k], with
 * a fresh on-the-fly dequantization; no weight gradient (frozen base).
 * Rows past offs[experts-1] are written as zeros.  Same preconditions and
 * errors as the forward; also MXQ_ERR_SHAPE when n > 2^22 or one expert's
 * packed weights reach 2 GiB (n * k / 2 >= 2^31), and MXQ_ERR_HIP past 2^23
 * output tiles of 256 x 256 (about tokens * k > 5.5e11).
 */
int mxfp4_grouped_mm_bwd_x(const void* grad_out, int64_t tokens, int64_t n,
                           const int8_t* packed, const uint8_t* scales, int64_t experts, int64_t k,
                           const int32_t* offs, void* grad_x, void* stream);

/*
 * mxq_validate_offs -- debug check of the offs precondition of the grouped
 * GEMM entry points ([MX] MXFP4GroupedMM: offs holds the cumulative token
 * counts of the experts, so it is non-decreasing and ends within the
 * tokens).  The GEMMs do not check offs on the host (that would need a device
 * sync) and clamp it instead; this entry point is for callers who want the
 * violation reported.  It copies offs int32 [experts] (DEVICE) to host memory
 * on `stream` and WAITS for the stream -- the one entry point that
 * synchronizes -- then checks 0 <= offs[0] <= offs[1] <= ... <=
 * offs[experts-1] <= tokens.  *first_bad (may be NULL) receives the first
 * expert index whose offset breaks it, else -1.
 * Returns MXQ_OK, MXQ_ERR_OFFS (violated), MXQ_ERR_NULL (offs NULL with
 * experts > 0), MXQ_ERR_SHAPE (experts or tokens negative, or experts >
 * 2^26), MXQ_ERR_HIP (the copy or the wait failed).  experts == 0 is MXQ_OK
 * without any HIP call.
 */
int mxq_validate_offs(const int32_t* offs, int64_t experts, int64_t tokens, int64_t* first_bad, void* stream);

/*
 * mxfp4_grouped_mm_fwd_w4a4 -- the forward with the activations in MXFP4 too
 * (W4A4; [MO] section "The claims, marked reported": weight-and-activation
 * FP4 is the variant that reaches the FP4 matrix units, where a
 * dequantize-to-BF16 fallback does not).
 * xq int8 [tokens, k/2] and xs E8M0 [tokens, k/32] are the activations as
 * quantize_mxfp4 writes them ([MX] quantize_mxfp4, the floor rule); weights
 * and offs as in mxfp4_grouped_mm_fwd.  Computes y[rows_e] = dq(xq)[rows_e] @
 * dq(W_e)^T into y bf16 [tokens, n] on the block-scaled fp4 MFMA: products
 * of codes and scales are exact, sums run in fp32, the output rounds
 * nearest-even; rows past offs[experts-1] are written as zeros, offsets are
 * clamped as in the forward.  A scale byte 0xFF makes the products it
 * scales NaN.
 * Needs k % 512 == 0 and k < 2^22, n % 8 == 0, one expert's packed weights
 * below 2 GiB (n * k / 2 < 2^31), else MXQ_ERR_SHAPE; xq, xs, packed, scales
 * and y 16-byte aligned, else MXQ_ERR_ALIGN; y must not overlap xq or xs
 * (MXQ_ERR_ALIAS).  MXQ_ERR_HIP past 2^23 output tiles of 256 x 256.
 */
int mxfp4_grouped_mm_fwd_w4a4(const int8_t* xq, const uint8_t* xs, int64_t tokens, int64_t k,
                              const int8_t* packed, const uint8_t* scales, int64_t experts, int64_t n,
                              const int32_t* offs, void* y, void* stream);

/*
 * mxfp4_grouped_mm_fwd_w4a8 -- the forward with the activations in fp8 (W4A8;
 * [MO] section "NVFP4 in the code: two scales and a nibble": activation
 * scales are computed at run time; section "The claims, marked reported"
 * names W4A8 among the weight-and-activation forms).
 * xq uint8 [tokens, k] are E4M3 (FN) codes and xs uint8 [tokens, k/32] their
 * E8M0 block scales, one per 32 consecutive k, as quantize_cache_packed
 * writes them for format fp8 and block_size 32 ([QC] quantize_cache: scale =
 * power-of-two ceiling of amax / 448); weights and offs as in
 * mxfp4_grouped_mm_fwd.  Computes y[rows_e] = dq(xq)[rows_e] @ dq(W_e)^T into
 * y bf16 [tokens, n] on the block-scaled MFMA (fp8 x fp4): products of codes
 * and scales are exact, sums run in fp32, the output rounds nearest-even;
 * rows past offs[experts-1] are written as zeros, offsets are clamped as in
 * the forward.  A scale byte 0xFF, or an E4M3 NaN code, makes the products it
 * scales NaN.
 * Needs k % 512 == 0 and k < 2^22, n % 8 == 0, one expert's packed weights
 * below 2 GiB (n * k / 2 < 2^31), else MXQ_ERR_SHAPE; xq, xs, packed, scales
 * and y 16-byte aligned, else MXQ_ERR_ALIGN; y must not overlap xq or xs
 * (MXQ_ERR_ALIAS).  MXQ_ERR_HIP past 2^23 output tiles of 96 x 256.
 */
int mxfp4_grouped_mm_fwd_w4a8(const uint8_t* xq, const uint8_t* xs, int64_t tokens, int64_t k,
                              const int8_t* packed, const uint8_t* scales, int64_t experts, int64_t n,
                              const int32_t* offs, void* y, void* stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char* mxq_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MXQ_H */
