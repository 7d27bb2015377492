/*
 * bqmm.h -- C ABI of the block-quantized projection matmul library for
 * AMD Instinct MI355X (gfx950).
 *
 * y[m][n] = x[m][k] . W[n][k]^T, the projection matmul of an LLM inference
 * engine, with two weight encodings:
 *   - Q8_0 weights (34-byte blocks: fp16 scale + 32 int8 quants) against
 *     q8_1 activations (int8 + f32 scale per 32 values): each 32-block dot
 *     product is summed in int32 and folded into f32 by the two scales;
 *   - OCP E4M3FN weights with one per-tensor f32 scale against activations
 *     quantized to e4m3 with one per-batch scale amax/448, f32 accumulate.
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is DEVICE memory owned by the caller; the
 *     library allocates nothing, keeps no pointer after returning, and
 *     never synchronizes the host.  All work is enqueued on `stream`
 *     (a hipStream_t; NULL means the default stream), in argument order.
 *   - Output buffers are fully overwritten; they may hold garbage on entry.
 *   - Matrices are row-major and dense, except Q8_0 weight rows, which
 *     start every `w_row_bytes` bytes (padding after k/32*34 bytes is
 *     ignored).
 *   - Return codes: BQM_OK; BQM_EINVAL for a null pointer or a size out of
 *     range; BQM_EUNSUPPORTED for a shape or alignment the kernels do not
 *     handle; BQM_EHIP_BASE + hipError_t when a launch fails.  Argument
 *     checks run before any HIP call, so a rejected call touches neither
 *     the device nor the stream.  After its launches a call reads the
 *     runtime's error state with hipPeekAtLastError(), which leaves the
 *     state in place: a failed launch stays pending for the caller to
 *     clear with hipGetLastError(), and an error the caller left pending
 *     before the call is reported by the call as well (the two cannot be
 *     told apart without consuming the caller's error).
 *   - Calls on one stream run in order; calls on different streams that
 *     write the same buffer race (the library has no internal state).
 *
 * Passages cited are from the memra-engine docs.rs source pages.
 */
#ifndef BQMM_H
#define BQMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BQM_OK 0
#define BQM_EINVAL 1
#define BQM_EUNSUPPORTED 2
#define BQM_EHIP_BASE 10000

/* Largest token count the GEMV takes ("decode_kernel_census.rs" and
 * "fp8_ffi.rs" module doc: decode and the m<=9 verify tier stay on the GEMV;
 * prefill m>=16 moves to the GEMM). */
#define BQM_GEMV_MAX_M 15
/* Largest m the e4m3 decode GEMV accepts. */
#define BQM_E4M3_GEMV_MAX_M 16

/*
 * q8_1 activation quantization, per token and 32-value block
 * ("decode_kernel_census.rs", fn q8: an int8 for every value and two f32
 * numbers for every 32-value block; the int8 rule d = amax/127, q =
 * clamp(round(x/d), -127, 127) with round half away from zero follows
 * "f16_ffi.rs", fn try_f16_gemm, W8A8 arm; "accprobe_bench.rs" module doc:
 * a block's largest magnitude always maps to +-127).
 *
 *   x   : f32 [m][k], 16-byte aligned.
 *   xq  : int8 [m][k] out, 4-byte aligned.
 *   xds : f32 [m][k/32][2] out, 8-byte aligned: (d, s) with d = amax/127
 *         (f32 division) and s = d * sum(q) (the pair's second value; the
 *         Q8_0 kernels never read it).  A block of zeros gives d = s = 0.
 *   m >= 1, k >= 32, k % 32 == 0 (else BQM_EUNSUPPORTED).
 * Bytes are identical to a correctly rounded f32 evaluation of the rule.
 */
int bqm_q8_1_quantize(const float *x, int8_t *xq, float *xds, int m, int k, void *stream);

/*
 * Q8_0 decode/verify GEMV, 1 <= m <= 15
 * ("decode_kernel_census.rs", fn q8: Q8_0 rows of in_f/32*34 bytes timed at
 * m=1; "fp8_ffi.rs" module doc: m<16 stays on this chain bit for bit and the
 * verify tier is m<=9).
 *
 *   w           : uint8 Q8_0 rows [n][w_row_bytes]; block b of row r is at
 *                 w + r*w_row_bytes + 34*b (fp16 little-endian d_w, then 32
 *                 int8 quants).  16-byte aligned.
 *   w_row_bytes : >= k/32*34 and a multiple of 16.
 *   xq, xds     : q8_1 activations as written by bqm_q8_1_quantize
 *                 (xq 16-byte aligned, xds 8-byte aligned).
 *   y           : f32 [m][n] out, 4-byte aligned.
 *   k % 256 == 0 (16-byte aligned row segments), and the activations must
 *   fit on chip: m*k*9/8 <= 98304 bytes (else BQM_EUNSUPPORTED).
 * y[t][r] = sum_b d_w[r][b] * d_x[t][b] * S[t][r][b], S the int32 block sum;
 * each token's floating-point operation order does not depend on m, so a
 * row of an m-token call is bitwise equal to the same row computed alone
 * ("decode_kernel_census.rs" module doc: identical per-row FP order).
 */
int bqm_q8_0_gemv(const uint8_t *w, int64_t w_row_bytes, const int8_t *xq, const float *xds,
                  float *y, int m, int k, int n, void *stream);

/*
 * The decode step in one launch: bqm_q8_1_quantize of the f32 activation
 * followed by bqm_q8_0_gemv, with the quantization done by every workgroup
 * into its on-chip copy (same rule, same device code), so xq/xds never go
 * through memory.  y is bitwise equal to the two-call path.
 *   w, w_row_bytes, y, k, n : as bqm_q8_0_gemv (k % 256 == 0).
 *   x : f32 activations [m][k], 16-byte aligned.
 *   m : 1 or 2 with m*k <= 8192 (decode); 3 <= m <= 15 or a larger m*k gives
 *       BQM_EUNSUPPORTED (every workgroup quantizes the whole activation,
 *       which only pays while it fits in registers; use the two calls).
 * ("decode_kernel_census.rs" fn q8: the q8_1 activation of the m=1 Q8_0
 * GEMV; the pages run the quantizer as its own step.)
 */
int bqm_q8_0_gemv_f32(const uint8_t *w, int64_t w_row_bytes, const float *x, float *y, int m, int k, int n,
                      void *stream);

/*
 * Q8_0 prefill GEMM (MMQ), any m >= 1, built for m >= 16
 * ("accprobe_bench.rs" module doc: int8 MMA with an s32 accumulator per
 * k32 block folded every k32; "fp8_ffi.rs" module doc: the m>=16 arms).
 * Same arguments, layouts, result and alignment rules as bqm_q8_0_gemv,
 * with no limit on m or on k beyond k % 256 == 0.
 */
int bqm_q8_0_gemm(const uint8_t *w, int64_t w_row_bytes, const int8_t *xq, const float *xds,
                  float *y, int m, int k, int n, void *stream);

/*
 * The accumulator instrument's f32 arm ("accprobe_bench.rs" page, module
 * doc): bqm_q8_0_gemm with its accumulator as the one free variable.  Same
 * arguments, checks, tiles, loads, launch and fold count; every quant byte
 * (weight and activation) is read as an OCP E4M3FN code and multiplied on the
 * fp8 matrix cores with f32 accumulation:
 *   y[t][r] = sum_b d_w[r][b] * d_x[t][b] * sum_i e4m3(q_w) * e4m3(q_x).
 * Bytes of magnitude 0x7F (e4m3 NaN) give NaN outputs; the instrument's
 * data avoids them.  Its output is compared only with its own definition;
 * the pair (this, bqm_q8_0_gemm) prices the accumulator by time.
 */
int bqm_q8_0_gemm_f8acc(const uint8_t *w, int64_t w_row_bytes, const int8_t *xq, const float *xds,
                        float *y, int m, int k, int n, void *stream);

/*
 * Per-batch e4m3 activation quantization ("fp8_ffi.rs" module doc: the
 * batch shares one e4m3 scale, amax/448, with the amax reduced on the device
 * and the scale multiplied by weight_scale into a device scalar, with no host
 * synchronization; Fp8Scratch doc: the scale block keeps the amax, the
 * quantization multiplier and the folded scale, in that order).
 *
 *   x       : f32 [m][k], 16-byte aligned.
 *   xq      : uint8 [m][k] OCP E4M3FN codes out, 4-byte aligned.
 *   scales  : f32 [4] out, device memory, 4-byte aligned:
 *             [0] amax = max|x| over all m*k values,
 *             [1] mul = 448/amax, [2] folded = (amax/448) * w_scale,
 *             [3] amax/448; all four are 0 when amax == 0.
 *   w_scale : the weight tensor's per-tensor scale, finite (else EINVAL).
 *   m >= 1, k >= 4, k % 4 == 0 (else BQM_EUNSUPPORTED).
 * xq = e4m3(clamp(x * mul, -448, 448)), round to nearest even, sign of
 * zero kept; NaN codes (magnitude 0x7F) are never written.  Two launches on
 * the stream; between them xq holds the partial maxima (it is the only
 * working memory), so it must not alias x or scales.
 */
int bqm_e4m3_quantize_amax(const float *x, uint8_t *xq, float *scales, float w_scale, int m,
                           int k, void *stream);

/*
 * FP8-E4M3 prefill GEMM ("fp8_ffi.rs" module doc and fn try_fp8_gemm: the
 * activation times the transposed e4m3 weight, with the activation scale and
 * weight_scale combined into one device scalar read through a pointer, and
 * f32 accumulation).
 *
 *   w      : uint8 E4M3FN codes [n][k], 16-byte aligned.
 *   xq     : uint8 E4M3FN codes [m][k], 16-byte aligned.
 *   scales : f32 [4] device; only scales[2] is read, on the device.
 *   y      : f32 [m][n] out, 4-byte aligned.
 *   k % 128 == 0 (else BQM_EUNSUPPORTED).  Codes with magnitude 0x7F are
 *   NaN to the matrix cores; callers must not pass them.
 * y[t][r] = scales[2] * sum_k dec(xq[t][k]) * dec(w[r][k]).
 */
int bqm_e4m3_gemm(const uint8_t *w, const uint8_t *xq, const float *scales, float *y, int m,
                  int k, int n, void *stream);

/*
 * The FP8-E4M3 prefill GEMM of bqm_e4m3_gemm ("fp8_ffi.rs" module doc and fn
 * try_fp8_gemm: the same result, y[t][r] = scales[2] * sum_k dec(xq[t][k]) *
 * dec(w[r][k]), f32 accumulation), computed with an error bound that holds
 * for any data: every output is within (27 + k/128) * 2^-24 * T of the exact
 * value, T = |scales[2]| * sum_k |dec(xq[t][k]) * dec(w[r][k])|, i.e. within
 * 1e-5 * T for every accepted k.  bqm_e4m3_gemm runs on the fp8 matrix
 * cores, whose summation cuts products 13 bits below the largest of each
 * 8-byte group (worst case about 8.5e-4 * T); this call converts the codes
 * exactly to fp16 and runs the fp16 matrix cores (24 bits kept per group),
 * summing each 128-k stage into a fresh partial, at roughly half the speed.
 *
 *   Arguments, layouts, alignment and NaN-code rule as bqm_e4m3_gemm.
 *   k % 128 == 0 and k <= 16384 (else BQM_EUNSUPPORTED).
 */
int bqm_e4m3_gemm_exact(const uint8_t *w, const uint8_t *xq, const float *scales, float *y, int m,
                        int k, int n, void *stream);

/*
 * e4m3 decode GEMV on raw e4m3 weights with a per-tensor scale ("fp8_ffi.rs"
 * st_e4m3_enabled doc: decode reads the checkpoint's own e4m3 bytes through
 * qmatvec_e4m3_mmvq, for the per-tensor scalar-scale class).  The pages do
 * not give that kernel's activation format; here the activation is the f32
 * values themselves.
 *
 *   w       : uint8 E4M3FN codes [n][k] (row-major, k bytes per row),
 *             16-byte aligned.
 *   x       : f32 [m][k] activations, 16-byte aligned.
 *   w_scale : the per-tensor f32 weight scale (a host value).
 *   y       : f32 [m][n] out, 4-byte aligned, fully overwritten.
 *   1 <= m <= BQM_E4M3_GEMV_MAX_M, n >= 1, k >= 256, w_scale finite (else
 *   BQM_EINVAL);
 *   k % 256 == 0 and k <= 8192 (else BQM_EUNSUPPORTED).  Codes with magnitude
 *   0x7F are NaN; callers must not pass them.
 * y[t][r] = w_scale * sum_k x[t][k] * dec(w[r][k]), f32 accumulation.  A
 * token's result does not depend on m or on the other tokens: decode (m = 1)
 * and a verify batch give the same bits.
 */
int bqm_e4m3_gemv(const uint8_t *w, const float *x, float w_scale, float *y, int m, int k, int n,
                  void *stream);

/*
 * fp16 mirror prefill path ("f16_ffi.rs" page, module doc and the
 * memra_q8_0_dequant_f16 / memra_f16_cvt / memra_f16_pp_gemm_pre
 * declarations): a resident fp16 copy of a Q8_0 projection, made once, an
 * f32 -> fp16 activation cast, and an fp16 GEMM with f32 accumulation and
 * f32 output.  Rounding enters only at the two casts (IEEE round to nearest
 * even, overflow to infinity, subnormals kept).
 *
 * bqm_q8_0_dequant_f16: w16[r][32b+i] = fp16(d * q) of block b of row r.
 *   w          : Q8_0 rows [n][w_row_bytes], 4-byte aligned, w_row_bytes % 4
 *                == 0 and >= k/32*34.
 *   w16        : fp16 [n][k] out (row-major), 16-byte aligned.
 *   k >= 64, n >= 1 (else BQM_EINVAL); k % 64 == 0 (else BQM_EUNSUPPORTED).
 */
int bqm_q8_0_dequant_f16(const uint8_t *w, int64_t w_row_bytes, uint16_t *w16, int k, int n,
                         void *stream);

/*
 * bqm_f16_cvt: x16[i] = fp16(x[i]) for count values.
 *   x : f32 [count], 16-byte aligned;  x16 : fp16 [count] out, 8-byte aligned.
 *   count >= 1 (else BQM_EINVAL).
 */
int bqm_f16_cvt(const float *x, uint16_t *x16, int64_t count, void *stream);

/*
 * bqm_f16_gemm: y[t][r] = sum_k x16[t][k] * w16[r][k], f32 accumulation.
 *   w16 : fp16 [n][k], 16-byte aligned;  x16 : fp16 [m][k], 16-byte aligned;
 *   y   : f32 [m][n] out, 4-byte aligned, fully overwritten.
 *   m, n >= 1, k >= 64 (else BQM_EINVAL); k % 64 == 0 (else BQM_EUNSUPPORTED).
 */
int bqm_f16_gemm(const uint16_t *w16, const uint16_t *x16, float *y, int m, int k, int n,
                 void *stream);

/*
 * Block-128 FP8 prefill path ("fp8_ffi.rs" page, memra-engine 0.70.0, the
 * per-block FP8 MMQ section: try_fp8_blk_mmq, fp8_mmq_enabled and
 * FP8_MMQ_NAN_OK docs).  The weight is the checkpoint's e4m3 codes with a
 * row-major f32 grid of one scale per 128x128 block and no per-tensor scale;
 * the kernel applies the scales once per 128 values of k ("accprobe_bench.rs"
 * module doc).
 *
 * bqm_e4m3_nan_count: *nan_count = number of bytes of w[0..count) whose low
 * 7 bits are all ones (the e4m3 NaN codes 0x7F / 0xFF, which the matrix cores
 * read as NaN), meant to run once per weight tensor; a tensor with any must
 * not go through bqm_e4m3_blk_gemm.
 *   w         : bytes, 16-byte aligned;  count >= 1 (else BQM_EINVAL).
 *   nan_count : one device uint64, 8-byte aligned, overwritten (zeroed by a
 *               kernel on the stream, then accumulated).
 */
int bqm_e4m3_nan_count(const uint8_t *w, int64_t count, unsigned long long *nan_count, void *stream);

/*
 * bqm_e4m3_blk_quantize: per (token t, 128-k block kb) e4m3 quantization of
 * the f32 activation with the pages' activation rule amax/448:
 *   amax = max |x[t][128kb .. min(128kb+128, k)-1]| (the last block of a row
 *   is short when k % 128 != 0); mul = 448/amax, xs = amax/448 (f32
 *   divisions; both 0 when amax is 0); xq = e4m3(clamp(x * mul, +-448)),
 *   round to nearest even, sign of zero kept, NaN codes never produced.
 *   x  : f32 [m][k], 16-byte aligned.      xq : uint8 [m][k] out, 4-byte aligned.
 *   xs : f32 [m][ceil(k/128)] out, 4-byte aligned.
 *   m >= 1, k >= 16 (else BQM_EINVAL); k % 16 == 0 (else BQM_EUNSUPPORTED):
 *   the pages' gate for this kernel class ("fp8_ffi.rs", try_fp8_blk_mmq:
 *   in_f a multiple of 16, grid blocks counted by div_ceil(128)).
 * The pages do not show this kernel's activation side; this is the reading
 * that gives one fold per 128-k block on both operands.
 */
int bqm_e4m3_blk_quantize(const float *x, uint8_t *xq, float *xs, int m, int k, void *stream);

/*
 * bqm_e4m3_blk_gemm: y[t][r] = sum_kb grid[r/128][kb] * xs[t][kb] *
 *   sum_{i in kb} e4m3(xq[t][i]) * e4m3(w[r][i]), f32 accumulation, one fold
 *   per 128-k block.
 *   w    : e4m3 codes [n][k], 16-byte aligned, free of NaN codes.
 *   grid : f32 [ceil(n/128)][ceil(k/128)] row-major, 4-byte aligned.
 *   xq   : e4m3 codes [m][k], 16-byte aligned;  xs : f32 [m][ceil(k/128)].
 *   y    : f32 [m][n] out, fully overwritten.
 *   m, n >= 1, k >= 16 (else BQM_EINVAL); k % 16 == 0 (else BQM_EUNSUPPORTED);
 *   the last 128-k block is short when k % 128 != 0.
 */
int bqm_e4m3_blk_gemm(const uint8_t *w, const float *grid, const uint8_t *xq, const float *xs, float *y, int m,
                      int k, int n, void *stream);

/* Text for a return code; never NULL, static storage. */
const char *bqm_strerror(int rc);

#ifdef __cplusplus
}
#endif

#endif /* BQMM_H */
