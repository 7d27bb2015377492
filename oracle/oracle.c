/*
 * Plain CPU oracle for the block-quantized projection matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this code: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no source, header, table or helper with the
 * HIP library; both sides read the same seeded input bytes and nothing else.
 *
 * Deliberately slow and literal: every function follows the definition in
 * the order the pages state it, with no blocking, fusion or reordering.
 * Built with -O2 -fno-fast-math -ffp-contract=off so every float operation
 * is the one written (no fused multiply-add, no reassociation).
 *
 * Sources (memra-engine docs.rs source pages):
 *  - Q8_0 weight block = fp16 scale + 32 int8 quants, 34 bytes; a row is
 *    in_f/32 blocks: "decode_kernel_census.rs" (0.113.0), fn q8;
 *    "accprobe_bench.rs" (0.124.1), fn synth_w_q8_0.
 *  - q8_1 activation: an int8 quant for every value and two f32 numbers
 *    for every 32-value block: "decode_kernel_census.rs", fn q8.
 *  - int8 quantization d = amax/127, q = clamp(round(v/d), -127, 127) with
 *    Rust's round (half away from zero): "f16_ffi.rs" (0.81.0), fn
 *    try_f16_gemm (the W8A8 simulation arm); the value with the largest
 *    magnitude in a block always becomes +127 or -127: "accprobe_bench.rs",
 *    module doc.
 *  - s32 accumulate per 32-block, folded into f32 by the two scales:
 *    "accprobe_bench.rs", module doc (the floor folds every k32).
 *  - e4m3: 0x7F magnitude is NaN ("accprobe_bench.rs" module doc;
 *    "fp8_ffi.rs" (0.70.0), FP8_MMQ_NAN_OK doc), codes 0x01-0x07 are
 *    denormals ("accprobe_bench.rs", fn synth_w_q8_0 doc); activation scale
 *    amax/448 per batch, one scalar, folded with weight_scale into a device
 *    scalar read by the GEMM; the device scale block holds the amax, then the
 *    quantization multiplier, then the folded scale ("fp8_ffi.rs", module
 *    doc and Fp8Scratch doc).
 *
 * Readings where the pages are silent are listed beside each function.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define QK 32
#define Q8_0_BYTES 34

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* IEEE 754 binary16 -> binary32, exact (normals, subnormals, inf, NaN). */
float oracle_fp16_to_f32(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    float v;
    if (e == 0)
        v = ldexpf((float)f, -24);               /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexpf((float)(1024 + f), e - 25);   /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* Round half away from zero (Rust's f32::round), written out. */
static float round_half_away(float v) {
    float a = fabsf(v);
    float fl = floorf(a);
    float r = (a - fl >= 0.5f) ? fl + 1.0f : fl;
    return v < 0.0f ? -r : r;
}

/*
 * q8_1 activation quantization, per (token, 32-block):
 *   amax = max |x_i|;  d = amax / 127 (f32 division);
 *   q_i = clamp(round_half_away(x_i / d), -127, 127) (f32 division);
 *   s = d * (float)sum(q_i)  -- the second value of the scale pair.
 * Readings: a block whose d is 0 -- amax == 0, or amax so small (below
 * 127 * 2^-150) that amax/127 underflows to 0 -- gives q = 0 and s = 0 (the
 * W8A8 arm leaves an all-zero row untouched; dividing by d = 0 has no int8
 * meaning); the second pair value is d times the quant sum (the pages only
 * say "a pair", the Q8_0 path never reads it).
 * xds layout: [m][k/32][2] = (d, s).
 */
void oracle_q8_1_quantize(const float *x, int8_t *xq, float *xds, int64_t m, int64_t k) {
    int64_t nb = k / QK;
    for (int64_t t = 0; t < m; t++) {
        for (int64_t b = 0; b < nb; b++) {
            const float *blk = x + t * k + b * QK;
            int8_t *q = xq + t * k + b * QK;
            float amax = 0.0f;
            for (int i = 0; i < QK; i++) {
                float a = fabsf(blk[i]);
                if (a > amax) amax = a;
            }
            float d = amax / 127.0f;
            int sum = 0;
            for (int i = 0; i < QK; i++) {
                float r = 0.0f;
                if (d > 0.0f) {
                    r = round_half_away(blk[i] / d);
                    if (r > 127.0f) r = 127.0f;
                    if (r < -127.0f) r = -127.0f;
                }
                q[i] = (int8_t)r;
                sum += (int)r;
            }
            xds[2 * (t * nb + b) + 0] = d;
            xds[2 * (t * nb + b) + 1] = d * (float)sum;
        }
    }
}

/* Weight block accessors: scale in bytes 0..1 (little-endian fp16), quants in 2..33. */
static float q8_0_scale(const uint8_t *blk) {
    return oracle_fp16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)));
}

/*
 * Integer block sums S[t][n][b] = sum_i q_w[n][b][i] * q_x[t][b][i] (int32).
 */
void oracle_q8_0_block_sums(const uint8_t *w, int64_t row_bytes, const int8_t *xq,
                            int64_t m, int64_t k, int64_t n, int32_t *S) {
    int64_t nb = k / QK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; r++) {
        for (int64_t t = 0; t < m; t++) {
            for (int64_t b = 0; b < nb; b++) {
                const uint8_t *blk = w + r * row_bytes + b * Q8_0_BYTES;
                int32_t s = 0;
                for (int i = 0; i < QK; i++)
                    s += (int32_t)(int8_t)blk[2 + i] * (int32_t)xq[t * k + b * QK + i];
                S[(t * n + r) * nb + b] = s;
            }
        }
    }
}

/* One output element: y = sum_b d_w * d_x * S_b in fp64; T = sum_b |d_w * d_x * S_b|. */
static void q8_0_dot(const uint8_t *wrow, const int8_t *xrow, const float *xdsrow, int64_t nb,
                     double *y, double *tabs) {
    double acc = 0.0, aabs = 0.0;
    for (int64_t b = 0; b < nb; b++) {
        const uint8_t *blk = wrow + b * Q8_0_BYTES;
        int32_t s = 0;
        for (int i = 0; i < QK; i++)
            s += (int32_t)(int8_t)blk[2 + i] * (int32_t)xrow[b * QK + i];
        double term = (double)q8_0_scale(blk) * (double)xdsrow[2 * b] * (double)s;
        acc += term;
        aabs += fabs(term);
    }
    *y = acc;
    *tabs = aabs;
}

/*
 * Q8_0 x q8_1 matmul, y[t][n] = sum_b d_w[n][b] * d_x[t][b] * S[t][n][b], in fp64.
 * w: [n] rows of row_bytes bytes (first k/32*34 used); xq [m][k]; xds [m][k/32][2].
 * Outputs y and T = sum of |terms|, both [m][n].
 */
void oracle_q8_0_matmul(const uint8_t *w, int64_t row_bytes, const int8_t *xq, const float *xds,
                        int64_t m, int64_t k, int64_t n, double *y, double *tabs) {
    int64_t nb = k / QK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; r++)
        for (int64_t t = 0; t < m; t++)
            q8_0_dot(w + r * row_bytes, xq + t * k, xds + t * nb * 2, nb,
                     &y[t * n + r], &tabs[t * n + r]);
}

/* Same as oracle_q8_0_matmul for a list of (token, row) pairs only. */
void oracle_q8_0_matmul_sampled(const uint8_t *w, int64_t row_bytes, const int8_t *xq,
                                const float *xds, int64_t k, int64_t npairs,
                                const int64_t *tok, const int64_t *row, double *y, double *tabs) {
    int64_t nb = k / QK;
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < npairs; p++)
        q8_0_dot(w + row[p] * row_bytes, xq + tok[p] * k, xds + tok[p] * nb * 2, nb,
                 &y[p], &tabs[p]);
}

/*
 * OCP E4M3FN decode: sign | 4-bit exponent (bias 7) | 3-bit mantissa.
 * Exponent field 0 is subnormal (m * 2^-9); magnitude 0x7F is NaN; no infinity.
 */
float oracle_e4m3_decode(uint8_t c) {
    int sign = c >> 7;
    int e = (c >> 3) & 15;
    int mant = c & 7;
    float v;
    if ((c & 0x7F) == 0x7F)
        return NAN;
    if (e == 0)
        v = ldexpf((float)mant, -9);
    else
        v = ldexpf((float)(8 + mant), e - 10);   /* (1 + m/8) * 2^(e-7) */
    return sign ? -v : v;
}

/*
 * f32 -> E4M3FN: clamp to [-448, 448], then round to the nearest representable
 * magnitude, ties to the even code (even mantissa), searching every finite
 * non-negative code.  The sign of x is kept, so -0 and negative values that
 * round to zero give 0x80.  NaN codes are never produced.
 * Readings: saturation (clamp before rounding) and round-to-nearest-even are
 * the plainest reading; the pages fix only the amax/448 scale and the NaN code.
 */
uint8_t oracle_e4m3_encode(float x) {
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    float a = fabsf(x);
    if (a > 448.0f) a = 448.0f;
    uint8_t best = 0;
    double best_d = INFINITY;
    for (int c = 0; c <= 0x7E; c++) {
        double d = fabs((double)oracle_e4m3_decode((uint8_t)c) - (double)a);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best_d = d;
            best = (uint8_t)c;
        }
    }
    return sign | best;
}

void oracle_e4m3_encode_array(const float *x, uint8_t *out, int64_t count) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; i++) out[i] = oracle_e4m3_encode(x[i]);
}

/*
 * Per-batch e4m3 activation quantization:
 *   amax = max |x| over all m*k values;
 *   mul = 448 / amax, x_scale = amax / 448 (f32; both 0 when amax == 0);
 *   folded = x_scale * w_scale (f32);
 *   xq = encode(x * mul) with the product in f32.
 * scales = {amax, mul, folded, x_scale}.
 */
void oracle_e4m3_quantize_amax(const float *x, uint8_t *xq, float *scales, float w_scale,
                               int64_t m, int64_t k) {
    int64_t count = m * k;
    float amax = 0.0f;
    for (int64_t i = 0; i < count; i++) {
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    float mul = 0.0f, xs = 0.0f;
    if (amax > 0.0f) {
        mul = 448.0f / amax;
        xs = amax / 448.0f;
    }
    float folded = xs * w_scale;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; i++) {
        float v = x[i] * mul;
        xq[i] = oracle_e4m3_encode(v);
    }
    scales[0] = amax;
    scales[1] = mul;
    scales[2] = folded;
    scales[3] = xs;
}

/* Decode table for the 256 codes, filled from oracle_e4m3_decode before use. */
static double e4m3_table[256];

static void e4m3_fill_table(void) {
    for (int c = 0; c < 256; c++) e4m3_table[c] = (double)oracle_e4m3_decode((uint8_t)c);
}

static void e4m3_dot(const uint8_t *wrow, const uint8_t *xrow, int64_t k, double folded,
                     double *y, double *tabs) {
    double acc = 0.0, aabs = 0.0;
    for (int64_t i = 0; i < k; i++) {
        double p = e4m3_table[xrow[i]] * e4m3_table[wrow[i]];
        acc += p;
        aabs += fabs(p);
    }
    *y = folded * acc;
    *tabs = fabs(folded) * aabs;
}

/*
 * e4m3 GEMM: y[t][n] = scales[2] * sum_k dec(xq[t][k]) * dec(w[n][k]), fp64.
 * The fp64 sum of e4m3 products is exact at these sizes.
 */
void oracle_e4m3_matmul(const uint8_t *w, const uint8_t *xq, const float *scales,
                        int64_t m, int64_t k, int64_t n, double *y, double *tabs) {
    double folded = (double)scales[2];
    e4m3_fill_table();
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; r++)
        for (int64_t t = 0; t < m; t++)
            e4m3_dot(w + r * k, xq + t * k, k, folded, &y[t * n + r], &tabs[t * n + r]);
}

void oracle_e4m3_matmul_sampled(const uint8_t *w, const uint8_t *xq, const float *scales,
                                int64_t k, int64_t npairs, const int64_t *tok,
                                const int64_t *row, double *y, double *tabs) {
    double folded = (double)scales[2];
    e4m3_fill_table();
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < npairs; p++)
        e4m3_dot(w + row[p] * k, xq + tok[p] * k, k, folded, &y[p], &tabs[p]);
}

/*
 * e4m3 decode GEMV on raw e4m3 weights with a per-tensor scale:
 * y[t][n] = w_scale * sum_k x[t][k] * dec(w[n][k]), the activation used as
 * the f32 values it is (the pages name the decode kernel, qmatvec_e4m3_mmvq,
 * and its per-tensor scalar-scale weight class, "fp8_ffi.rs" st_e4m3_enabled
 * doc, but not its activation format; the plainest reading is the f32
 * activation against the decoded weights).  Accumulated in fp64, so the
 * result is within ~1e-12 relative of the exact sum; tabs is the fp64
 * sum of |terms| times |w_scale|.
 */
static void e4m3_gemv_dot(const uint8_t *wrow, const float *xrow, int64_t k, double ws, double *y,
                          double *tabs) {
    double acc = 0.0, aabs = 0.0;
    for (int64_t i = 0; i < k; i++) {
        double p = (double)xrow[i] * e4m3_table[wrow[i]];
        acc += p;
        aabs += fabs(p);
    }
    *y = ws * acc;
    *tabs = fabs(ws) * aabs;
}

void oracle_e4m3_gemv(const uint8_t *w, const float *x, float w_scale, int64_t m, int64_t k, int64_t n,
                      double *y, double *tabs) {
    e4m3_fill_table();
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; r++)
        for (int64_t t = 0; t < m; t++)
            e4m3_gemv_dot(w + r * k, x + t * k, k, (double)w_scale, &y[t * n + r], &tabs[t * n + r]);
}

void oracle_e4m3_gemv_sampled(const uint8_t *w, const float *x, float w_scale, int64_t k, int64_t npairs,
                              const int64_t *tok, const int64_t *row, double *y, double *tabs) {
    e4m3_fill_table();
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < npairs; p++)
        e4m3_gemv_dot(w + row[p] * k, x + tok[p] * k, k, (double)w_scale, &y[p], &tabs[p]);
}

/*
 * fp16 mirror of the Q8_0 weights and the fp16 prefill GEMM ("f16_ffi.rs"
 * page, memra-engine 0.81.0, module doc and the memra_q8_0_dequant_f16 /
 * memra_f16_cvt / memra_f16_pp_gemm_pre declarations): the int8 quants are
 * exact in fp16, rounding enters only at the d*q product's cast to fp16 and at
 * the activation's f32 -> fp16 cast; the GEMM accumulates in f32 and writes
 * f32.  Both casts are read as IEEE round-to-nearest-even with overflow to
 * infinity and subnormals kept (the pages do not say; the plainest reading of
 * a cast).
 */
uint16_t oracle_f32_to_f16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t exp = (u >> 23) & 0xFFu, man = u & 0x7FFFFFu;
    if (exp == 0xFFu) return (uint16_t)(sign | 0x7C00u | (man ? 0x200u : 0u));   /* inf, NaN */
    /* value = 1.man * 2^(exp-127) for normal f32 (f32 subnormals are far below fp16's range) */
    int e = (int)exp - 127;
    if (exp == 0) return sign;                         /* f32 zero or subnormal: rounds to zero */
    uint32_t sig = man | 0x800000u;                    /* 24-bit significand, value = sig * 2^(e-23) */
    /* target: integer multiple of the fp16 quantum at this exponent */
    int q = e >= -14 ? e - 10 : -24;                   /* quantum exponent: 2^q (normal: 11 bits; subnormal: 2^-24) */
    int shift = q - (e - 23);                          /* bits of sig below the quantum */
    uint32_t mant;
    if (shift >= 32) {
        mant = 0;
    } else if (shift <= 0) {
        mant = sig << (-shift);
    } else {
        uint32_t keep = sig >> shift, rem = sig & ((1u << shift) - 1u), half = 1u << (shift - 1);
        mant = keep + ((rem > half || (rem == half && (keep & 1u))) ? 1u : 0u);
    }
    /* mant * 2^q; renormalize */
    if (mant == 0) return sign;
    int E;
    if (q == -24) {
        if (mant < 1024u) return (uint16_t)(sign | mant);            /* subnormal */
        E = -14;                                                      /* rounded up into the normals */
        mant >>= 0;
        if (mant >= 2048u) { mant >>= 1; E += 1; }
    } else {
        E = e;
        if (mant >= 2048u) { mant >>= 1; E += 1; }                    /* carry out of the significand */
    }
    if (E > 15) return (uint16_t)(sign | 0x7C00u);                    /* overflow to infinity */
    return (uint16_t)(sign | ((uint32_t)(E + 15) << 10) | (mant & 0x3FFu));
}

void oracle_f32_to_f16_array(const float *x, uint16_t *out, int64_t count) {
    for (int64_t i = 0; i < count; i++) out[i] = oracle_f32_to_f16(x[i]);
}

/* Q8_0 rows -> row-major fp16: w16[r][32b+i] = fp16(d * q), d*q exact in f32. */
void oracle_q8_0_dequant_f16(const uint8_t *w, int64_t row_bytes, uint16_t *w16, int64_t k, int64_t n) {
    const int64_t nb = k / 32;
    for (int64_t r = 0; r < n; r++)
        for (int64_t b = 0; b < nb; b++) {
            const uint8_t *blk = w + r * row_bytes + b * 34;
            const float d = q8_0_scale(blk);
            for (int i = 0; i < 32; i++) {
                const float v = d * (float)(int8_t)blk[2 + i];
                w16[r * k + b * 32 + i] = oracle_f32_to_f16(v);
            }
        }
}

static double f16_value(uint16_t h) { return (double)oracle_fp16_to_f32(h); }

static void f16_dot(const uint16_t *wrow, const uint16_t *xrow, int64_t k, double *y, double *tabs) {
    double acc = 0.0, aabs = 0.0;
    for (int64_t i = 0; i < k; i++) {
        double p = f16_value(xrow[i]) * f16_value(wrow[i]);
        acc += p;
        aabs += fabs(p);
    }
    *y = acc;
    *tabs = aabs;
}

/* y[t][r] = sum_k x16[t][k] * w16[r][k] in fp64 (products of two fp16 are exact). */
void oracle_f16_gemm(const uint16_t *w16, const uint16_t *x16, int64_t m, int64_t k, int64_t n, double *y,
                     double *tabs) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; r++)
        for (int64_t t = 0; t < m; t++) f16_dot(w16 + r * k, x16 + t * k, k, &y[t * n + r], &tabs[t * n + r]);
}

/*
 * The accumulator instrument's f32 arm ("accprobe_bench.rs" page, memra-engine
 * 0.124.1, module doc): the Q8_0 MMQ with the int8 MMA swapped for an e4m3 x
 * e4m3 MMA that accumulates in f32, on the same bytes, with the same fold by
 * the two block scales every 32 values.  Every quant byte, weight and
 * activation, is read as an OCP E4M3FN code instead of an int8:
 *   y[t][n] = sum_b d_w[n][b] * d_x[t][b] * sum_i dec(q_w[n][b][i]) * dec(q_x[t][b][i])
 * in fp64 (the block sum of e4m3 products is exact; each block term carries
 * one fp64 rounding).  tabs = sum_b |d_w d_x| * sum_i |dec * dec|, the sum of
 * the magnitudes of every product term.  The instrument's bytes avoid the NaN
 * codes (magnitudes <= 126, module doc), so every term is finite.
 */
static void q8_0_e4m3_dot(const uint8_t *wrow, const uint8_t *xrow, const float *xdsrow, int64_t nb,
                          double *y, double *tabs) {
    double acc = 0.0, aabs = 0.0;
    for (int64_t b = 0; b < nb; b++) {
        const uint8_t *blk = wrow + b * Q8_0_BYTES;
        double s = 0.0, sabs = 0.0;
        for (int i = 0; i < QK; i++) {
            double p = e4m3_table[blk[2 + i]] * e4m3_table[xrow[b * QK + i]];
            s += p;
            sabs += fabs(p);
        }
        double scale = (double)q8_0_scale(blk) * (double)xdsrow[2 * b];
        acc += scale * s;
        aabs += fabs(scale) * sabs;
    }
    *y = acc;
    *tabs = aabs;
}

void oracle_q8_0_matmul_e4m3(const uint8_t *w, int64_t row_bytes, const uint8_t *xq, const float *xds,
                             int64_t m, int64_t k, int64_t n, double *y, double *tabs) {
    int64_t nb = k / QK;
    e4m3_fill_table();
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; r++)
        for (int64_t t = 0; t < m; t++)
            q8_0_e4m3_dot(w + r * row_bytes, xq + t * k, xds + t * nb * 2, nb, &y[t * n + r], &tabs[t * n + r]);
}

/*
 * Block-128 FP8 operands ("fp8_ffi.rs" page, memra-engine 0.70.0, the
 * per-block FP8 MMQ section: try_fp8_blk_mmq, fp8_mmq_enabled and the
 * FP8_MMQ_NAN_OK docs; "accprobe_bench.rs" module doc: the per-block kernel
 * sums the four k32 steps of a 128-k block in one accumulator and applies
 * the block's scales a single time).  The weight is e4m3 codes [n][k] with a row-major f32 grid
 * [ceil(n/128)][ceil(k/128)], one scale per 128x128 block, and a per-tensor
 * scale of 1.  Magnitude 0x7F is NaN to the hardware, so a weight holding
 * one is refused after a one-time count.
 *
 * The pages do not show the activation side of this kernel.  Reading: the
 * f32 activation is quantized to e4m3 per (token, 128-k block) with the
 * pages' activation rule, scale amax/448 and multiplier 448/amax (f32
 * divisions), values scaled in f32, clamped to +-448, rounded to nearest
 * even; a block whose amax is 0 gets multiplier and scale 0.  A trailing
 * block shorter than 128 (k % 128 != 0) is quantized over the values it has.
 */
uint64_t oracle_e4m3_nan_count(const uint8_t *b, int64_t count) {
    uint64_t c = 0;
    for (int64_t i = 0; i < count; i++)
        if ((b[i] & 0x7F) == 0x7F) c++;
    return c;
}

/* xq [m][k] codes, xs [m][ceil(k/128)] scales amax/448. */
void oracle_e4m3_blk_quantize(const float *x, int64_t m, int64_t k, uint8_t *xq, float *xs) {
    int64_t kbn = (k + 127) / 128;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < m; t++) {
        for (int64_t kb = 0; kb < kbn; kb++) {
            int64_t k0 = kb * 128, k1 = k0 + 128 < k ? k0 + 128 : k;
            float amax = 0.0f;
            for (int64_t i = k0; i < k1; i++) {
                float a = fabsf(x[t * k + i]);
                if (a > amax) amax = a;
            }
            float mul = 0.0f, s = 0.0f;
            if (amax > 0.0f) {
                mul = 448.0f / amax;
                s = amax / 448.0f;
            }
            for (int64_t i = k0; i < k1; i++) xq[t * k + i] = oracle_e4m3_encode(x[t * k + i] * mul);
            xs[t * kbn + kb] = s;
        }
    }
}

/*
 * y[t][r] = sum_kb grid[r/128][kb] * xs[t][kb] * sum_{i in kb} dec(xq[t][i]) * dec(w[r][i]),
 * fp64: each block's e4m3 product sum is exact, then one fp64 rounding per
 * block term.  tabs = sum_kb |grid * xs| * sum_i |dec * dec|.
 */
static void e4m3_blk_dot(const uint8_t *wrow, const float *grow, const uint8_t *xrow, const float *xsrow,
                         int64_t k, double *y, double *tabs) {
    int64_t kbn = (k + 127) / 128;
    double acc = 0.0, aabs = 0.0;
    for (int64_t kb = 0; kb < kbn; kb++) {
        int64_t k0 = kb * 128, k1 = k0 + 128 < k ? k0 + 128 : k;
        double s = 0.0, sabs = 0.0;
        for (int64_t i = k0; i < k1; i++) {
            double p = e4m3_table[xrow[i]] * e4m3_table[wrow[i]];
            s += p;
            sabs += fabs(p);
        }
        double scale = (double)grow[kb] * (double)xsrow[kb];
        acc += scale * s;
        aabs += fabs(scale) * sabs;
    }
    *y = acc;
    *tabs = aabs;
}

void oracle_e4m3_blk_matmul(const uint8_t *w, const float *grid, const uint8_t *xq, const float *xs, int64_t m,
                            int64_t k, int64_t n, double *y, double *tabs) {
    int64_t kbn = (k + 127) / 128;
    e4m3_fill_table();
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; r++)
        for (int64_t t = 0; t < m; t++)
            e4m3_blk_dot(w + r * k, grid + (r / 128) * kbn, xq + t * k, xs + t * kbn, k, &y[t * n + r],
                         &tabs[t * n + r]);
}

void oracle_e4m3_blk_matmul_sampled(const uint8_t *w, const float *grid, const uint8_t *xq, const float *xs,
                                    int64_t k, int64_t npairs, const int64_t *tok, const int64_t *row, double *y,
                                    double *tabs) {
    int64_t kbn = (k + 127) / 128;
    e4m3_fill_table();
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < npairs; p++)
        e4m3_blk_dot(w + row[p] * k, grid + (row[p] / 128) * kbn, xq + tok[p] * k, xs + tok[p] * kbn, k, &y[p],
                     &tabs[p]);
}
