// FP8-E4M3 prefill path for gfx950: per-batch activation quantization and the
// e4m3 x e4m3 GEMM with f32 accumulation.
//
// From the "fp8_ffi.rs" page (memra-engine 0.70.0), module doc, fn
// try_fp8_gemm and the Fp8Scratch doc: the activation is quantized f32 ->
// e4m3 with ONE per-batch scale amax/448 reduced on the device; the act scale
// and the per-tensor weight_scale are folded into one device scalar that the
// GEMM reads by pointer (scale block [0]=amax, [1]=quant mul, [2]=folded);
// y[m,out] = x[m,in] @ (e4m3 W)^T, no host synchronization anywhere.
//
// Quantization is three launches on the caller's stream, with no atomics and
// no scratch allocation:
//   1. partial maxima of |x|, one per workgroup, parked in the first bytes of
//      the xq output buffer (it is overwritten in step 3 anyway);
//   2. one workgroup reduces the partials and writes the 4-float scale block;
//   3. every value is scaled by scales[1], clamped to +-448 and converted with
//      the hardware round-to-nearest-even converter (v_cvt_pk_fp8_f32).
// The result is deterministic (max is exact and order-free).
//
// The GEMM uses v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales
// (E8M0 127 = 2^0): 32x32 outputs per 64-deep step, f32 accumulation, the
// folded scale applied once in the epilogue.
#include "bqmm_internal.h"

namespace bqm {

constexpr int kAmaxThreads = 256;
constexpr int kAmaxMaxBlocks = 512;

__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false)));
    v = swap16_max(v);
    return swap32_max(v);
}

__device__ __forceinline__ float block_max(float v, float *red) {
    v = wave_max(v);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    float r = red[0];
    for (int i = 1; i < (int)(blockDim.x >> 6); i++) r = fmaxf(r, red[i]);
    return r;
}

// Step 1: partial[blockIdx.x] = max |x| over a grid-strided share of x.
__global__ __launch_bounds__(kAmaxThreads) void e4m3_amax_partial_kernel(const float4 *__restrict__ x, int64_t nvec,
                                                                         int64_t count, float *__restrict__ partial) {
    __shared__ float red[kAmaxThreads / 64];
    float a = 0.0f;
    const int64_t stride = (int64_t)gridDim.x * kAmaxThreads;
    for (int64_t i = (int64_t)blockIdx.x * kAmaxThreads + threadIdx.x; i < nvec; i += stride) {
        float4 v = x[i];
        a = fmaxf(a, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    (void)count;
    float r = block_max(a, red);
    if (threadIdx.x == 0) partial[blockIdx.x] = r;
}

// Step 2: reduce the partials and write the scale block.
__global__ __launch_bounds__(kAmaxThreads) void e4m3_amax_finalize_kernel(const float *__restrict__ partial, int np,
                                                                          float w_scale, float *__restrict__ scales) {
    __shared__ float red[kAmaxThreads / 64];
    float a = 0.0f;
    for (int i = threadIdx.x; i < np; i += kAmaxThreads) a = fmaxf(a, partial[i]);
    float amax = block_max(a, red);
    if (threadIdx.x == 0) {
        float mul = 0.0f, xs = 0.0f;
        if (amax > 0.0f) {
            mul = 448.0f / amax;
            xs = amax / 448.0f;
        }
        scales[0] = amax;
        scales[1] = mul;
        scales[2] = xs * w_scale;
        scales[3] = xs;
    }
}

__device__ __forceinline__ float clamp448(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }

// Step 3: xq = e4m3(clamp(x * mul)), four values per thread.
__global__ __launch_bounds__(256) void e4m3_quantize_kernel(const float4 *__restrict__ x, int64_t nvec,
                                                            const float *__restrict__ scales,
                                                            unsigned *__restrict__ xq) {
    const float mul = scales[1];
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nvec; i += stride) {
        float4 v = x[i];
        int lo = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(v.x * mul), clamp448(v.y * mul), 0, false);
        int both = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(v.z * mul), clamp448(v.w * mul), lo, true);
        xq[i] = (unsigned)both;
    }
}

// ------------------------------------------------------------------ GEMM

constexpr int kF8BM = 128;
constexpr int kF8BN = 128;
constexpr int kF8KB = 128;        // k per LDS stage (two 64-deep MFMA steps)
constexpr int kF8Threads = 256;   // 4 waves, 2 x 2, each 64 x 64

__device__ __forceinline__ __amdgpu_buffer_rsrc_t f8_rsrc(const void *base, int64_t bytes) {
    uint32_t b = bytes <= 0 ? 0u : (bytes > 0x7FFFFFF0ll ? 0x7FFFFFF0u : (uint32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)b, 0x00020000);
}

__global__ __launch_bounds__(kF8Threads) void e4m3_gemm_kernel(const uint8_t *__restrict__ w,
                                                             const uint8_t *__restrict__ xq,
                                                             const float *__restrict__ scales, float *__restrict__ y,
                                                             int m, int k, int n) {
    __shared__ __attribute__((aligned(16))) uint8_t sA[kF8BM * kF8KB];
    __shared__ __attribute__((aligned(16))) uint8_t sB[kF8BN * kF8KB];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int n0 = blockIdx.x * kF8BN;
    const int m0 = blockIdx.y * kF8BM;
    const int nstage = k / kF8KB;

    const __amdgpu_buffer_rsrc_t rA = f8_rsrc(xq + (int64_t)m0 * k, (int64_t)(m - m0) * k);
    const __amdgpu_buffer_rsrc_t rB = f8_rsrc(w + (int64_t)n0 * k, (int64_t)(n - n0) * k);

    u32x4 ra[4], rb[4];
    auto load_stage = [&](int kc) {
#pragma unroll
        for (int s = 0; s < 4; s++) {
            int q = tid + 256 * s;
            int row = q >> 3, c = q & 7;
            uint32_t off = (uint32_t)(row * k + kc * kF8KB + 16 * c);
            ra[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rA, off, 0, 0));
            rb[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rB, off, 0, 0));
        }
    };
    auto store_stage = [&]() {
#pragma unroll
        for (int s = 0; s < 4; s++) {
            int q = tid + 256 * s;
            int row = q >> 3, c = q & 7;
            *reinterpret_cast<u32x4 *>(sA + row * kF8KB + 16 * (c ^ (row & 7))) = ra[s];
            *reinterpret_cast<u32x4 *>(sB + row * kF8KB + 16 * (c ^ (row & 7))) = rb[s];
        }
    };

    v16f acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[i][j][v] = 0.0f;

    const int khalf = lane >> 5;
    load_stage(0);
    for (int kc = 0; kc < nstage; kc++) {
        store_stage();
        __syncthreads();
        if (kc + 1 < nstage) load_stage(kc + 1);
#pragma unroll
        for (int ks = 0; ks < kF8KB / 64; ks++) {
            const int c0 = ks * 4 + 2 * khalf;   // first 16-byte chunk of this lane's 32 k-values
            v8i a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; i++) {
                int row = wm * 64 + i * 32 + (lane & 31);
                u32x4 lo = *reinterpret_cast<const u32x4 *>(sA + row * kF8KB + 16 * (c0 ^ (row & 7)));
                u32x4 hi = *reinterpret_cast<const u32x4 *>(sA + row * kF8KB + 16 * ((c0 + 1) ^ (row & 7)));
                a[i] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            }
#pragma unroll
            for (int j = 0; j < 2; j++) {
                int row = wn * 64 + j * 32 + (lane & 31);
                u32x4 lo = *reinterpret_cast<const u32x4 *>(sB + row * kF8KB + 16 * (c0 ^ (row & 7)));
                u32x4 hi = *reinterpret_cast<const u32x4 *>(sB + row * kF8KB + 16 * ((c0 + 1) ^ (row & 7)));
                b[j] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            }
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < 2; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], 0, 0, 0, 127, 0, 127);
        }
        __syncthreads();
    }

    const float sc = scales[2];
#pragma unroll
    for (int j = 0; j < 2; j++) {
        int col = n0 + wn * 64 + j * 32 + (lane & 31);
        if (col >= n) continue;
#pragma unroll
        for (int i = 0; i < 2; i++) {
#pragma unroll
            for (int v = 0; v < 16; v++) {
                int row = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * khalf + (v & 3);
                if (row < m) y[(int64_t)row * n + col] = acc[i][j][v] * sc;
            }
        }
    }
}

}  // namespace bqm

extern "C" int bqm_e4m3_quantize_amax(const float *x, uint8_t *xq, float *scales, float w_scale, int m, int k,
                                      void *stream) {
    using namespace bqm;
    if (!x || !xq || !scales) return BQM_EINVAL;
    if (m < 1 || k < 4) return BQM_EINVAL;
    if (!(w_scale == w_scale) || w_scale > 3.4e38f || w_scale < -3.4e38f) return BQM_EINVAL;
    if (k % 4 != 0) return BQM_EUNSUPPORTED;
    if (!aligned(x, 16) || !aligned(xq, 4) || !aligned(scales, 4)) return BQM_EUNSUPPORTED;
    const int64_t count = (int64_t)m * k;
    const int64_t nvec = count / 4;
    // partials live in xq: nblocks floats must fit in count bytes
    int64_t nblocks = (nvec + kAmaxThreads * 8 - 1) / (kAmaxThreads * 8);
    if (nblocks > kAmaxMaxBlocks) nblocks = kAmaxMaxBlocks;
    if (nblocks > count / 4) nblocks = count / 4;
    if (nblocks < 1) nblocks = 1;
    hipStream_t s = as_stream(stream);
    float *partial = reinterpret_cast<float *>(xq);
    hipLaunchKernelGGL(e4m3_amax_partial_kernel, dim3((unsigned)nblocks), dim3(kAmaxThreads), 0, s,
                       reinterpret_cast<const float4 *>(x), nvec, count, partial);
    int rc = launch_status();
    if (rc) return rc;
    hipLaunchKernelGGL(e4m3_amax_finalize_kernel, dim3(1), dim3(kAmaxThreads), 0, s, partial, (int)nblocks, w_scale,
                       scales);
    rc = launch_status();
    if (rc) return rc;
    int64_t qblocks = (nvec + 256 * 4 - 1) / (256 * 4);
    if (qblocks > 4096) qblocks = 4096;
    if (qblocks < 1) qblocks = 1;
    hipLaunchKernelGGL(e4m3_quantize_kernel, dim3((unsigned)qblocks), dim3(256), 0, s,
                       reinterpret_cast<const float4 *>(x), nvec, scales, reinterpret_cast<unsigned *>(xq));
    return launch_status();
}

extern "C" int bqm_e4m3_gemm(const uint8_t *w, const uint8_t *xq, const float *scales, float *y, int m, int k, int n,
                             void *stream) {
    using namespace bqm;
    if (!w || !xq || !scales || !y) return BQM_EINVAL;
    if (m < 1 || k < 128 || n < 1) return BQM_EINVAL;
    if (k % 128 != 0) return BQM_EUNSUPPORTED;
    if (!aligned(w, 16) || !aligned(xq, 16) || !aligned(scales, 4) || !aligned(y, 4)) return BQM_EUNSUPPORTED;
    if ((int64_t)kF8BM * k > 0x7FFFFFF0ll) return BQM_EUNSUPPORTED;
    dim3 grid((n + kF8BN - 1) / kF8BN, (m + kF8BM - 1) / kF8BM);
    if (grid.y > 65535) return BQM_EUNSUPPORTED;
    hipLaunchKernelGGL(e4m3_gemm_kernel, grid, dim3(kF8Threads), 0, as_stream(stream), w, xq, scales, y, m, k, n);
    return launch_status();
}
