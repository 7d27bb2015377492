// FP8-E4M3 prefill path for gfx950: per-batch activation quantization and the
// e4m3 x e4m3 GEMM with f32 accumulation.
//
// From the "fp8_ffi.rs" page (memra-engine 0.70.0), module doc, fn
// try_fp8_gemm and the Fp8Scratch doc: the whole activation batch shares a
// single e4m3 scale, amax/448, whose amax is reduced on the device; that
// scale times the per-tensor weight_scale is one device scalar the GEMM reads
// through a pointer (the scale block keeps the amax, the quantization
// multiplier and this folded scale, in that order); the output is the
// activation times the transposed e4m3 weight, with no host synchronization.
//
// Quantization is two launches on the caller's stream, with no atomics and
// no scratch allocation:
//   1. partial maxima of |x|, one per workgroup (at most 256), each written
//      into every quantize workgroup's region of the xq output buffer: region
//      j is the first 256 4-byte words that quantize workgroup j writes;
//   2. each quantize workgroup reduces the partials in its own region, so it
//      has the batch amax, before a barrier after which it overwrites them;
//      it scales every value of its share by 448/amax, clamps to +-448 and
//      converts with the hardware round-to-nearest-even converter
//      (v_cvt_pk_fp8_f32); workgroup 0 writes the 4-float scale block.
// The result is deterministic (max is exact and order-free), and every
// workgroup forms the same amax and multiplier.
//
// The GEMM uses v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales
// (E8M0 127 = 2^0): 32x32 outputs per 64-deep step, f32 accumulation, the
// folded scale applied once in the epilogue.
// Workgroup tile 128 x 64*NT (8 waves in 4 x 2, each 32 x 32*NT, two per
// SIMD; NT = 2..5 chosen per shape so the tiles spread evenly over the CUs:
// m=512, N=20480 takes NT=5, 256 tiles of 128 x 320, one per CU); k staged
// 128 at a time in double-buffered LDS with padded 144-byte rows
// (conflict-free reads, immediate offsets), global loads two stages ahead
// in registers, operand reads for the next 64-deep step slotted between the
// current step's MFMAs.
#include "bqmm_internal.h"

namespace bqm {

constexpr int kAmaxThreads = 1024;   // partial-max workgroup, at most (512 below 64 full workgroups)
constexpr int kAmaxMaxBlocks = 64;   // partials; each takes one 4-byte word of every region
constexpr int kQuantThreads = 256;   // quantize workgroup; its region is its first 256 words
constexpr int kQuantMaxBlocks = 4096;

__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false)));
    v = swap16_max(v);
    return swap32_max(v);
}

// Max over the workgroup, returned to every thread; `red` holds one float per
// wave.  Every thread's v is final before the barrier.
__device__ __forceinline__ float block_max(float v, float *red) {
    v = wave_max(v);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    float r = red[0];
    for (int i = 1; i < (int)(blockDim.x >> 6); i++) r = fmaxf(r, red[i]);
    return r;
}

// Step 1: the max |x| over a grid-strided share of x, written to word
// 256 j + blockIdx.x of xq for every quantize workgroup j < nq (one scattered
// 4-byte store per region and partial: few, wide workgroups keep them few).
__global__ __launch_bounds__(kAmaxThreads) void e4m3_amax_partial_kernel(const float4 *__restrict__ x, int64_t nvec,
                                                                         float *__restrict__ regions, int nq) {
    __shared__ float red[kAmaxThreads / 64];
    float a = 0.0f;
    // four independent 16-byte loads in flight per thread and step
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < nvec; i += 4 * stride) {
        float4 v[4];
#pragma unroll
        for (int u = 0; u < 4; u++) v[u] = x[i + u * stride];
#pragma unroll
        for (int u = 0; u < 4; u++)
            a = fmaxf(a, fmaxf(fmaxf(fabsf(v[u].x), fabsf(v[u].y)), fmaxf(fabsf(v[u].z), fabsf(v[u].w))));
    }
    for (; i < nvec; i += stride) {
        float4 v = x[i];
        a = fmaxf(a, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    const float r = block_max(a, red);
    for (int j = threadIdx.x; j < nq; j += blockDim.x) regions[(int64_t)j * kQuantThreads + blockIdx.x] = r;
}

__device__ __forceinline__ float clamp448(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }

// Step 2: the batch amax from this workgroup's region (np partials), then
// xq = e4m3(clamp(x * 448/amax)), four values per thread and step.  The first
// step's loads are issued before the region is reduced.  The region is the
// first word of each thread's first store, read before the barrier in
// block_max, so no store of this workgroup can land before every read.
__global__ __launch_bounds__(kQuantThreads) void e4m3_quantize_kernel(const float4 *__restrict__ x, int64_t nvec,
                                                                      int np, float w_scale,
                                                                      float *__restrict__ scales,
                                                                      unsigned *__restrict__ xq) {
    __shared__ float red[kQuantThreads / 64];
    const int64_t stride = (int64_t)gridDim.x * kQuantThreads;
    const int64_t i0 = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x;
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; u++) v[u] = i0 + u * stride < nvec ? x[i0 + u * stride] : make_float4(0.f, 0.f, 0.f, 0.f);
    const float *region = reinterpret_cast<const float *>(xq) + (int64_t)blockIdx.x * kQuantThreads;
    const float amax = block_max((int)threadIdx.x < np ? region[threadIdx.x] : 0.0f, red);
    float mul = 0.0f, xs = 0.0f;
    if (amax > 0.0f) {
        mul = 448.0f / amax;
        xs = amax / 448.0f;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        scales[0] = amax;
        scales[1] = mul;
        scales[2] = xs * w_scale;
        scales[3] = xs;
    }
    auto q4 = [&](float4 f) {
        int lo = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(f.x * mul), clamp448(f.y * mul), 0, false);
        return (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(clamp448(f.z * mul), clamp448(f.w * mul), lo, true);
    };
#pragma unroll
    for (int u = 0; u < 4; u++)
        if (i0 + u * stride < nvec) xq[i0 + u * stride] = q4(v[u]);
    // past the first step (only where the grid is capped), four independent
    // 16-byte loads in flight per thread and step
    int64_t i = i0 + 4 * stride;
    for (; i + 3 * stride < nvec; i += 4 * stride) {
#pragma unroll
        for (int u = 0; u < 4; u++) v[u] = x[i + u * stride];
#pragma unroll
        for (int u = 0; u < 4; u++) xq[i + u * stride] = q4(v[u]);
    }
    for (; i < nvec; i += stride) xq[i] = q4(x[i]);
}

// ------------------------------------------------------------------ GEMM

constexpr int kF8BM = 128;                 // workgroup tile rows (tokens)
constexpr int kF8KB = 128;                 // k per LDS stage (two 64-deep MFMA steps)
constexpr int kF8Threads = 512;            // 8 waves, 4 x 2: two waves per SIMD
constexpr int kF8RowStride = kF8KB + 16;   // 144: padded LDS row (conflict-free, immediate offsets)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t f8_rsrc(const void *base, int64_t bytes) {
    uint32_t b = bytes <= 0 ? 0u : (bytes > 0x7FFFFFF0ll ? 0x7FFFFFF0u : (uint32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)b, 0x00020000);
}

// Workgroup tile 128 x 64*NT: 8 waves in 4 x 2, each 32 x 32*NT (NT 32x32
// MFMA tiles).  Two waves share each SIMD, so one wave's LDS reads and
// barrier waits hide behind the other's MFMAs.  A wave reads 1 + NT operand
// tiles per 64-deep step for NT MFMAs.
template <int NT>
struct F8Stage {
    uint8_t a[kF8BM * kF8RowStride];
    uint8_t b[64 * NT * kF8RowStride];
};

template <int NT>
struct F8Regs {
    u32x4 a[2];        // 128 rows x 128 bytes = 1024 chunks, 2 per thread
    u32x4 b[NT];       // 64*NT rows x 128 bytes, NT per thread
};

template <int NT>
__global__ __launch_bounds__(kF8Threads) void e4m3_gemm_kernel(const uint8_t *__restrict__ w,
                                                             const uint8_t *__restrict__ xq,
                                                             const float *__restrict__ scales, float *__restrict__ y,
                                                             int m, int k, int n) {
    constexpr int BN = 64 * NT;
    __shared__ __attribute__((aligned(16))) F8Stage<NT> st[2];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int n0 = blockIdx.x * BN;
    const int m0 = blockIdx.y * kF8BM;
    const int nstage = k / kF8KB;

    const __amdgpu_buffer_rsrc_t rA = f8_rsrc(xq + (int64_t)m0 * k, (int64_t)(m - m0) * k);
    const __amdgpu_buffer_rsrc_t rB = f8_rsrc(w + (int64_t)n0 * k, (int64_t)(n - n0) * k);

    // Thread slots: chunk q = tid + 512*s -> row q>>3 (s adds 64 rows), 16-byte
    // chunk q&7.  The stage offset is a uniform scalar added by the load.
    const uint32_t goff = (uint32_t)((tid >> 3) * k + 16 * (tid & 7));
    const uint32_t grow64 = (uint32_t)(64 * k);
    auto load_stage = [&](F8Regs<NT> &R, int kc) {
        const int so = kc * kF8KB;
#pragma unroll
        for (int s = 0; s < 2; s++)
            R.a[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rA, goff + s * grow64, so, 0));
#pragma unroll
        for (int s = 0; s < NT; s++)
            R.b[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rB, goff + s * grow64, so, 0));
    };
    const int lds_off = (tid >> 3) * kF8RowStride + 16 * (tid & 7);
    auto store_stage = [&](F8Stage<NT> &S, const F8Regs<NT> &R) {
#pragma unroll
        for (int s = 0; s < 2; s++)
            *reinterpret_cast<u32x4 *>(S.a + lds_off + s * 64 * kF8RowStride) = R.a[s];
#pragma unroll
        for (int s = 0; s < NT; s++)
            *reinterpret_cast<u32x4 *>(S.b + lds_off + s * 64 * kF8RowStride) = R.b[s];
    };

    v16f acc[NT];
#pragma unroll
    for (int j = 0; j < NT; j++)
#pragma unroll
        for (int v = 0; v < 16; v++) acc[j][v] = 0.0f;

    const int khalf = lane >> 5;
    // Lane l supplies row l%32 of each 32-row operand tile and k values
    // 32*(l/32) .. +31 of the 64-deep step (the same k set for A and B).
    // Operands of a 64-deep step live in slot 0 (step 0 of a stage) or slot 1
    // (step 1), kept across stages.
    v8i a[2], b[2][NT];
    auto ld8 = [](const uint8_t *p) {
        const u32x4 lo = *reinterpret_cast<const u32x4 *>(p);
        const u32x4 hi = *reinterpret_cast<const u32x4 *>(p + 16);
        return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    };
    auto rd = [&](const F8Stage<NT> &S, int ks, int slot) {
        const uint8_t *pa = S.a + (wm * 32 + (lane & 31)) * kF8RowStride + 32 * khalf + 64 * ks;
        const uint8_t *pb = S.b + (wn * 32 * NT + (lane & 31)) * kF8RowStride + 32 * khalf + 64 * ks;
        a[slot] = ld8(pa);
#pragma unroll
        for (int j = 0; j < NT; j++) b[slot][j] = ld8(pb + j * 32 * kF8RowStride);
    };
    auto mfma_step = [&](int slot) {
#pragma unroll
        for (int j = 0; j < NT; j++)
            acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[slot], b[slot][j], acc[j], 0, 0, 0, 127, 0,
                                                                   127);
    };
    // Scheduling groups (masks: 0x020 VMEM read, 0x100 DS read, 0x200 DS
    // write, 0x008 MFMA).  Before the barrier: the global loads, then step
    // 0's MFMAs one at a time with step 1's operand reads and the next
    // stage's stores between them.  After it: step 1's MFMAs with the next
    // stage's step-0 operand reads between them.
    auto groups_before = [&]() {
        __builtin_amdgcn_sched_group_barrier(0x020, 2 + NT, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int r = 0; r < NT; r++) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);
    };
    auto groups_after = [&]() {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int r = 0; r < NT; r++) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        // end of the scheduling region: nothing of the next stage moves up
        __builtin_amdgcn_sched_barrier(0);
    };

    // Two register copies: the loads of stage kc+2 are issued while stage kc
    // is computed, and written to LDS one stage later.  Past the last stage
    // the loads re-read it (unconditional loads keep the compiler's count of
    // loads in flight exact).  The barrier sits between a stage's two 64-deep
    // steps: once the next stage's stores are complete, its step-0 operands
    // are read while this stage's step-1 MFMAs run, so no stage starts by
    // waiting for its own LDS reads.  (__syncthreads waits for this wave's
    // LDS reads too, so a buffer is fully consumed before it is rewritten one
    // stage later.)
    F8Regs<NT> R0, R1;
    const int last = nstage - 1;
    load_stage(R0, 0);
    load_stage(R1, min(1, last));
    store_stage(st[0], R0);
    __syncthreads();
    rd(st[0], 0, 0);
    int kc = 0;
#pragma unroll 1
    for (; kc + 1 < nstage; kc += 2) {
        // stage kc in st[0]; R1 holds stage kc+1
        load_stage(R0, min(kc + 2, last));
        rd(st[0], 1, 1);
        mfma_step(0);
        store_stage(st[1], R1);
        groups_before();
        __syncthreads();
        rd(st[1], 0, 0);
        mfma_step(1);
        groups_after();
        // stage kc+1 in st[1]; R0 holds stage kc+2
        load_stage(R1, min(kc + 3, last));
        rd(st[1], 1, 1);
        mfma_step(0);
        store_stage(st[0], R0);
        groups_before();
        __syncthreads();
        rd(st[0], 0, 0);
        mfma_step(1);
        groups_after();
    }
    if (kc < nstage) {
        // an odd last stage, in st[0], its step-0 operands already read
        rd(st[0], 1, 1);
        mfma_step(0);
        mfma_step(1);
    }

    const float sc = scales[2];
#pragma unroll
    for (int j = 0; j < NT; j++) {
        const int col = n0 + wn * 32 * NT + j * 32 + (lane & 31);
        if (col >= n) continue;
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int row = m0 + wm * 32 + 8 * (v >> 2) + 4 * khalf + (v & 3);
            if (row < m) y[(int64_t)row * n + col] = acc[j][v] * sc;
        }
    }
}

// Pick the tile width (NT) that needs the fewest rounds of workgroups over
// the CUs, weighting each round by its tile width; ties go to the wider tile
// (less LDS traffic per MFMA).
static int pick_nt(int m, int n, int cus) {
    int best = 5;
    int64_t best_cost = -1;
    for (int nt = 5; nt >= 2; nt--) {
        const int64_t tiles = (int64_t)((m + kF8BM - 1) / kF8BM) * ((n + 64 * nt - 1) / (64 * nt));
        const int64_t rounds = (tiles + cus - 1) / cus;
        const int64_t cost = rounds * nt;
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best = nt;
        }
    }
    return best;
}

template <int NT>
static int launch_f8(const uint8_t *w, const uint8_t *xq, const float *scales, float *y, int m, int k, int n,
                     hipStream_t s) {
    dim3 grid((n + 64 * NT - 1) / (64 * NT), (m + kF8BM - 1) / kF8BM);
    if (grid.y > 65535) return BQM_EUNSUPPORTED;
    hipLaunchKernelGGL(e4m3_gemm_kernel<NT>, grid, dim3(kF8Threads), 0, s, w, xq, scales, y, m, k, n);
    return launch_status();
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
    // quantize workgroups: one pass of four loads per thread where the grid
    // allows; partial workgroups: at most one per word of a region
    int64_t nq = (nvec + kQuantThreads * 4 - 1) / (kQuantThreads * 4);
    if (nq > kQuantMaxBlocks) nq = kQuantMaxBlocks;
    const int pt = nvec >= (int64_t)kAmaxMaxBlocks * kAmaxThreads * 4 ? kAmaxThreads : kAmaxThreads / 2;
    int64_t np = (nvec + pt * 4 - 1) / (pt * 4);
    if (np > kAmaxMaxBlocks) np = kAmaxMaxBlocks;
    // region j (words 256 j .. 256 j + np - 1) lies in the words quantize
    // workgroup j writes in its first step: words 256 j + t, t < 256, below nvec
    if (np > nvec - (nq - 1) * kQuantThreads) np = nvec - (nq - 1) * kQuantThreads;
    if (np < 1 || np > kQuantThreads) return BQM_EINVAL;   // unreachable for nvec >= 1
    hipStream_t s = as_stream(stream);
    hipLaunchKernelGGL(e4m3_amax_partial_kernel, dim3((unsigned)np), dim3(pt), 0, s,
                       reinterpret_cast<const float4 *>(x), nvec, reinterpret_cast<float *>(xq), (int)nq);
    const int rc = launch_status();
    if (rc) return rc;
    hipLaunchKernelGGL(e4m3_quantize_kernel, dim3((unsigned)nq), dim3(kQuantThreads), 0, s,
                       reinterpret_cast<const float4 *>(x), nvec, (int)np, w_scale, scales,
                       reinterpret_cast<unsigned *>(xq));
    return launch_status();
}

extern "C" int bqm_e4m3_gemm(const uint8_t *w, const uint8_t *xq, const float *scales, float *y, int m, int k, int n,
                             void *stream) {
    using namespace bqm;
    if (!w || !xq || !scales || !y) return BQM_EINVAL;
    if (m < 1 || k < 128 || n < 1) return BQM_EINVAL;
    if (k % 128 != 0) return BQM_EUNSUPPORTED;
    if (!aligned(w, 16) || !aligned(xq, 16) || !aligned(scales, 4) || !aligned(y, 4)) return BQM_EUNSUPPORTED;
    if ((int64_t)kF8BM * k > 0x7FFFFFF0ll || (int64_t)320 * k > 0x7FFFFFF0ll) return BQM_EUNSUPPORTED;
    const int cus = device_cus();
    hipStream_t s = as_stream(stream);
    switch (pick_nt(m, n, cus)) {
        case 2: return launch_f8<2>(w, xq, scales, y, m, k, n, s);
        case 3: return launch_f8<3>(w, xq, scales, y, m, k, n, s);
        case 4: return launch_f8<4>(w, xq, scales, y, m, k, n, s);
        default: return launch_f8<5>(w, xq, scales, y, m, k, n, s);
    }
}
