// FP8-E4M3 prefill GEMM with a proven error bound: the same result definition
// as bqm_e4m3_gemm ("fp8_ffi.rs" page, memra-engine 0.70.0, module doc and fn
// try_fp8_gemm: the activation times the transposed e4m3 weight, one folded
// device scalar, f32 accumulation), computed so that every output is within
// 1e-5 of the sum of |terms| whatever the data.
//
// Why a second kernel.  The fp8 matrix-core instruction the fast GEMM uses
// (v_mfma_scale_f32_32x32x64_f8f6f4) sums the eight products one lane
// supplies from each 8-byte group after aligning them to the largest and
// cutting them 13 bits below its leading bit (toward zero), so one group can
// lose up to 7 * 2^-13 of its largest product: about 8.5e-4 of the sum of
// |terms| in the worst case, far above 1e-5.  The fp16 instruction used here,
// v_mfma_f32_32x32x16_f16, keeps 24 bits below the largest product of a
// lane's group of eight and rounds each group sum to f32 to nearest even
// before the groups and the accumulator input are added (measured on gfx950,
// element by element; worst observed 3.4 u of the sum of |terms| per
// instruction on random operands).  Every e4m3 value is exact in fp16
// (v_cvt_scalef32_pk_f16_fp8 with scale 1, checked on all 254 finite codes)
// and every fp16 x fp16 product is exact, so per 16-deep step the error is at
// most 7u * (sum of the two group maxima) + u * |group sums| + 2u * (sum |p| +
// |C|) <= 10u * sum|p| + 2u * |C|, u = 2^-24.
//
// Accumulation order.  A 128-k stage is summed into a fresh f32 partial
// (eight 16-deep steps: at most (10 + 2*8) u = 26u of the stage's sum of
// |terms|), and the stage partials are added into the output accumulator on
// the VALU (one rounding each, at most k/128 * u * T), then one multiply by
// the folded scale.  Bound: (27 + k/128) * 2^-24 * T, 3.5e-6 * T at k = 4096
// and below 1e-5 * T for every k <= 16384, the largest k accepted.
//
// Tiles, LDS layout and loads are those of the fast kernel: workgroup tile
// 128 x 64*NT (8 waves in 4 x 2, each 32 x 32*NT, two waves per SIMD), k
// staged 128 at a time as e4m3 bytes in double-buffered LDS with padded
// 144-byte rows, global loads two stages ahead in registers.  Each 64-deep
// step reads the same 32 bytes per lane and operand as the fast kernel and
// feeds them to four 16-deep fp16 MFMAs, 8 bytes (converted to 8 fp16 values)
// each: lane l supplies row l%32 of an operand and, in chunk c, k values
// 32*(l/32) + 8c .. +7 of the step, the same k set for A and B.
#include "bqmm_internal.h"

namespace bqm {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int kExBM = 128;                 // workgroup tile rows (tokens)
constexpr int kExKB = 128;                 // k per LDS stage and per fresh partial
constexpr int kExThreads = 512;            // 8 waves, 4 x 2
constexpr int kExRowStride = kExKB + 16;   // 144: padded LDS row
constexpr int kExMaxK = 16384;             // the bound stays below 1e-5 * T up to here

__device__ __forceinline__ __amdgpu_buffer_rsrc_t ex_rsrc(const void *base, int64_t bytes) {
    uint32_t b = bytes <= 0 ? 0u : (bytes > 0x7FFFFFF0ll ? 0x7FFFFFF0u : (uint32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)b, 0x00020000);
}

// Eight e4m3 codes (two dwords, byte j -> element j) to eight exact fp16 values.
__device__ __forceinline__ v8h e4m3x8_to_f16(unsigned lo, unsigned hi) {
    const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
    const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
    const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
    const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
    const _Float16 e0 = p0[0], e1 = p0[1], e2 = p1[0], e3 = p1[1];
    const _Float16 e4 = p2[0], e5 = p2[1], e6 = p3[0], e7 = p3[1];
    return v8h{e0, e1, e2, e3, e4, e5, e6, e7};
}

template <int NT>
struct ExStage {
    uint8_t a[kExBM * kExRowStride];
    uint8_t b[64 * NT * kExRowStride];
};

template <int NT>
struct ExRegs {
    u32x4 a[2];        // 128 rows x 128 bytes = 1024 chunks, 2 per thread
    u32x4 b[NT];       // 64*NT rows x 128 bytes, NT per thread
};

template <int NT>
__global__ __launch_bounds__(kExThreads) void e4m3_gemm_exact_kernel(const uint8_t *__restrict__ w,
                                                                   const uint8_t *__restrict__ xq,
                                                                   const float *__restrict__ scales,
                                                                   float *__restrict__ y, int m, int k, int n) {
    constexpr int BN = 64 * NT;
    __shared__ __attribute__((aligned(16))) ExStage<NT> st[2];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int n0 = blockIdx.x * BN;
    const int m0 = blockIdx.y * kExBM;
    const int nstage = k / kExKB;

    const __amdgpu_buffer_rsrc_t rA = ex_rsrc(xq + (int64_t)m0 * k, (int64_t)(m - m0) * k);
    const __amdgpu_buffer_rsrc_t rB = ex_rsrc(w + (int64_t)n0 * k, (int64_t)(n - n0) * k);

    // chunk q = tid + 512*s -> row q>>3 (s adds 64 rows), 16-byte chunk q&7
    const uint32_t goff = (uint32_t)((tid >> 3) * k + 16 * (tid & 7));
    const uint32_t grow64 = (uint32_t)(64 * k);
    auto load_stage = [&](ExRegs<NT> &R, int kc) {
        const int so = kc * kExKB;
#pragma unroll
        for (int s = 0; s < 2; s++)
            R.a[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rA, goff + s * grow64, so, 0));
#pragma unroll
        for (int s = 0; s < NT; s++)
            R.b[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rB, goff + s * grow64, so, 0));
    };
    const int lds_off = (tid >> 3) * kExRowStride + 16 * (tid & 7);
    auto store_stage = [&](ExStage<NT> &S, const ExRegs<NT> &R) {
#pragma unroll
        for (int s = 0; s < 2; s++)
            *reinterpret_cast<u32x4 *>(S.a + lds_off + s * 64 * kExRowStride) = R.a[s];
#pragma unroll
        for (int s = 0; s < NT; s++)
            *reinterpret_cast<u32x4 *>(S.b + lds_off + s * 64 * kExRowStride) = R.b[s];
    };

    v16f acc[NT], part[NT];
#pragma unroll
    for (int j = 0; j < NT; j++)
#pragma unroll
        for (int v = 0; v < 16; v++) acc[j][v] = 0.0f;
    const v16f zero = {0};

    const int khalf = lane >> 5;
    v8i a[2], b[2][NT];
    auto ld8 = [](const uint8_t *p) {
        const u32x4 lo = *reinterpret_cast<const u32x4 *>(p);
        const u32x4 hi = *reinterpret_cast<const u32x4 *>(p + 16);
        return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    };
    auto rd = [&](const ExStage<NT> &S, int ks, int slot) {
        const uint8_t *pa = S.a + (wm * 32 + (lane & 31)) * kExRowStride + 32 * khalf + 64 * ks;
        const uint8_t *pb = S.b + (wn * 32 * NT + (lane & 31)) * kExRowStride + 32 * khalf + 64 * ks;
        a[slot] = ld8(pa);
#pragma unroll
        for (int j = 0; j < NT; j++) b[slot][j] = ld8(pb + j * 32 * kExRowStride);
    };
    // One 64-deep step: four 16-deep fp16 MFMAs per output tile.  Step 0 of a
    // stage starts the stage's partial from +0; step 1 ends the stage, whose
    // partial is then added into the accumulator.
    auto mfma_step = [&](int slot, bool first) {
#pragma unroll
        for (int c = 0; c < 4; c++) {
            const v8h ah = e4m3x8_to_f16((unsigned)a[slot][2 * c], (unsigned)a[slot][2 * c + 1]);
#pragma unroll
            for (int j = 0; j < NT; j++) {
                const v8h bh = e4m3x8_to_f16((unsigned)b[slot][j][2 * c], (unsigned)b[slot][j][2 * c + 1]);
                part[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bh, (first && c == 0) ? zero : part[j], 0, 0, 0);
            }
        }
    };
    auto end_stage = [&]() {
#pragma unroll
        for (int j = 0; j < NT; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[j][v] += part[j][v];
    };

    // The pipeline of the fast kernel: loads of stage kc+2 issued while stage
    // kc is computed and stored to LDS one stage later (unconditional: past
    // the last stage they re-read it), the barrier between a stage's two
    // steps, the next stage's step-0 operands read under step 1's MFMAs.
    ExRegs<NT> R0, R1;
    const int last = nstage - 1;
    load_stage(R0, 0);
    load_stage(R1, min(1, last));
    store_stage(st[0], R0);
    __syncthreads();
    rd(st[0], 0, 0);
    int kc = 0;
#pragma unroll 1
    for (; kc + 1 < nstage; kc += 2) {
        load_stage(R0, min(kc + 2, last));
        rd(st[0], 1, 1);
        mfma_step(0, true);
        store_stage(st[1], R1);
        __syncthreads();
        rd(st[1], 0, 0);
        mfma_step(1, false);
        end_stage();
        load_stage(R1, min(kc + 3, last));
        rd(st[1], 1, 1);
        mfma_step(0, true);
        store_stage(st[0], R0);
        __syncthreads();
        rd(st[0], 0, 0);
        mfma_step(1, false);
        end_stage();
    }
    if (kc < nstage) {
        rd(st[0], 1, 1);
        mfma_step(0, true);
        mfma_step(1, false);
        end_stage();
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

// The tile width with the fewest rounds of workgroups over the CUs, each
// round weighted by its width; ties go to the wider tile.
static int ex_pick_nt(int m, int n, int cus, int max_nt) {
    int best = max_nt;
    int64_t best_cost = -1;
    for (int nt = max_nt; nt >= 2; nt--) {
        const int64_t tiles = (int64_t)((m + kExBM - 1) / kExBM) * ((n + 64 * nt - 1) / (64 * nt));
        const int64_t cost = (tiles + cus - 1) / cus * nt;
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best = nt;
        }
    }
    return best;
}

template <int NT>
static int launch_ex(const uint8_t *w, const uint8_t *xq, const float *scales, float *y, int m, int k, int n,
                     hipStream_t s) {
    dim3 grid((n + 64 * NT - 1) / (64 * NT), (m + kExBM - 1) / kExBM);
    if (grid.y > 65535) return BQM_EUNSUPPORTED;
    hipLaunchKernelGGL(e4m3_gemm_exact_kernel<NT>, grid, dim3(kExThreads), 0, s, w, xq, scales, y, m, k, n);
    return launch_status();
}

}  // namespace bqm

extern "C" int bqm_e4m3_gemm_exact(const uint8_t *w, const uint8_t *xq, const float *scales, float *y, int m, int k,
                                   int n, void *stream) {
    using namespace bqm;
    if (!w || !xq || !scales || !y) return BQM_EINVAL;
    if (m < 1 || k < 128 || n < 1) return BQM_EINVAL;
    if (k % 128 != 0 || k > kExMaxK) return BQM_EUNSUPPORTED;
    if (!aligned(w, 16) || !aligned(xq, 16) || !aligned(scales, 4) || !aligned(y, 4)) return BQM_EUNSUPPORTED;
    const int cus = device_cus();
    hipStream_t s = as_stream(stream);
    // NT = 3 is the widest tile whose registers fit two waves per SIMD (248
    // VGPRs; NT = 4 spills)
    switch (ex_pick_nt(m, n, cus, 3)) {
        case 2: return launch_ex<2>(w, xq, scales, y, m, k, n, s);
        default: return launch_ex<3>(w, xq, scales, y, m, k, n, s);
    }
}
