// fp16 mirror prefill path for gfx950: Q8_0 -> fp16 weight dequant (load
// time), f32 -> fp16 activation cast, and the fp16 GEMM with f32
// accumulation and f32 output.
//
// From the "f16_ffi.rs" page (memra-engine 0.81.0), module doc and the
// memra_q8_0_dequant_f16 / memra_f16_cvt / memra_f16_pp_gemm_pre
// declarations: a resident row-major fp16 copy of each Q8_0 projection, the
// activation cast once to fp16, then an fp16 GEMM that accumulates in f32 with
// no mid-loop reads of the accumulator (the per-32-block scale fold is paid
// once, at dequant time).  Rounding enters only at the two casts: the int8
// quants are exact in fp16 and d*q is exact in f32 before its cast.
//
//  * Dequant: one thread per 68-byte block pair (4-byte aligned), 17 dword
//    loads, the even block realigned with v_alignbit; d*q in f32 (exact),
//    then v_cvt_f16_f32 (round to nearest even, fp16 denormals kept).
//  * Cast: four values per thread, the same conversion.
//  * GEMM: the e4m3 GEMM's organisation with v_mfma_f32_32x32x16_f16:
//    workgroup tile 128 x 64*NT, 8 waves of 32 x 32*NT (two per SIMD), k
//    staged 64 values (128 bytes) at a time in double-buffered LDS with padded
//    144-byte rows, global loads two stages ahead in registers, each 16-deep
//    step's operands read between the previous step's MFMAs.  Lane l supplies
//    row l%32 of an operand tile and k values 8*(l/32) .. +7 of the step (the
//    same k set for both operands, so the products pair up whatever order the
//    matrix core sums them in).
#include <type_traits>

#include "bqmm_internal.h"

namespace bqm {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------------ dequant / cast

__global__ __launch_bounds__(256) void q8_0_dequant_f16_kernel(const uint8_t *__restrict__ w, int64_t w_row_bytes,
                                                             uint16_t *__restrict__ w16, int k, int n) {
    const int pairs = k / 64;
    const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (id >= (int64_t)pairs * n) return;
    const int64_t r = id / pairs;
    const int p = (int)(id - r * pairs);
    const uint32_t *src = reinterpret_cast<const uint32_t *>(w + r * w_row_bytes + 68 * p);
    uint32_t d[17];
#pragma unroll
    for (int i = 0; i < 17; i++) d[i] = src[i];
    const float da = half_bits_to_float(d[0] & 0xFFFFu);
    const float db = half_bits_to_float(d[8] >> 16);
    uint32_t out[32];   // 64 fp16 values, two per dword
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const uint32_t qa = __builtin_amdgcn_alignbit(d[i + 1], d[i], 16u);   // quants 4i..4i+3 of block a
        const uint32_t qb = d[9 + i];                                           // quants 4i..4i+3 of block b
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int8_t a0 = (int8_t)(qa >> (16 * h)), a1 = (int8_t)(qa >> (16 * h + 8));
            const int8_t b0 = (int8_t)(qb >> (16 * h)), b1 = (int8_t)(qb >> (16 * h + 8));
            float pa0 = da * (float)a0, pa1 = da * (float)a1, pb0 = db * (float)b0, pb1 = db * (float)b1;
            // Keep the f32 product and the fp16 conversion apart: fused into
            // one mixed-precision fma the product gains a +0 addend, which
            // turns a -0 product (d = -0, or q = 0 with d < 0) into +0.
            asm volatile("" : "+v"(pa0), "+v"(pa1), "+v"(pb0), "+v"(pb1));
            const _Float16 ha0 = (_Float16)pa0, ha1 = (_Float16)pa1;
            const _Float16 hb0 = (_Float16)pb0, hb1 = (_Float16)pb1;
            out[2 * i + h] = (uint32_t)__builtin_bit_cast(uint16_t, ha0) | ((uint32_t)__builtin_bit_cast(uint16_t, ha1) << 16);
            out[16 + 2 * i + h] = (uint32_t)__builtin_bit_cast(uint16_t, hb0) | ((uint32_t)__builtin_bit_cast(uint16_t, hb1) << 16);
        }
    }
    u32x4 *dst = reinterpret_cast<u32x4 *>(w16 + r * k + 64 * p);
#pragma unroll
    for (int i = 0; i < 8; i++) dst[i] = u32x4{out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]};
}

__global__ __launch_bounds__(256) void f16_cvt_kernel(const float4 *__restrict__ x, int64_t nvec, const float *__restrict__ xt,
                                                    int64_t count, uint2 *__restrict__ out, uint16_t *__restrict__ out_t) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nvec; i += stride) {
        const float4 v = x[i];
        const uint16_t h0 = __builtin_bit_cast(uint16_t, (_Float16)v.x), h1 = __builtin_bit_cast(uint16_t, (_Float16)v.y);
        const uint16_t h2 = __builtin_bit_cast(uint16_t, (_Float16)v.z), h3 = __builtin_bit_cast(uint16_t, (_Float16)v.w);
        out[i] = uint2{(uint32_t)h0 | ((uint32_t)h1 << 16), (uint32_t)h2 | ((uint32_t)h3 << 16)};
    }
    // the count % 4 tail
    const int64_t t = nvec * 4 + (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t < count) out_t[t] = __builtin_bit_cast(uint16_t, (_Float16)xt[t]);
}

// ------------------------------------------------------------------ GEMM

constexpr int kH16BM = 128;                 // workgroup tile rows (tokens)
constexpr int kH16KB = 128;                 // bytes of k per LDS stage = 64 fp16 values
constexpr int kH16Threads = 512;            // 8 waves, 4 x 2
constexpr int kH16RowStride = kH16KB + 16;  // 144: padded LDS row

__device__ __forceinline__ __amdgpu_buffer_rsrc_t h16_rsrc(const void *base, int64_t bytes) {
    uint32_t b = bytes <= 0 ? 0u : (bytes > 0x7FFFFFF0ll ? 0x7FFFFFF0u : (uint32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)b, 0x00020000);
}

template <int NT>
struct H16Stage {
    uint8_t a[kH16BM * kH16RowStride];
    uint8_t b[64 * NT * kH16RowStride];
};

template <int NT>
struct H16Regs {
    u32x4 a[2];        // 128 rows x 128 bytes = 1024 chunks, 2 per thread
    u32x4 b[NT];       // 64*NT rows x 128 bytes, NT per thread
};

template <int NT>
__global__ __launch_bounds__(kH16Threads) void f16_gemm_kernel(const uint16_t *__restrict__ w16,
                                                             const uint16_t *__restrict__ x16, float *__restrict__ y,
                                                             int m, int k, int n) {
    constexpr int BN = 64 * NT;
    __shared__ __attribute__((aligned(16))) H16Stage<NT> st[2];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int n0 = blockIdx.x * BN;
    const int m0 = blockIdx.y * kH16BM;
    const int kbytes = 2 * k;
    const int nstage = kbytes / kH16KB;

    const __amdgpu_buffer_rsrc_t rA = h16_rsrc(x16 + (int64_t)m0 * k, (int64_t)(m - m0) * kbytes);
    const __amdgpu_buffer_rsrc_t rB = h16_rsrc(w16 + (int64_t)n0 * k, (int64_t)(n - n0) * kbytes);

    // chunk q = tid + 512*s -> row q>>3 (s adds 64 rows), 16-byte chunk q&7
    const uint32_t goff = (uint32_t)((tid >> 3) * kbytes + 16 * (tid & 7));
    const uint32_t grow64 = (uint32_t)(64 * kbytes);
    auto load_stage = [&](H16Regs<NT> &R, int kc) {
        const int so = kc * kH16KB;
#pragma unroll
        for (int s = 0; s < 2; s++)
            R.a[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rA, goff + s * grow64, so, 0));
#pragma unroll
        for (int s = 0; s < NT; s++)
            R.b[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rB, goff + s * grow64, so, 0));
    };
    const int lds_off = (tid >> 3) * kH16RowStride + 16 * (tid & 7);
    auto store_stage = [&](H16Stage<NT> &S, const H16Regs<NT> &R) {
#pragma unroll
        for (int s = 0; s < 2; s++)
            *reinterpret_cast<u32x4 *>(S.a + lds_off + s * 64 * kH16RowStride) = R.a[s];
#pragma unroll
        for (int s = 0; s < NT; s++)
            *reinterpret_cast<u32x4 *>(S.b + lds_off + s * 64 * kH16RowStride) = R.b[s];
    };

    v16f acc[NT];
#pragma unroll
    for (int j = 0; j < NT; j++)
#pragma unroll
        for (int v = 0; v < 16; v++) acc[j][v] = 0.0f;

    const int khalf = lane >> 5;
    constexpr int kSteps = kH16KB / 32;   // 16 fp16 values (32 bytes) per MFMA step
    static_assert(kSteps % 2 == 0, "operand slots alternate by step parity across stages");
    // Operands of a 16-deep step in slot (step parity), kept across stages.
    v8h a[2], b[2][NT];
    auto rd = [&](const H16Stage<NT> &S, int ks, int slot) {
        const uint8_t *pa = S.a + (wm * 32 + (lane & 31)) * kH16RowStride + 16 * khalf + 32 * ks;
        const uint8_t *pb = S.b + (wn * 32 * NT + (lane & 31)) * kH16RowStride + 16 * khalf + 32 * ks;
        a[slot] = *reinterpret_cast<const v8h *>(pa);
#pragma unroll
        for (int j = 0; j < NT; j++) b[slot][j] = *reinterpret_cast<const v8h *>(pb + j * 32 * kH16RowStride);
    };
    auto mfma_step = [&](int slot) {
#pragma unroll
        for (int j = 0; j < NT; j++)
            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[slot], b[slot][j], acc[j], 0, 0, 0);
    };
    // One stage: steps 0 .. kSteps-2 with the next step's operand reads under
    // their MFMAs and the next stage's stores after them; then the barrier;
    // then the last step's MFMAs with the next stage's step-0 reads under
    // them, so no stage starts by waiting for its own LDS reads.  The
    // scheduling barrier closes the region so the compiler does not pull the
    // next stage's reads forward.  (__syncthreads waits for this wave's LDS
    // reads too, so a buffer is fully consumed before it is rewritten one
    // stage later.)
    // Scheduling groups (masks: 0x020 VMEM read, 0x100 DS read, 0x200 DS
    // write, 0x008 MFMA): the stage's global loads, then per step one operand
    // read and NT x (one MFMA, one read), then the stores; after the barrier
    // the same pattern for the last step.
    auto stage_body = [&](const H16Stage<NT> &cur, H16Stage<NT> &nxt, const H16Regs<NT> &Rn, bool store) {
#pragma unroll
        for (int ks = 0; ks + 1 < kSteps; ks++) {
            rd(cur, ks + 1, (ks + 1) & 1);
            mfma_step(ks & 1);
        }
        if (store) store_stage(nxt, Rn);
        __builtin_amdgcn_sched_group_barrier(0x020, 2 + NT, 0);
#pragma unroll
        for (int ks = 0; ks + 1 < kSteps; ks++) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
            for (int j = 0; j < NT; j++) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        }
        __builtin_amdgcn_sched_group_barrier(0x200, 2 + NT, 0);
        __syncthreads();
        rd(nxt, 0, 0);
        mfma_step((kSteps - 1) & 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
        for (int j = 0; j < NT; j++) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // Two register copies: the loads of stage kc+2 are issued while stage kc
    // is computed and written to LDS one stage later; past the last stage the
    // loads re-read it (unconditional loads keep the compiler's count of loads
    // in flight exact).
    H16Regs<NT> R0, R1;
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
        stage_body(st[0], st[1], R1, true);    // stage kc; stores stage kc+1
        load_stage(R1, min(kc + 3, last));
        stage_body(st[1], st[0], R0, true);    // stage kc+1; stores stage kc+2 (the last again past the end)
    }
    if (kc < nstage) {
        // an odd last stage, in st[0], its step-0 operands already read
#pragma unroll
        for (int ks = 0; ks + 1 < kSteps; ks++) {
            rd(st[0], ks + 1, (ks + 1) & 1);
            mfma_step(ks & 1);
        }
        mfma_step((kSteps - 1) & 1);
    }

#pragma unroll
    for (int j = 0; j < NT; j++) {
        const int col = n0 + wn * 32 * NT + j * 32 + (lane & 31);
        if (col >= n) continue;
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int row = m0 + wm * 32 + 8 * (v >> 2) + 4 * khalf + (v & 3);
            if (row < m) y[(int64_t)row * n + col] = acc[j][v];
        }
    }
}

// The tile width (NT) that needs the fewest rounds of workgroups over the CUs,
// weighting each round by its width; ties go to the wider tile.
static int h16_pick_nt(int m, int n, int cus) {
    int best = 5;
    int64_t best_cost = -1;
    for (int nt = 5; nt >= 2; nt--) {
        const int64_t tiles = (int64_t)((m + kH16BM - 1) / kH16BM) * ((n + 64 * nt - 1) / (64 * nt));
        const int64_t cost = (tiles + cus - 1) / cus * nt;
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best = nt;
        }
    }
    return best;
}

template <int NT>
static int launch_h16(const uint16_t *w16, const uint16_t *x16, float *y, int m, int k, int n, hipStream_t s) {
    dim3 grid((n + 64 * NT - 1) / (64 * NT), (m + kH16BM - 1) / kH16BM);
    if (grid.y > 65535) return BQM_EUNSUPPORTED;
    hipLaunchKernelGGL(f16_gemm_kernel<NT>, grid, dim3(kH16Threads), 0, s, w16, x16, y, m, k, n);
    return launch_status();
}

}  // namespace bqm

extern "C" int bqm_q8_0_dequant_f16(const uint8_t *w, int64_t w_row_bytes, uint16_t *w16, int k, int n, void *stream) {
    using namespace bqm;
    if (!w || !w16) return BQM_EINVAL;
    if (k < 64 || n < 1) return BQM_EINVAL;
    if (k % 64 != 0) return BQM_EUNSUPPORTED;
    if (w_row_bytes < (int64_t)(k / kQK) * kQ80Bytes || w_row_bytes % 4 != 0) return BQM_EUNSUPPORTED;
    if (!aligned(w, 4) || !aligned(w16, 16)) return BQM_EUNSUPPORTED;
    const int64_t threads = (int64_t)(k / 64) * n;
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7FFFFFFF) return BQM_EUNSUPPORTED;
    hipLaunchKernelGGL(q8_0_dequant_f16_kernel, dim3((unsigned)blocks), dim3(256), 0, as_stream(stream), w, w_row_bytes,
                       w16, k, n);
    return launch_status();
}

extern "C" int bqm_f16_cvt(const float *x, uint16_t *x16, int64_t count, void *stream) {
    using namespace bqm;
    if (!x || !x16) return BQM_EINVAL;
    if (count < 1) return BQM_EINVAL;
    if (!aligned(x, 16) || !aligned(x16, 8)) return BQM_EUNSUPPORTED;
    const int64_t nvec = count / 4;
    int64_t blocks = (nvec + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(f16_cvt_kernel, dim3((unsigned)blocks), dim3(256), 0, as_stream(stream),
                       reinterpret_cast<const float4 *>(x), nvec, x, count, reinterpret_cast<uint2 *>(x16), x16);
    return launch_status();
}

extern "C" int bqm_f16_gemm(const uint16_t *w16, const uint16_t *x16, float *y, int m, int k, int n, void *stream) {
    using namespace bqm;
    if (!w16 || !x16 || !y) return BQM_EINVAL;
    if (m < 1 || k < 64 || n < 1) return BQM_EINVAL;
    if (k % 64 != 0) return BQM_EUNSUPPORTED;
    if (!aligned(w16, 16) || !aligned(x16, 16) || !aligned(y, 4)) return BQM_EUNSUPPORTED;
    if ((int64_t)kH16BM * 2 * k > 0x7FFFFFF0ll || (int64_t)320 * 2 * k > 0x7FFFFFF0ll) return BQM_EUNSUPPORTED;
    const int cus = device_cus();
    hipStream_t s = as_stream(stream);
    switch (h16_pick_nt(m, n, cus)) {
        case 2: return launch_h16<2>(w16, x16, y, m, k, n, s);
        case 3: return launch_h16<3>(w16, x16, y, m, k, n, s);
        case 4: return launch_h16<4>(w16, x16, y, m, k, n, s);
        default: return launch_h16<5>(w16, x16, y, m, k, n, s);
    }
}
