// Block-128 FP8 prefill path for gfx950: the e4m3 NaN-code count of a weight,
// the per-(token, 128-k block) activation quantization, and the per-block FP8
// GEMM that applies the block scales a single time per 128 values of k.
//
// From the "fp8_ffi.rs" page (memra-engine 0.70.0), the per-block FP8 MMQ
// section (try_fp8_blk_mmq, fp8_mmq_enabled and FP8_MMQ_NAN_OK docs): the
// weight is the checkpoint's e4m3 codes [n][k] with a row-major f32 grid
// [ceil(n/128)][ceil(k/128)], one scale per 128x128 block, and no second
// (per-tensor) scale; the hardware reads magnitude 0x7F as NaN, so a weight
// holding any is refused after a one-time count; y[m,out] = x[m,in] @ W^T with
// each weight block scaled by its own f32.  The "accprobe_bench.rs" module
// doc describes the kernel class: products chained into one accumulator per
// 128-k block and folded once per block.  The activation side is not shown on
// the pages; it is quantized here per (token, 128-k block) with the pages'
// amax/448 rule, so block kb of output (t, r) folds by grid[r/128][kb] *
// xs[t][kb].
//
// GEMM design (MFMA-bound, one fold per 128-k block):
//  * The e4m3 GEMM's organisation: workgroup tile 128 x 64*NT, 8 waves of
//    32 x 32*NT (two per SIMD), k staged 128 at a time (exactly one grid
//    block) in double-buffered LDS with padded 144-byte rows, global loads
//    two stages ahead in registers; NT (2..5) chosen per shape so the tiles
//    fill whole rounds of the CUs (m=512, N=20480: NT=5, 256 tiles).
//  * Per stage and 32x32 tile a wave runs two v_mfma_scale_f32_32x32x64_f8f6f4
//    (unit E8M0 scales) into a block partial P started at zero and folds it,
//    acc += P * (xs[t] * g).  g is one scalar per 32-column tile (a 32-aligned
//    tile never straddles a 128-row block of the grid), read with scalar
//    loads one stage ahead; the 128 token scales of the stage go through LDS
//    with the operand tiles.
//  * NT >= 3: the weight tile is the MFMA's A operand, so the partial is
//    [weight row][token] and a lane's 16 outputs share one token, hence one
//    scale xs[t] * g: one multiply and 16 fma per tile and stage.  Three
//    partials rotate, so a tile is folded while the next two tiles' MFMAs
//    run (a fold that reads MFMA results issued just before it barely
//    overlaps the matrix cores).  Interleaved on one box at m=512, K=4096,
//    N=20480: 68.4 us against 73.1 with [token][row] partials, two in flight
//    and 16 multiplies per tile; bitwise the same results.
//  * NT = 2 keeps the [token][row] layout with two partials (faster there).
#include "bqmm_internal.h"

namespace bqm {

// ------------------------------------------------------------------ NaN count

// Bytes whose low 7 bits are all ones, counted per dword without branches:
// t is zero exactly in those bytes, and the high bit of each byte of the
// final mask is set exactly where t's byte is zero (no carries cross bytes).
__device__ __forceinline__ unsigned nan_bytes(unsigned d) {
    const unsigned t = (d & 0x7F7F7F7Fu) ^ 0x7F7F7F7Fu;
    const unsigned y = (t & 0x7F7F7F7Fu) + 0x7F7F7F7Fu;
    return (unsigned)__builtin_popcount(~(y | t | 0x7F7F7F7Fu));
}

__global__ void e4m3_nan_zero_kernel(unsigned long long *out) {
    if (threadIdx.x == 0) *out = 0ull;
}

__global__ __launch_bounds__(256) void e4m3_nan_count_kernel(const u32x4 *__restrict__ b, int64_t nvec,
                                                             const uint8_t *__restrict__ bytes, int64_t count,
                                                             unsigned long long *out) {
    __shared__ unsigned part[4];
    unsigned c = 0;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nvec; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(b + i);
        c += nan_bytes(v[0]) + nan_bytes(v[1]) + nan_bytes(v[2]) + nan_bytes(v[3]);
    }
    // the count % 16 tail, one byte per thread of the first workgroup
    if (blockIdx.x == 0) {
        const int64_t t = nvec * 16 + threadIdx.x;
        if (t < count) c += ((bytes[t] & 0x7F) == 0x7F) ? 1u : 0u;
    }
    // wave sums: DPP within rows of 16, then the row and half exchanges
    c += (unsigned)__builtin_amdgcn_update_dpp(0, (int)c, 0xB1, 0xF, 0xF, false);
    c += (unsigned)__builtin_amdgcn_update_dpp(0, (int)c, 0x4E, 0xF, 0xF, false);
    c += (unsigned)__builtin_amdgcn_update_dpp(0, (int)c, 0x141, 0xF, 0xF, false);
    c += (unsigned)__builtin_amdgcn_update_dpp(0, (int)c, 0x140, 0xF, 0xF, false);
    {
        auto s = __builtin_amdgcn_permlane16_swap(c, c, false, false);
        unsigned a0 = s[0], a1 = s[1];
        c = a0 + a1;
        auto s2 = __builtin_amdgcn_permlane32_swap(c, c, false, false);
        unsigned b0 = s2[0], b1 = s2[1];
        c = b0 + b1;
    }
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned long long total = (unsigned long long)part[0] + part[1] + part[2] + part[3];
        if (total) atomicAdd(out, total);
    }
}

// ------------------------------------------------------------------ activation quantization

__device__ __forceinline__ float dpp_max16(float v) {
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false)));
    return v;
}

__device__ __forceinline__ float clamp448b(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }

// One 128-value block per 32 lanes (a float4 each), eight blocks per
// workgroup.  Blocks are numbered t * kbn + kb (kbn = ceil(k/128)), the order
// of xs; block kb of token t holds values 128*kb .. min(128*kb + 128, k) - 1
// of row t (the last block of a row is short when k % 128 != 0; k % 16 == 0,
// so a lane's float4 is wholly inside or wholly past it).
__global__ __launch_bounds__(256) void e4m3_blk_quantize_kernel(const float4 *__restrict__ x, int64_t nblocks,
                                                                int k, int kbn, unsigned *__restrict__ xq,
                                                                float *__restrict__ xs) {
    const int64_t g0 = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
    const bool live = g0 < nblocks;
    const int64_t g = live ? g0 : nblocks - 1;   // past the end: recompute the last block, store nothing
    const int l = threadIdx.x & 31;
    const int64_t t = g / kbn;
    const int kb = (int)(g - t * kbn);
    const bool in = 128 * kb + 4 * l < k;          // this lane's four values exist
    const int64_t v4 = (t * k + 128 * kb) / 4 + l;  // its float4 in x (and dword in xq)
    const float4 v = in ? x[v4] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    a = dpp_max16(a);
    a = swap16_max(a);   // lanes l and l^16: the block's 32 lanes
    float mul = 0.0f, s = 0.0f;
    if (a > 0.0f) {
        mul = 448.0f / a;
        s = a / 448.0f;
    }
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448b(v.x * mul), clamp448b(v.y * mul), 0, false);
    const int both = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448b(v.z * mul), clamp448b(v.w * mul), lo, true);
    if (live) {
        if (in) xq[v4] = (unsigned)both;
        if (l == 0) xs[g] = s;
    }
}

// ------------------------------------------------------------------ GEMM

constexpr int kB8BM = 128;                 // workgroup tile rows (tokens)
constexpr int kB8KB = 128;                 // k per stage = one grid block
constexpr int kB8Threads = 512;            // 8 waves, 4 x 2
constexpr int kB8RowStride = kB8KB + 16;   // 144: padded LDS row

__device__ __forceinline__ __amdgpu_buffer_rsrc_t b8_rsrc(const void *base, int64_t bytes) {
    uint32_t b = bytes <= 0 ? 0u : (bytes > 0x7FFFFFF0ll ? 0x7FFFFFF0u : (uint32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)b, 0x00020000);
}

template <int NT>
struct B8Stage {
    uint8_t a[kB8BM * kB8RowStride];
    uint8_t b[64 * NT * kB8RowStride];
    float xs[kB8Threads];    // token scale of row (i & 127), written by every thread
};

template <int NT>
struct B8Regs {
    u32x4 a[2];        // 128 rows x 128 bytes = 1024 chunks, 2 per thread
    u32x4 b[NT];       // 64*NT rows x 128 bytes, NT per thread
    float xs;          // the token scale of row (tid & 127)
    float g[NT];       // grid scale of each 32-column tile of this wave (uniform)
};

template <int NT>
__global__ __launch_bounds__(kB8Threads) void e4m3_blk_gemm_kernel(const uint8_t *__restrict__ w,
                                                                 const float *__restrict__ grid,
                                                                 const uint8_t *__restrict__ xq,
                                                                 const float *__restrict__ xs,
                                                                 float *__restrict__ y, int m, int k, int n) {
    constexpr int BN = 64 * NT;
    // NT >= 3: partials in [weight row][token] layout, three in flight (see
    // compute_stage); NT = 2 keeps [token][weight row] and two partials,
    // which measured faster there (33.4 against 36.3 us at m=512, K=4096,
    // N=4096; both bitwise the same).
    constexpr bool kSwap = NT >= 3;
    __shared__ __attribute__((aligned(16))) B8Stage<NT> st[2];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int n0 = blockIdx.x * BN;
    const int m0 = blockIdx.y * kB8BM;
    const int nstage = (k + kB8KB - 1) / kB8KB;   // = ceil(k/128) grid columns; the last may be short
    const int nbn = (n + 127) / 128;     // grid rows

    const __amdgpu_buffer_rsrc_t rA = b8_rsrc(xq + (int64_t)m0 * k, (int64_t)(m - m0) * k);
    const __amdgpu_buffer_rsrc_t rB = b8_rsrc(w + (int64_t)n0 * k, (int64_t)(n - n0) * k);
    const __amdgpu_buffer_rsrc_t rS = b8_rsrc(xs + (int64_t)m0 * nstage, (int64_t)(m - m0) * nstage * 4);

    // grid rows of this wave's 32-column tiles; a tile past n reads the last
    // grid row (its outputs are not stored)
    const float *gcol[NT];
#pragma unroll
    for (int j = 0; j < NT; j++) {
        const int cb = min((n0 + wn * 32 * NT + 32 * j) >> 7, nbn - 1);
        gcol[j] = grid + (int64_t)cb * nstage;
    }

    const uint32_t goff = (uint32_t)((tid >> 3) * k + 16 * (tid & 7));
    const uint32_t grow64 = (uint32_t)(64 * k);
    const uint32_t soff = (uint32_t)((tid & 127) * nstage * 4);
    auto load_stage = [&](B8Regs<NT> &R, int kc) {
        const int so = kc * kB8KB;
        // A 16-byte chunk past k (only in a short last stage) would read the
        // next row: its offset is moved past the resource, so it reads zeros
        // (0x7FFFFFF0 plus any stage offset stays below 2^32).
        const bool in = so + 16 * (tid & 7) < k;
#pragma unroll
        for (int s = 0; s < 2; s++)
            R.a[s] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(rA, in ? goff + s * grow64 : 0x7FFFFFF0u, so, 0));
#pragma unroll
        for (int s = 0; s < NT; s++)
            R.b[s] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(rB, in ? goff + s * grow64 : 0x7FFFFFF0u, so, 0));
        R.xs = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rS, soff, kc * 4, 0));
#pragma unroll
        for (int j = 0; j < NT; j++) R.g[j] = gcol[j][kc];
    };
    const int lds_off = (tid >> 3) * kB8RowStride + 16 * (tid & 7);
    float G0[NT], G1[NT];   // grid scales of the stage held in st[0] / st[1]
    auto store_stage = [&](B8Stage<NT> &S, const B8Regs<NT> &R, float (&G)[NT]) {
#pragma unroll
        for (int s = 0; s < 2; s++)
            *reinterpret_cast<u32x4 *>(S.a + lds_off + s * 64 * kB8RowStride) = R.a[s];
#pragma unroll
        for (int s = 0; s < NT; s++)
            *reinterpret_cast<u32x4 *>(S.b + lds_off + s * 64 * kB8RowStride) = R.b[s];
        S.xs[tid] = R.xs;
#pragma unroll
        for (int j = 0; j < NT; j++) G[j] = R.g[j];
    };

    v16f acc[NT];
#pragma unroll
    for (int j = 0; j < NT; j++)
#pragma unroll
        for (int v = 0; v < 16; v++) acc[j][v] = 0.0f;

    const int khalf = lane >> 5;
    // Lane l supplies row l%32 of each 32-row operand tile and k values
    // 32*(l/32) .. +31 of the 64-deep step (the same k set for A and B).
    auto compute_stage = [&](const B8Stage<NT> &S, const float (&G)[NT]) {
        const uint8_t *pa = S.a + (wm * 32 + (lane & 31)) * kB8RowStride + 32 * khalf;
        const uint8_t *pb = S.b + (wn * 32 * NT + (lane & 31)) * kB8RowStride + 32 * khalf;
        auto ld8 = [](const uint8_t *p) {
            const u32x4 lo = *reinterpret_cast<const u32x4 *>(p);
            const u32x4 hi = *reinterpret_cast<const u32x4 *>(p + 16);
            return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        };
        const v8i a0 = ld8(pa), a1 = ld8(pa + 64);
        const v16f z = {0};
        if constexpr (kSwap) {
            // The weight tile is the MFMA's A operand and the tokens its B
            // operand, so the partial is [weight row][token]: lane l holds
            // token wm*32 + l%32 and weight rows 8*(v/4) + 4*khalf + v%4 of
            // the tile, and the scale xs[t] * g of its 16 outputs is one value
            // (one multiply and 16 fma per tile instead of 16 of each).
            const float sxt = S.xs[wm * 32 + (lane & 31)];
            struct BT { v8i b0, b1; };
            auto rdt = [&](int j) -> BT { return BT{ld8(pb + j * 32 * kB8RowStride), ld8(pb + j * 32 * kB8RowStride + 64)}; };
            // The pair of MFMAs is issued at raised wave priority, so that
            // the other wave of the SIMD, busy with its fold, does not delay
            // their issue (interleaved at m=512, K=4096: N=20480 65.8 ->
            // 63.3 us, N=16384 57.0 -> 56.4; bitwise the same results).
            auto part = [&](const BT &b) {
                __builtin_amdgcn_s_setprio(1);
                v16f P = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b.b0, a0, z, 0, 0, 0, 127, 0, 127);
                P = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b.b1, a1, P, 0, 0, 0, 127, 0, 127);
                __builtin_amdgcn_s_setprio(0);
                return P;
            };
            // Three partial sets, indexed at compile time: tiles j+1 and j+2
            // are on the matrix cores while tile j is folded; the operands of
            // tile j+3 are read from LDS meanwhile.
            v16f P[3];
            BT bn = rdt(0);
            P[0] = part(bn);
            bn = rdt(1);
            P[1] = part(bn);
            if (2 < NT) bn = rdt(2);
#pragma unroll
            for (int j = 0; j < NT; j++) {
                if (j + 2 < NT) {
                    const BT cur = bn;
                    if (j + 3 < NT) bn = rdt(j + 3);
                    P[(j + 2) % 3] = part(cur);
                }
                const float sj = sxt * G[j];
#pragma unroll
                for (int v = 0; v < 16; v++) acc[j][v] = __builtin_fmaf(P[j % 3][v], sj, acc[j][v]);
            }
        } else {
            // token scales of the 16 output rows of this lane: rows
            // wm*32 + 8*(v/4) + 4*khalf + v%4, four consecutive per float4
            float sx[16];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float4 q = *reinterpret_cast<const float4 *>(S.xs + wm * 32 + 8 * i + 4 * khalf);
                sx[4 * i + 0] = q.x;
                sx[4 * i + 1] = q.y;
                sx[4 * i + 2] = q.z;
                sx[4 * i + 3] = q.w;
            }
            auto part = [&](int j) {
                const v8i b0 = ld8(pb + j * 32 * kB8RowStride), b1 = ld8(pb + j * 32 * kB8RowStride + 64);
                v16f P = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, b0, z, 0, 0, 0, 127, 0, 127);
                return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, b1, P, 0, 0, 0, 127, 0, 127);
            };
            // two partial sets, indexed at compile time: tile j+1's MFMAs are
            // issued before tile j is folded, with no register copies between
            v16f P[2];
            P[0] = part(0);
#pragma unroll
            for (int j = 0; j < NT; j++) {
                if (j + 1 < NT) P[(j + 1) & 1] = part(j + 1);
#pragma unroll
                for (int v = 0; v < 16; v++) acc[j][v] = __builtin_fmaf(P[j & 1][v], sx[v] * G[j], acc[j][v]);
            }
        }
    };

    B8Regs<NT> R0, R1;
    const int last = nstage - 1;
    load_stage(R0, 0);
    load_stage(R1, min(1, last));
    store_stage(st[0], R0, G0);
    __syncthreads();
    int kc = 0;
#pragma unroll 1
    for (; kc + 1 < nstage; kc += 2) {
        load_stage(R0, min(kc + 2, last));
        compute_stage(st[0], G0);
        store_stage(st[1], R1, G1);
        __syncthreads();
        load_stage(R1, min(kc + 3, last));
        compute_stage(st[1], G1);
        store_stage(st[0], R0, G0);
        __syncthreads();
    }
    if (kc < nstage) compute_stage(st[0], G0);

    if constexpr (kSwap) {
        // Output (token t, weight rows r..r+3) as one 16-byte store where the
        // four rows are in range and the address 16-byte aligned, else one
        // float each.
        const int t = m0 + wm * 32 + (lane & 31);
        if (t < m) {
            float *yt = y + (int64_t)t * n;
            const bool vec = (n & 3) == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0;
#pragma unroll
            for (int j = 0; j < NT; j++) {
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    const int r = n0 + wn * 32 * NT + j * 32 + 8 * g + 4 * khalf;
                    if (vec && r + 3 < n) {
                        *reinterpret_cast<float4 *>(yt + r) =
                            make_float4(acc[j][4 * g], acc[j][4 * g + 1], acc[j][4 * g + 2], acc[j][4 * g + 3]);
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; i++)
                            if (r + i < n) yt[r + i] = acc[j][4 * g + i];
                    }
                }
            }
        }
    } else {
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
}

// The tile width (NT) that needs the fewest rounds of workgroups over the
// CUs, weighting each round by its width; ties go to the wider tile.
static int b8_pick_nt(int m, int n, int cus) {
    int best = 5;
    int64_t best_cost = -1;
    for (int nt = 5; nt >= 2; nt--) {
        const int64_t tiles = (int64_t)((m + kB8BM - 1) / kB8BM) * ((n + 64 * nt - 1) / (64 * nt));
        const int64_t cost = (tiles + cus - 1) / cus * nt;
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best = nt;
        }
    }
    return best;
}

template <int NT>
static int launch_b8(const uint8_t *w, const float *grid, const uint8_t *xq, const float *xs, float *y, int m, int k,
                     int n, hipStream_t s) {
    dim3 g((n + 64 * NT - 1) / (64 * NT), (m + kB8BM - 1) / kB8BM);
    if (g.y > 65535) return BQM_EUNSUPPORTED;
    hipLaunchKernelGGL(e4m3_blk_gemm_kernel<NT>, g, dim3(kB8Threads), 0, s, w, grid, xq, xs, y, m, k, n);
    return launch_status();
}

}  // namespace bqm

extern "C" int bqm_e4m3_nan_count(const uint8_t *w, int64_t count, unsigned long long *nan_count, void *stream) {
    using namespace bqm;
    if (!w || !nan_count) return BQM_EINVAL;
    if (count < 1) return BQM_EINVAL;
    if (!aligned(w, 16) || !aligned(nan_count, 8)) return BQM_EUNSUPPORTED;
    hipStream_t s = as_stream(stream);
    hipLaunchKernelGGL(e4m3_nan_zero_kernel, dim3(1), dim3(64), 0, s, nan_count);
    int rc = launch_status();
    if (rc) return rc;
    const int64_t nvec = count / 16;
    int64_t blocks = (nvec + 256 * 8 - 1) / (256 * 8);
    if (blocks > 2048) blocks = 2048;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(e4m3_nan_count_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const u32x4 *>(w), nvec, w, count, nan_count);
    return launch_status();
}

extern "C" int bqm_e4m3_blk_quantize(const float *x, uint8_t *xq, float *xs, int m, int k, void *stream) {
    using namespace bqm;
    if (!x || !xq || !xs) return BQM_EINVAL;
    if (m < 1 || k < 16) return BQM_EINVAL;
    if (k % 16 != 0) return BQM_EUNSUPPORTED;
    if (!aligned(x, 16) || !aligned(xq, 4) || !aligned(xs, 4)) return BQM_EUNSUPPORTED;
    const int kbn = (k + 127) / 128;
    const int64_t nblocks = (int64_t)m * kbn;
    const int64_t wgs = (nblocks + 7) / 8;
    if (wgs > 0x7FFFFFFF) return BQM_EUNSUPPORTED;
    hipLaunchKernelGGL(e4m3_blk_quantize_kernel, dim3((unsigned)wgs), dim3(256), 0, as_stream(stream),
                       reinterpret_cast<const float4 *>(x), nblocks, k, kbn, reinterpret_cast<unsigned *>(xq), xs);
    return launch_status();
}

extern "C" int bqm_e4m3_blk_gemm(const uint8_t *w, const float *grid, const uint8_t *xq, const float *xs, float *y,
                                 int m, int k, int n, void *stream) {
    using namespace bqm;
    if (!w || !grid || !xq || !xs || !y) return BQM_EINVAL;
    if (m < 1 || k < 16 || n < 1) return BQM_EINVAL;
    if (k % 16 != 0) return BQM_EUNSUPPORTED;
    if (!aligned(w, 16) || !aligned(xq, 16) || !aligned(grid, 4) || !aligned(xs, 4) || !aligned(y, 4))
        return BQM_EUNSUPPORTED;
    if ((int64_t)kB8BM * k > 0x7FFFFFF0ll || (int64_t)320 * k > 0x7FFFFFF0ll) return BQM_EUNSUPPORTED;
    hipStream_t s = as_stream(stream);
    switch (b8_pick_nt(m, n, device_cus())) {
        case 2: return launch_b8<2>(w, grid, xq, xs, y, m, k, n, s);
        case 3: return launch_b8<3>(w, grid, xq, xs, y, m, k, n, s);
        case 4: return launch_b8<4>(w, grid, xq, xs, y, m, k, n, s);
        default: return launch_b8<5>(w, grid, xq, xs, y, m, k, n, s);
    }
}
