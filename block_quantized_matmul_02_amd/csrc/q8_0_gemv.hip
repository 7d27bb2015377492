// Q8_0 x q8_1 decode/verify GEMV for gfx950 (m = 1..15).
//
// What it computes (memra-engine pages): y[t][r] = sum_b d_w[r][b] * d_x[t][b]
// * S[t][r][b], S the int32 dot product of a 32-block of int8 weight quants
// with the matching int8 activation quants ("accprobe_bench.rs" module doc:
// s32 per k32 folded by the two scales; "decode_kernel_census.rs", fn q8: the
// m=1 Q8_0 GEMV over rows of in_f/32*34 bytes).
//
// Design (HBM-bound: every weight byte is read exactly once):
//  * A weight row is P = K/64 "pairs" of blocks; a pair is 68 bytes = 17
//    dwords, so pairs are 4-byte aligned while single blocks are not.
//    Each row is handled by L lanes (L = next power of two >= P, at most
//    64); lane i of the row owns pairs i, i+L, ...  A wave covers G = 64/L
//    rows per row-step.
//  * A wave streams a tile of RT whole rows (<= 5 KiB) with 16-byte buffer
//    loads: slot s of lane l loads chunk 64*s + l of the tile, so every load
//    instruction reads 1 KiB of consecutive bytes.  Buffer loads check the
//    range in hardware: rows past n and unused slots read zeros, never fault.
//    Two tiles are in flight per wave (register double buffer).
//  * The tile is written unchanged into a wave-private LDS buffer and read
//    back pair by pair (17 x ds_read_b32, stride 17 dwords: conflict-free);
//    the even block's quants sit at a 2-byte offset and are realigned with
//    v_alignbit (8 ops per pair).
//  * Activations (int8 quants and d_x) are staged once per workgroup in LDS,
//    with each pair's four 16-byte chunks rotated by (pair/4) so that sixteen
//    lanes reading sixteen consecutive pairs hit distinct banks of the 64-bank
//    LDS (a rotation by pair/2 left 2-way conflicts that counters showed on
//    the m=9 GEMV; measured 2-5% faster across the sweep).
//  * Per pair and token: 16 v_dot4_i32_i8, then the two block sums are folded
//    with fma(float(S), d_w*d_x, acc).  The L per-lane partial sums of a row
//    are combined by a fixed DPP / permlane-swap butterfly.
//  * Every token's operation order is the same for any m, so an m-token call
//    reproduces single-token calls bit for bit ("decode_kernel_census.rs"
//    module doc: identical per-row FP order across decode and verify).
//  * The QX variants take the f32 activation itself: every workgroup applies
//    the q8_1 rule (the same device code as bqm_q8_1_quantize) to it while
//    its first weight tiles are in flight and writes the quants and d_x
//    straight into its LDS copy, so the quantize launch and the round trip
//    of xq/xds through memory disappear from the decode step.  Results are
//    bitwise those of bqm_q8_1_quantize followed by bqm_q8_0_gemv.
#include "bqmm_internal.h"

namespace bqm {

constexpr int kGemvThreads = 256;      // 4 waves, each streaming its own tiles
constexpr int kGemvWaves = kGemvThreads / 64;
constexpr int kSlots = 5;              // 5 x 1 KiB of loads per tile (one row of K=4096, 4352 B)
constexpr int kTileBytes = kSlots * 1024;
constexpr int kMaxPairsPerSeg = 72;    // 72 * 68 = 4896 bytes <= one tile
constexpr int kActLdsMax = 98304;      // activation bytes staged per workgroup
// Cache policy of the weight loads: non-temporal.  Every weight byte is read
// exactly once, so keeping it out of the caches frees them for the activations
// (measured: a plain 280 MB stream reads at 5.75 TB/s with the default policy
// and 6.5 TB/s non-temporal on MI355X).
constexpr int kWeightLoadPolicy = 2;

struct GemvGeom {
    int P;         // pairs per row
    int PS;        // pairs per segment (divides P, multiple of 4)
    int nseg;      // segments per row
    int L;         // lanes per row
    int Llog2;
    int J;         // pair slots per lane per row-step = ceil(PS / L)
    int G;         // rows per row-step = 64 / L
    int RT;        // rows per tile
    int RS;        // row-steps per tile = RT / G
    int CPS;       // 16-byte chunks per row segment = 68*PS/16
    int TC;        // chunks per tile = RT * CPS
    int TB;        // LDS bytes of one staged tile = 16 * TC
    int n_row_tiles;
};

// Buffer resource for raw 16-byte loads from [base, base + bytes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, kWeightLoadPolicy));
}

// Activation chunks a thread can hold in registers while the first weight
// tiles are issued (PRE variants): up to 2 x 256 chunks of 16 bytes, m*k <= 8192.
constexpr int kActPre = 2;

// The four f32 values held in a 16-byte load.  The whole vector is bit cast:
// clang lowers a bit cast of a vector-element expression to a read of the
// vector's first element.
__device__ __forceinline__ float4 as_float4(u32x4 b) {
    typedef float v4f __attribute__((ext_vector_type(4)));
    const v4f f = __builtin_bit_cast(v4f, b);
    return make_float4(f[0], f[1], f[2], f[3]);
}

// f32 activation float4s per thread a QX variant can hold in registers
// (m*k <= 8192).
constexpr int kActPreX = 8;

// PRE = activation chunks per thread loaded ahead of the tiles (0 = none):
// 16-byte chunks of xq, or with QX float4s of x.
// Most tokens whose activation operands a lane holds in registers (XR).
// Measured on the sweep shapes: holding them for 3..9 tokens costs more in
// occupancy (178..320 VGPRs) than it saves in LDS reads (m=9, 4096 -> 20480:
// 40.5 us against 36.5 us).
constexpr int kXregMaxM = 2;

// XR: every row gives a lane the same pairs (whole rows, one pair per lane:
// K <= 4096), so the lane's activation operands for all M tokens are loaded
// from LDS once and held in registers.
template <int M, bool SINGLE, int PRE, bool QX, bool XR, int WG>
__global__ __launch_bounds__(WG) void q8_0_gemv_kernel(
    const uint8_t *__restrict__ w, int64_t w_row_bytes, const int8_t *__restrict__ xq,
    const float *__restrict__ xds, const float *__restrict__ x, float *__restrict__ y, int k, int n, GemvGeom g) {
    static_assert(!QX || PRE > 0, "f32 activations are held in registers");
    static_assert(!XR || M <= kXregMaxM, "register-held activations for at most kXregMaxM tokens");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int nb = k / kQK;
    uint8_t *act_q = lds;                                  // [M][k] swizzled per pair
    float *act_d = reinterpret_cast<float *>(lds + M * k);  // [M][nb]
    const int act_bytes = (M * k + M * nb * 4 + 15) & ~15;
    // wave index as a scalar: everything derived from it (tile, segment, buffer
    // resource) is then wave-uniform and lives in SGPRs
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    // two staged tiles per wave, back to back
    uint8_t *tile0 = lds + act_bytes + wave * 2 * g.TB;
    uint8_t *tile1 = tile0 + g.TB;

    // Activations (int8 quants and d_x) are staged once per workgroup, after
    // the first weight tiles are in flight so HBM starts streaming at once.
    // Plain loads issued after the tiles' loads can only be waited for
    // together with them, so the first arithmetic would wait for every
    // tile of the first wave of requests.  The PRE variants (m*k <= 8192,
    // m*k/32 <= 256) therefore issues its activation loads into registers
    // before the tiles' loads and waits for those alone.
    const __amdgpu_buffer_rsrc_t rxq = make_rsrc(QX ? (const void *)x : (const void *)xq,
                                                 (uint32_t)(QX ? M * k * 4 : M * k));
    const __amdgpu_buffer_rsrc_t rxd = make_rsrc(xds, (uint32_t)(QX ? 0 : M * nb * 8));
    u32x4 pre_q[PRE > 0 ? PRE : 1];
    float pre_d;
    auto preload_activations = [&]() {
#pragma unroll
        for (int i = 0; i < PRE; i++)
            pre_q[i] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(rxq, (uint32_t)(threadIdx.x + WG * i) * 16u, 0, 0));
        if (!QX) pre_d = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rxd, threadIdx.x * 8u, 0, 0));
    };
    // QX: float4 number c of x (values 4c..4c+3) quantized by its 8-lane
    // group; its dword goes into the staged quants, and the group's first
    // lane writes d_x.  Groups past the activation write into this wave's
    // first tile, which is overwritten before it is read.
    auto quantize_store = [&](float4 v, int c) {
        const Q81Lane r = q8_1_block_lane(v);
        const bool valid = c < M * k / 4;
        const int t = (4 * c) / k;
        const int e = 4 * c - t * k;                 // value index inside the token
        const int cc = e >> 4, p = cc >> 2, ci = cc & 3;
        uint8_t *dq = valid ? act_q + t * k + 64 * p + 16 * ((ci + (p >> 2)) & 3) + 4 * (c & 3) : tile0 + 4 * lane;
        *reinterpret_cast<unsigned *>(dq) = r.packed;
        float *dd = (valid && (c & 7) == 0) ? act_d + t * nb + (e >> 5) : reinterpret_cast<float *>(tile0) + lane;
        *dd = r.d;
    };
    // Every preloaded value is stored unconditionally (values past the
    // activations go to this wave's first tile, which is overwritten before
    // it is read): a store behind a branch lets the compiler sink its load
    // into the branch, behind the tiles' loads.
    auto store_preloaded = [&]() {
        if (QX) {
#pragma unroll
            for (int i = 0; i < PRE; i++) {
                quantize_store(as_float4(pre_q[i]), (int)threadIdx.x + WG * i);
            }
            __syncthreads();
            return;
        }
        const int chunks = M * k / 16;
#pragma unroll
        for (int i = 0; i < PRE; i++) {
            const int c = threadIdx.x + WG * i;
            const int t = c / (k / 16);
            const int cc = c - t * (k / 16);
            const int p = cc >> 2, ci = cc & 3;
            uint8_t *dst = c < chunks ? act_q + t * k + 64 * p + 16 * ((ci + (p >> 2)) & 3) : tile0 + 16 * lane;
            *reinterpret_cast<u32x4 *>(dst) = pre_q[i];
        }
        float *dd = (int)threadIdx.x < M * nb ? act_d + threadIdx.x : reinterpret_cast<float *>(tile0) + lane;
        *dd = pre_d;
        __syncthreads();
    };
    auto stage_activations = [&]() {
        const int chunks = M * k / 16;
        for (int c = threadIdx.x; c < chunks; c += WG) {
            int t = c / (k / 16);
            int cc = c - t * (k / 16);
            int p = cc >> 2, ci = cc & 3;
            u32x4 v = *reinterpret_cast<const u32x4 *>(xq + (int64_t)t * k + 16 * cc);
            int dst = t * k + 64 * p + 16 * ((ci + (p >> 2)) & 3);
            *reinterpret_cast<u32x4 *>(act_q + dst) = v;
        }
        for (int c = threadIdx.x; c < M * nb; c += WG) act_d[c] = xds[2 * c];
        __syncthreads();
    };

    const int nwaves = gridDim.x * (WG / 64);
    const int wid = blockIdx.x * (WG / 64) + wave;
    // Waves without a tile still take part in the workgroup barrier.
    const int my_tiles = wid < g.n_row_tiles ? (g.n_row_tiles - 1 - wid) / nwaves + 1 : 0;
    const int Q = my_tiles * g.nseg;   // work items of this wave: (row tile, segment)

    // Per-slot byte offset of this lane's chunk inside a tile (fixed for all tiles).
    uint32_t voff[kSlots];
#pragma unroll
    for (int s = 0; s < kSlots; s++) {
        int c = 64 * s + lane;
        if (c < g.TC) {
            int r = c / g.CPS;
            int col = c - r * g.CPS;
            voff[s] = (uint32_t)(r * w_row_bytes + 16 * col);
        } else {
            voff[s] = 0xFFFFFFF0u;   // past num_records: the load returns zeros
        }
    }

    // Issue the loads of work item q.  Items past the wave's last one get an
    // empty resource: the loads return zeros without touching memory.
    auto issue = [&](u32x4 (&buf)[kSlots], int q) {
        int rt = wid + nwaves * (q / g.nseg);
        int sg = q - (q / g.nseg) * g.nseg;
        int64_t row0 = (int64_t)rt * g.RT;
        const uint8_t *base = w + row0 * w_row_bytes + (int64_t)sg * g.PS * 68;
        int64_t rem = (int64_t)(n - row0) * w_row_bytes - (int64_t)sg * g.PS * 68;
        uint32_t bytes = q >= Q ? 0u : (rem > 0x7FFFFFF0ll ? 0x7FFFFFF0u : (uint32_t)rem);
        if (q >= Q) base = w;
        __amdgpu_buffer_rsrc_t rs = make_rsrc(base, bytes);
#pragma unroll
        for (int s = 0; s < kSlots; s++) buf[s] = buf_load16(rs, voff[s]);
    };

    auto stage = [&](const u32x4 (&buf)[kSlots], uint8_t *tl) {
        // Wave-private buffer; LDS accesses of one wave complete in order, so the
        // previous tile's reads are done before these writes land.  Chunks past
        // the tile (zeros) are not written.
#pragma unroll
        for (int s = 0; s < kSlots; s++)
            if (64 * s + lane < g.TC) *reinterpret_cast<u32x4 *>(tl + 1024 * s + 16 * lane) = buf[s];
    };

    const int li = lane & (g.L - 1);     // lane index inside its row
    const int gr = lane >> g.Llog2;      // row inside the row-step
    float acc[M];
#pragma unroll
    for (int t = 0; t < M; t++) acc[t] = 0.0f;

    // Activation operands of one pair and token: the pair's four 16-byte
    // chunks of int8 quants (undoing the rotation of the staged copy) and the
    // two block scales d_x.
    struct ActPair {
        v4i x[4];
        float2 dx;
    };
    auto load_act = [&](int t, int p) {
        ActPair r;
        const uint8_t *ap = act_q + t * k + 64 * p;
        const int rot = (p >> 2) & 3;
#pragma unroll
        for (int c = 0; c < 4; c++) r.x[c] = *reinterpret_cast<const v4i *>(ap + 16 * ((c + rot) & 3));
        r.dx = *reinterpret_cast<const float2 *>(act_d + t * nb + 2 * p);
        return r;
    };

    // Register copy of this lane's activation pair, filled once the
    // activations are staged (used when every row gives the lane the same
    // pair; see compute).
    ActPair xreg[XR ? M : 1];

    // One pair (two blocks) of tile row rl, pair pl of the segment, for every
    // token: a[t] += d_w*d_x*S for both blocks.  The activation operands come
    // from LDS, or from xr when the lane's pair is the same for every row.
    auto pair_dot = [&](const uint8_t *tl, int rl, int pl, int sg, float (&a)[M], const ActPair *xr) {
        const uint32_t *pw = reinterpret_cast<const uint32_t *>(tl + rl * (68 * g.PS) + 68 * pl);
        uint32_t dw[17];
#pragma unroll
        for (int d = 0; d < 17; d++) dw[d] = pw[d];
        int qa[8], qb[8];
#pragma unroll
        for (int d = 0; d < 8; d++) {
            qa[d] = (int)__builtin_amdgcn_alignbit(dw[d + 1], dw[d], 16u);
            qb[d] = (int)dw[9 + d];
        }
        const float da = half_bits_to_float(dw[0]);
        const float db = half_bits_to_float(dw[8] >> 16);
        const int p = sg * g.PS + pl;   // pair index in the row
#pragma unroll
        for (int t = 0; t < M; t++) {
            const ActPair x = xr ? xr[t] : load_act(t, p);
            int sa = 0, sb = 0;
#pragma unroll
            for (int d = 0; d < 4; d++) sa = __builtin_amdgcn_sdot4(qa[d], x.x[0][d], sa, false);
#pragma unroll
            for (int d = 0; d < 4; d++) sa = __builtin_amdgcn_sdot4(qa[4 + d], x.x[1][d], sa, false);
#pragma unroll
            for (int d = 0; d < 4; d++) sb = __builtin_amdgcn_sdot4(qb[d], x.x[2][d], sb, false);
#pragma unroll
            for (int d = 0; d < 4; d++) sb = __builtin_amdgcn_sdot4(qb[4 + d], x.x[3][d], sb, false);
            const float sca = da * x.dx.x;
            const float scb = db * x.dx.y;
            a[t] = __builtin_fmaf((float)sa, sca, a[t]);
            a[t] = __builtin_fmaf((float)sb, scb, a[t]);
        }
    };

    // Sum the L per-lane partials of a row and store y (lane 0 of the row).
    auto reduce_store = [&](float (&a)[M], int row) {
#pragma unroll
        for (int t = 0; t < M; t++) {
            float v = a[t];
            v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
            v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
            if (g.L >= 8) v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
            if (g.L >= 16) v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
            if (g.L >= 32) v = swap16_sum(v);
            if (g.L >= 64) v = swap32_sum(v);
            if (li == 0 && row < n) y[(int64_t)t * n + row] = v;
        }
    };

    // Work item q, staged in tile tl.
    auto compute = [&](int q, const uint8_t *tl) {
        const int rt = wid + nwaves * (q / g.nseg);
        const int sg = q - (q / g.nseg) * g.nseg;
        const int row0 = rt * g.RT;
        if (g.nseg == 1) {
            // Whole rows.
            for (int rs = 0; rs < g.RS; rs++) {
                const int rl = rs * g.G + gr;
                float a0[M];
#pragma unroll
                for (int t = 0; t < M; t++) a0[t] = 0.0f;
                for (int j = 0; j < g.J; j++) {
                    const int pl = li + g.L * j;
                    if (pl < g.PS) pair_dot(tl, rl, pl, 0, a0, XR ? xreg : nullptr);
                }
                reduce_store(a0, row0 + rl);
            }
        } else {
            // One segment of one row (one row per tile); the accumulators carry
            // over the row's segments, which this wave takes in order.
            if (sg == 0) {
#pragma unroll
                for (int t = 0; t < M; t++) acc[t] = 0.0f;
            }
            for (int j = 0; j < g.J; j++) {
                const int pl = li + g.L * j;
                if (pl < g.PS) pair_dot(tl, gr, pl, sg, acc, nullptr);
            }
            if (sg == g.nseg - 1) reduce_store(acc, row0 + gr);
        }
    };

    // Items q (tile t0) and q+1 (tile t1, present when two) when every row
    // gives a lane the same pair (whole rows, one pair per lane: K <= 4096)
    // and m <= 2: the activation operands sit in registers, and the two tiles
    // run as two independent chains so the LDS and dot-product latencies of
    // one overlap the other's.
    constexpr bool fast = XR && M <= 2;
    auto compute_pair_fast = [&](int q, const uint8_t *t0, const uint8_t *t1, bool two) {
        const int row0 = (wid + nwaves * q) * g.RT;
        const int row1 = (wid + nwaves * (q + 1)) * g.RT;
        for (int rs = 0; rs < g.RS; rs++) {
            const int rl = rs * g.G + gr;
            float a0[M], a1[M];
#pragma unroll
            for (int t = 0; t < M; t++) a0[t] = a1[t] = 0.0f;
            if (li < g.PS) {
                pair_dot(t0, rl, li, 0, a0, xreg);
                pair_dot(t1, rl, li, 0, a1, xreg);
            }
            reduce_store(a0, row0 + rl);
            if (two) reduce_store(a1, row1 + rl);
        }
    };

    auto load_xreg = [&]() {
        if (XR && li < g.PS) {
#pragma unroll
            for (int t = 0; t < (XR ? M : 1); t++) xreg[t] = load_act(t, li);
        }
    };

    u32x4 bufA[kSlots], bufB[kSlots];
    if (SINGLE) {
        // Launched with at most one item per wave: no pipeline (every wave
        // still stages the activations, which ends in a workgroup barrier).
        if (PRE) preload_activations();
        if (Q == 1) issue(bufA, 0);
        if (PRE) store_preloaded();
        else stage_activations();
        load_xreg();
        if (Q == 1) {
            stage(bufA, tile0);
            if (fast) compute_pair_fast(0, tile0, tile0, false);
            else compute(0, tile0);
        }
        return;
    }
    // Two items in flight, each staged into its own LDS tile before either is
    // computed, so both refills are issued before the arithmetic starts and no
    // buffer sits idle behind it.  Every fill in the loop is issued
    // unconditionally (a refill past the last item is empty), so the compiler
    // knows that the other buffer's loads are still in flight when a buffer is
    // staged and waits only for the older loads; a fill behind a branch would
    // make it wait for all of them.  The last one or two items are drained
    // after the loop.
    if (PRE) preload_activations();
    issue(bufA, 0);
    issue(bufB, 1);
    if (PRE) store_preloaded();
    else stage_activations();
    load_xreg();
    int q = 0;
    for (; q + 2 < Q; q += 2) {
        stage(bufA, tile0);
        issue(bufA, q + 2);
        stage(bufB, tile1);
        issue(bufB, q + 3);
        if (fast) {
            compute_pair_fast(q, tile0, tile1, true);
        } else {
            compute(q, tile0);
            compute(q + 1, tile1);
        }
    }
    stage(bufA, tile0);
    stage(bufB, tile1);
    if (fast) {
        compute_pair_fast(q, tile0, tile1, q + 1 < Q);
    } else {
        compute(q, tile0);
        if (q + 1 < Q) compute(q + 1, tile1);
    }
}

static bool make_geom(int k, int n, int64_t w_row_bytes, GemvGeom &g) {
    g.P = k / 64;
    g.PS = g.P;
    if (g.P > kMaxPairsPerSeg) {
        g.PS = 4;
        for (int d = kMaxPairsPerSeg; d >= 4; d -= 4)
            if (g.P % d == 0) { g.PS = d; break; }
    }
    g.nseg = g.P / g.PS;
    int L = 4;
    while (L < g.P && L < 64) L *= 2;
    g.L = L;
    g.Llog2 = __builtin_ctz(L);
    g.J = (g.PS + L - 1) / L;
    g.G = 64 / L;
    int seg_bytes = 68 * g.PS;
    g.CPS = seg_bytes / 16;
    if (g.nseg > 1) {
        g.RT = 1;   // accumulators of one row persist across the segments
    } else {
        int steps = kTileBytes / (g.G * seg_bytes);
        if (steps < 1) return false;
        if (steps > 8) steps = 8;
        g.RT = g.G * steps;
    }
    g.RS = g.RT / g.G;
    g.TC = g.RT * g.CPS;
    g.TB = 16 * g.TC;
    if (g.TC > kSlots * 64) return false;
    g.n_row_tiles = (n + g.RT - 1) / g.RT;
    (void)w_row_bytes;
    return true;
}

template <int M, bool SINGLE, int PRE, bool QX, bool XR, int WG>
static int launch_variant(const uint8_t *w, int64_t w_row_bytes, const int8_t *xq, const float *xds, const float *x,
                          float *y, int k, int n, const GemvGeom &g, int grid, int lds_bytes, hipStream_t stream) {
    static LaunchCache cache;
    const int rc = raise_lds_limit(cache, reinterpret_cast<const void *>(&q8_0_gemv_kernel<M, SINGLE, PRE, QX, XR, WG>),
                                   160 * 1024);
    if (rc != BQM_OK) return rc;
    hipLaunchKernelGGL((q8_0_gemv_kernel<M, SINGLE, PRE, QX, XR, WG>), dim3(grid), dim3(WG), lds_bytes, stream, w,
                       w_row_bytes, xq, xds, x, y, k, n, g);
    return launch_status();
}

// Resident workgroups per CU of the pipelined variant (registers and LDS),
// at most 4.
template <int M, int PRE, bool QX, bool XR, int WG>
static int gemv_per_cu(int lds_bytes) {
    static LaunchCache cache;
    const void *fn = reinterpret_cast<const void *>(&q8_0_gemv_kernel<M, false, PRE, QX, XR, WG>);
    if (raise_lds_limit(cache, fn, 160 * 1024) != BQM_OK) return 1;   // allow up to 160 KiB before asking
    return blocks_per_cu(cache, fn, WG, lds_bytes, 4);
}

// Grid size and the pipelined / single-item choice, then the launch.
template <int M, int PRE, bool QX, bool XR, int WG>
static int launch_sized(const uint8_t *w, int64_t w_row_bytes, const int8_t *xq, const float *xds, const float *x,
                        float *y, int k, int n, const GemvGeom &g, int lds_bytes, hipStream_t stream) {
    const int cus = device_cus();
    int per_cu = gemv_per_cu<M, PRE, QX, XR, WG>(lds_bytes);
    if (QX) {
        // Every workgroup of the one-launch step reads and quantizes the whole
        // f32 activation (16 KiB at K=4096), so at four workgroups per CU a
        // 17.8 MB weight matrix came with 16 MB of activation reads.  One
        // workgroup per CU below 48 MB of weights, two below 128 MB, no cap
        // above (measured, m=1: 4096->4096 8.7 -> 6.6 us, 1280->4096 4.7 ->
        // 3.8, 4096->20480 17.0 -> 16.2; the 280 MB head runs 0.5 us faster
        // with four; bitwise the same results).
        const int64_t wbytes = (int64_t)n * w_row_bytes;
        const int cap = wbytes < (48ll << 20) ? 1 : wbytes < (128ll << 20) ? 2 : 4;
        if (per_cu > cap) per_cu = cap;
    }
    int want = (g.n_row_tiles + (WG / 64) - 1) / (WG / 64);
    int grid = cus * per_cu;
    if (want < grid) grid = want;
    // as few workgroups as give every wave the same number of items (the
    // last items of the longest waves otherwise run alone; measured 0.5 us
    // on the 4096 -> 64448 head)
    const int64_t tpw = ((int64_t)g.n_row_tiles + (int64_t)grid * (WG / 64) - 1) / ((int64_t)grid * (WG / 64));
    grid = (int)(((int64_t)g.n_row_tiles + tpw * (WG / 64) - 1) / (tpw * (WG / 64)));
    // every wave holds at most one item: the variant without the pipeline
    const bool single = (int64_t)g.n_row_tiles * g.nseg <= (int64_t)grid * (WG / 64);
    if (single)
        return launch_variant<M, true, PRE, QX, XR, WG>(w, w_row_bytes, xq, xds, x, y, k, n, g, grid, lds_bytes, stream);
    return launch_variant<M, false, PRE, QX, XR, WG>(w, w_row_bytes, xq, xds, x, y, k, n, g, grid, lds_bytes, stream);
}

template <int M, int PRE, bool QX, int WG = kGemvThreads>
static int launch_xr(const uint8_t *w, int64_t w_row_bytes, const int8_t *xq, const float *xds, const float *x,
                     float *y, int k, int n, const GemvGeom &g, int lds_bytes, hipStream_t stream) {
    if constexpr (M <= kXregMaxM) {
        if (g.nseg == 1 && g.J == 1)
            return launch_sized<M, PRE, QX, true, WG>(w, w_row_bytes, xq, xds, x, y, k, n, g, lds_bytes, stream);
    }
    return launch_sized<M, PRE, QX, false, WG>(w, w_row_bytes, xq, xds, x, y, k, n, g, lds_bytes, stream);
}

template <int M>
static int launch_gemv(const uint8_t *w, int64_t w_row_bytes, const int8_t *xq, const float *xds, const float *x,
                       float *y, int k, int n, const GemvGeom &g, hipStream_t stream) {
    const int nb = k / kQK;
    const int act_bytes = (M * k + M * nb * 4 + 15) & ~15;
    const int lds_bytes = act_bytes + kGemvWaves * 2 * g.TB;
    if constexpr (M <= 2) {
        const int64_t wbytes16 = (int64_t)n * w_row_bytes;
        if (x && (wbytes16 < (48ll << 20) || wbytes16 >= (128ll << 20)) && g.RT == 1 && n >= 16 * device_cus()) {
            // One 16-wave workgroup per CU for the one-launch step, where a
            // tile is one row and every CU gets at least 16 rows: all of a
            // CU's rows are in flight at once while the activation is
            // quantized once per CU instead of once per 4-wave workgroup.
            // Measured in a graph, bitwise the same: m=1 4096->4096 6.77 ->
            // 6.58 us, 4096->5152 7.68 -> 7.49, m=2 4096->4096 8.68 -> 7.40;
            // the 4096->64448 head m=1 44.25 -> 43.79 and 44.17 -> 43.95, m=2
            // 47.31 -> 45.27.  Not taken between 48 and 128 MB (4096->20480:
            // 15.93 -> 16.34, where 4-wave workgroups run two per CU) nor at
            // K=1280, two rows per tile (3.84 -> 4.71).
            constexpr int WG = 1024;
            const int lds16 = act_bytes + (WG / 64) * 2 * g.TB;
            const int f4 = (M * k / 4 + WG - 1) / WG;
            if (lds16 <= 160 * 1024) {
                if (f4 <= 1) return launch_xr<M, 1, true, WG>(w, w_row_bytes, xq, xds, x, y, k, n, g, lds16, stream);
                return launch_xr<M, 2, true, WG>(w, w_row_bytes, xq, xds, x, y, k, n, g, lds16, stream);
            }
        }
        if (x) {
            // f32 activations held in registers, 1, 2, 4 or 8 float4s per
            // thread (the entry point admits m <= 2, m*k <= 8192)
            const int f4 = (M * k / 4 + kGemvThreads - 1) / kGemvThreads;
            if (f4 <= 1) return launch_xr<M, 1, true>(w, w_row_bytes, xq, xds, x, y, k, n, g, lds_bytes, stream);
            if (f4 <= 2) return launch_xr<M, 2, true>(w, w_row_bytes, xq, xds, x, y, k, n, g, lds_bytes, stream);
            if (f4 <= 4) return launch_xr<M, 4, true>(w, w_row_bytes, xq, xds, x, y, k, n, g, lds_bytes, stream);
            return launch_xr<M, 8, true>(w, w_row_bytes, xq, xds, x, y, k, n, g, lds_bytes, stream);
        }
    }
    // the activations fit in the registers of the workgroup's threads
    // (PRE variants are built for m <= 2, the decode sizes)
    const int pre_chunks = (M * k / 16 + kGemvThreads - 1) / kGemvThreads;
    const int pre = (M <= 2 && pre_chunks <= kActPre && M * nb <= kGemvThreads) ? pre_chunks : 0;
    if (pre == 1) return launch_xr<M, (M <= 2 ? 1 : 0), false>(w, w_row_bytes, xq, xds, x, y, k, n, g, lds_bytes, stream);
    if (pre == 2) return launch_xr<M, (M <= 2 ? 2 : 0), false>(w, w_row_bytes, xq, xds, x, y, k, n, g, lds_bytes, stream);
    return launch_xr<M, 0, false>(w, w_row_bytes, xq, xds, x, y, k, n, g, lds_bytes, stream);
}

// Shared checks and the dispatch on m; x == nullptr selects the q8_1 inputs.
static int gemv_entry(const uint8_t *w, int64_t w_row_bytes, const int8_t *xq, const float *xds, const float *x,
                      float *y, int m, int k, int n, void *stream) {
    if (m < 1 || m > BQM_GEMV_MAX_M || k < 256 || n < 1) return BQM_EINVAL;
    if (k % 256 != 0) return BQM_EUNSUPPORTED;
    // in-kernel quantization is for decode: every workgroup quantizes the
    // whole activation, which only pays while it fits in registers
    if (x && (m > 2 || m * k > kActPreX * kGemvThreads * 4)) return BQM_EUNSUPPORTED;
    if (w_row_bytes < (int64_t)(k / kQK) * kQ80Bytes || w_row_bytes % 16 != 0) return BQM_EUNSUPPORTED;
    if (!aligned(w, 16) || !aligned(y, 4)) return BQM_EUNSUPPORTED;
    if (x ? !aligned(x, 16) : (!aligned(xq, 16) || !aligned(xds, 8))) return BQM_EUNSUPPORTED;
    if ((int64_t)m * k * 9 / 8 > kActLdsMax) return BQM_EUNSUPPORTED;
    if (w_row_bytes > 0x7FFFFFFF / 64) return BQM_EUNSUPPORTED;
    // 3..15 tokens on the matrix cores (same per-row order as below)
    if (!x && gemv_mma_applies(m, k, n)) return gemv_mma(w, w_row_bytes, xq, xds, y, m, k, n, as_stream(stream));
    GemvGeom g;
    if (!make_geom(k, n, w_row_bytes, g)) return BQM_EUNSUPPORTED;
    // the per-slot offsets r*w_row_bytes + 16*col must fit in 32 bits
    if ((int64_t)g.RT * w_row_bytes > 0x7FFFFFF0ll) return BQM_EUNSUPPORTED;
    hipStream_t s = as_stream(stream);
    switch (m) {
        case 1: return launch_gemv<1>(w, w_row_bytes, xq, xds, x, y, k, n, g, s);
        case 2: return launch_gemv<2>(w, w_row_bytes, xq, xds, x, y, k, n, g, s);
        case 3: return launch_gemv<3>(w, w_row_bytes, xq, xds, x, y, k, n, g, s);
        case 4: return launch_gemv<4>(w, w_row_bytes, xq, xds, x, y, k, n, g, s);
        case 5: return launch_gemv<5>(w, w_row_bytes, xq, xds, x, y, k, n, g, s);
        case 6: return launch_gemv<6>(w, w_row_bytes, xq, xds, x, y, k, n, g, s);
        case 7: return launch_gemv<7>(w, w_row_bytes, xq, xds, x, y, k, n, g, s);
        case 8: return launch_gemv<8>(w, w_row_bytes, xq, xds, x, y, k, n, g, s);
        case 9: return launch_gemv<9>(w, w_row_bytes, xq, xds, x, y, k, n, g, s);
        case 10: return launch_gemv<10>(w, w_row_bytes, xq, xds, x, y, k, n, g, s);
        case 11: return launch_gemv<11>(w, w_row_bytes, xq, xds, x, y, k, n, g, s);
        case 12: return launch_gemv<12>(w, w_row_bytes, xq, xds, x, y, k, n, g, s);
        case 13: return launch_gemv<13>(w, w_row_bytes, xq, xds, x, y, k, n, g, s);
        case 14: return launch_gemv<14>(w, w_row_bytes, xq, xds, x, y, k, n, g, s);
        case 15: return launch_gemv<15>(w, w_row_bytes, xq, xds, x, y, k, n, g, s);
        default: return BQM_EINVAL;
    }
}

}  // namespace bqm

extern "C" int bqm_q8_0_gemv(const uint8_t *w, int64_t w_row_bytes, const int8_t *xq, const float *xds, float *y,
                             int m, int k, int n, void *stream) {
    if (!w || !xq || !xds || !y) return BQM_EINVAL;
    return bqm::gemv_entry(w, w_row_bytes, xq, xds, nullptr, y, m, k, n, stream);
}

extern "C" int bqm_q8_0_gemv_f32(const uint8_t *w, int64_t w_row_bytes, const float *x, float *y, int m, int k, int n,
                                 void *stream) {
    if (!w || !x || !y) return BQM_EINVAL;
    return bqm::gemv_entry(w, w_row_bytes, nullptr, nullptr, x, y, m, k, n, stream);
}
