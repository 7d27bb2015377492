// Q8_0 x q8_1 verify GEMV on the int8 matrix cores (3..15 tokens, K <= 4096).
//
// What it computes is the GEMV's: y[t][r] = sum_b d_w[r][b] * d_x[t][b] *
// S[t][r][b], S the int32 dot product of one 32-block ("accprobe_bench.rs"
// module doc: s32 per k32 folded by the two scales), with exactly the per-row
// floating-point order of the 1- and 2-token kernel, so a verify batch
// reproduces single-token decode bit for bit ("decode_kernel_census.rs" module
// doc: identical per-row FP order across decode and verify).
//
// Why matrix cores: with 3..15 tokens the dot4 kernel spends its time reading
// every token's activation operands from LDS once per weight row (36 bytes per
// token, row and block) and on 8 v_dot4 per token and pair.  Here one
// v_mfma_i32_16x16x32_i8 gives the 32-value block sums of 16 weight rows x 16
// tokens (K = 32 is one Q8_0 block), so the activations are read once per 16
// rows and the VALU work per output is the fold alone.  The kernel stays
// HBM-bound: every weight byte is read once.
//
// The order it must reproduce.  A row is P = K/64 block pairs (68 bytes,
// 4-byte aligned).  The dot4 kernel gives pair p of a row to lane p of the
// row (P <= 64 lanes, one pair each), where
//     leaf_p = fma(float(S_odd), d_w*d_x, fma(float(S_even), d_w*d_x, +0)),
// and sums the leaves by a butterfly: a perfect binary tree over the pair
// index, missing leaves (p >= P, up to the next power of two) being +0.
// A leaf is never -0 (its first fma adds +0 to a product; a sum of values that
// are not -0 is not -0), so x + (+0) == x for every value that occurs, and
// subtrees made only of missing leaves can be dropped.  Here:
//  * a row is cut into chunks of 8 pairs; one wave computes the 8 leaves of a
//    chunk for 16 rows x 16 tokens and their subtree ((l0+l1)+(l2+l3)) +
//    ((l4+l5)+(l6+l7)), in registers;
//  * the chunks of a row group go to different waves of one workgroup, which
//    write their subtrees to LDS; after a barrier each output is finished as
//    ((c0+c1)+(c2+c3)) + ((c4+c5)+(c6+c7)), absent chunks being +0.
//  That is the same tree.  d_w*d_x comes from v_mfma_f32_16x16x1_4b_f32 (a
//  K=1 outer product of 4 blocks, one rounding, then + 0): it can differ from
//  the VALU product only in the sign of a zero, which fma(S, +-0, a) with a
//  not -0 cannot show.
//
// gfx950 mapping:
//  * The MFMA operands hold 8 bytes of k per lane (lane l: row or token l%16,
//    k group l/16).  Any permutation of k applied to both operands leaves the
//    integer block sum unchanged; lane group g takes k = 4g..4g+3 and
//    16+4g..16+4g+3, so every operand is two dwords: for the odd block of a
//    pair the dwords 9+g and 13+g of the pair, for the even block (quants 2
//    bytes into the pair) dwords g..g+1 and g+4..g+5 realigned by v_alignbit.
//  * LDS banks, as measured with the bank-conflict counter on gfx950: a
//    ds_read_b32 (and each half of a ds_read2_b32) serves 32 lanes at a time
//    from 32 banks of 4 bytes, so the 16 rows x 2 lane groups of a half-wave
//    must hit 32 distinct dwords mod 32.
//  * Weights: each wave streams its chunk (16 rows x 544 bytes) with 16-byte
//    buffer loads (1 KiB per instruction, rows past n read zeros), two chunks
//    in flight in registers, written unchanged (as 8-byte halves) to a
//    wave-private LDS tile with a row stride of 552 bytes: 138 dwords puts
//    the 16 rows on the 16 even banks mod 32 and the lane groups g, g+1 of a
//    half-wave on both parities, so every operand read is conflict-free (a
//    16-byte-aligned stride always maps rows r and r+8 to one bank).
//  * Activations: staged once per workgroup, already permuted: [token][pair]
//    [g][16 bytes] (the lane's 8 bytes of the even block, then of the odd
//    one), token stride K + 32 bytes, so a lane reads the B operands of a pair
//    with one ds_read_b128, conflict-free (a stride of K + 16 is not); d_x as
//    [token][K/32 + 4] floats.  Lanes of tokens past m read token m-1: their
//    outputs are never stored.
//  * Persistent workgroups of 8 waves (one per CU: the tiles, the combine
//    buffers and up to 15 tokens of activations take up to 155 KiB of LDS);
//    a workgroup iteration is RG row groups (RG = 8 / chunks per row, at most
//    32/m so that every thread stores at most one output).  The outputs are
//    written with range-checked buffer stores, exactly one per thread and
//    iteration, so the compiler's wait before staging a chunk counts the
//    other chunk's loads exactly and never waits for it.
#include "bqmm_internal.h"

namespace bqm {

constexpr int kMvWaves = 8;
constexpr int kMvThreads = 64 * kMvWaves;
constexpr int kMvRows = 16;                         // weight rows per row group (MFMA M)
constexpr int kMvChunkPairs = 8;                    // block pairs per chunk
constexpr int kMvChunkRowBytes = kMvChunkPairs * 68; // 544
constexpr int kMvTileStride = 552;                  // LDS bytes per tile row (544 + 8; 138 dwords)
constexpr int kMvTileBytes = kMvRows * kMvTileStride + 16;   // + 16 bytes that absorb the unused load slots
constexpr int kMvSlots = 9;                         // 16-byte loads per lane and chunk (544 of 576 used)
constexpr int kMvCombV = 68;                        // floats per output register v in the combine area
constexpr int kMvCombWave = 4 * kMvCombV;           // floats per wave
constexpr int kMvCombBytes = 2 * kMvWaves * kMvCombWave * 4;
constexpr uint32_t kMvNoOffset = 0xFFFFFFF0u;       // past every resource: loads read 0, stores drop

struct MvGeom {
    int nb;      // blocks per row (K/32)
    int P;       // block pairs per row
    int nch;     // chunks per row, ceil(P/8)
    int RG;      // row groups per workgroup iteration
    int nrg;     // row groups, ceil(n/16)
    int iters;   // workgroup iterations, ceil(nrg/RG)
    int ts;      // LDS bytes per token of staged quants (K + 32)
    int ds;      // floats per token of staged d_x (K/32 + 4)
    int act_bytes;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t mv_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

template <int M>
__global__ __launch_bounds__(kMvThreads) void q8_0_gemv_mma_kernel(const uint8_t *__restrict__ w, int64_t w_row_bytes,
                                                                     const int8_t *__restrict__ xq,
                                                                     const float *__restrict__ xds, float *__restrict__ y,
                                                                     int k, int n, MvGeom g) {
    static_assert(M >= 1 && M <= 16, "one 16-token MFMA tile");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    uint8_t *act_q = lds;                                           // [M][ts]
    float *act_d = reinterpret_cast<float *>(lds + M * g.ts);      // [M][ds]
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    uint8_t *tile = lds + g.act_bytes + wave * kMvTileBytes;
    float *comb = reinterpret_cast<float *>(lds + g.act_bytes + kMvWaves * kMvTileBytes);

    // This wave's part of a workgroup iteration: row group slot and chunk.
    const int slot = wave / g.nch;
    const int c = wave - slot * g.nch;
    const bool active = slot < g.RG;
    const int cp = min(kMvChunkPairs, g.P - kMvChunkPairs * c);   // pairs in the chunk: 8, or 4 for a last one
    const int cpr = cp * 68 / 16;                                   // 16-byte columns per chunk row
    const int my_iters = (int)blockIdx.x < g.iters ? (g.iters - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;

    // Per-slot offsets of this lane's 16-byte piece: in memory (relative to the
    // chunk's first row) and in the tile.
    uint32_t voff[kMvSlots], loff[kMvSlots];
#pragma unroll
    for (int s = 0; s < kMvSlots; s++) {
        const int ci = 64 * s + lane;
        const int r = ci / cpr, col = ci - (ci / cpr) * cpr;
        const bool ok = active && ci < kMvRows * cpr;
        voff[s] = ok ? (uint32_t)(r * w_row_bytes + 16 * col) : kMvNoOffset;
        // pieces past the chunk land in the never-read 16 bytes at the end of the tile
        loff[s] = ok ? (uint32_t)(r * kMvTileStride + 16 * col) : (uint32_t)(kMvRows * kMvTileStride);
    }
    // Materialize the offsets here, before any load is in flight: computed
    // later, their 64-bit arithmetic was placed in registers next to pending
    // load results and waited for them.
#pragma unroll
    for (int s = 0; s < kMvSlots; s++) asm volatile("" ::"v"(voff[s]), "v"(loff[s]));

    // Issue the loads of iteration i; past the last one the resource is empty.
    auto issue = [&](u32x4 (&buf)[kMvSlots], int i) {
        const int64_t rg = (int64_t)((int)blockIdx.x + (int)gridDim.x * i) * g.RG + slot;
        const int64_t row0 = rg * kMvRows;
        const bool ok = active && i < my_iters && row0 < n;
        const int64_t rem = ok ? (n - row0) * w_row_bytes - (int64_t)kMvChunkRowBytes * c : 0;
        const uint8_t *base = ok ? w + row0 * w_row_bytes + kMvChunkRowBytes * c : w;
        const __amdgpu_buffer_rsrc_t rs = mv_rsrc(base, rem > 0x7FFFFFF0ll ? 0x7FFFFFF0u : (uint32_t)rem);
#pragma unroll
        for (int s = 0; s < kMvSlots; s++)
            buf[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff[s], 0, 2));
    };
    // Wave-private tile: LDS operations of a wave complete in order, so the
    // previous chunk's reads are done before these writes land.  Every slot is
    // written (no branch), so the compiler's wait before each write counts the
    // loads issued since exactly.
    auto stage = [&](const u32x4 (&buf)[kMvSlots]) {
#pragma unroll
        for (int s = 0; s < kMvSlots; s++) {
            *reinterpret_cast<uint2 *>(tile + loff[s]) = make_uint2(buf[s][0], buf[s][1]);
            *reinterpret_cast<uint2 *>(tile + loff[s] + 8) = make_uint2(buf[s][2], buf[s][3]);
        }
    };

    // The operands of this lane: weight row / token r, k group gq.
    const int r = lane & 15, gq = lane >> 4;
    const int tt = r < M ? r : M - 1;
    const uint8_t *arow = act_q + tt * g.ts + 16 * gq;       // + 64 * pair
    const float *drow = act_d + tt * g.ds + gq;              // + block of the 4-block group
    const uint8_t *wrow = tile + r * kMvTileStride;
    const int blk0 = 2 * kMvChunkPairs * c;                   // first block of the chunk

    // Subtree of the chunk's leaves for this lane's 4 outputs (weight rows
    // 4*gq + v, token r), a 4-pair quad at a time (the quad loop is not
    // unrolled: that keeps the block sums and scale products of one quad in
    // registers, not a whole chunk's).
    auto compute = [&](float (&sub)[4]) {
#pragma unroll 1
        for (int qd = 0; qd < cp / 4; qd++) {
            float leaf[4][4];
#pragma unroll
            for (int dd = 0; dd < 2; dd++) {
                const int duo = 2 * qd + dd;               // pairs 2*duo, 2*duo + 1 of the chunk
                // scale products of the duo's 4 blocks: lane group gq supplies block 4*duo + gq
                const int pr = 2 * duo + (gq >> 1);
                const float dw = half_bits_to_float(*reinterpret_cast<const uint16_t *>(wrow + 68 * pr + 34 * (gq & 1)));
                const float dx = drow[blk0 + 4 * duo];
                const v16f z16 = {0};
                const v16f P = __builtin_amdgcn_mfma_f32_16x16x1f32(dw, dx, z16, 0, 0, 0);
#pragma unroll
                for (int jj = 0; jj < 2; jj++) {
                    const int p = 2 * duo + jj;
                    const uint32_t *pw = reinterpret_cast<const uint32_t *>(wrow + 68 * p);
                    const uint32_t e0 = pw[gq], e1 = pw[gq + 1], e4 = pw[gq + 4], e5 = pw[gq + 5];
                    const uint32_t o9 = pw[gq + 9], o13 = pw[gq + 13];
                    const long ae = (long)((uint64_t)__builtin_amdgcn_alignbit(e1, e0, 16u) |
                                           ((uint64_t)__builtin_amdgcn_alignbit(e5, e4, 16u) << 32));
                    const long ao = (long)((uint64_t)o9 | ((uint64_t)o13 << 32));
                    const u32x4 bb = *reinterpret_cast<const u32x4 *>(arow + 32 * (blk0 + 2 * p));
                    const long be = (long)((uint64_t)bb[0] | ((uint64_t)bb[1] << 32));
                    const long bo = (long)((uint64_t)bb[2] | ((uint64_t)bb[3] << 32));
                    const v4i z4 = {0, 0, 0, 0};
                    const v4i se = __builtin_amdgcn_mfma_i32_16x16x32_i8(ae, be, z4, 0, 0, 0);
                    const v4i so = __builtin_amdgcn_mfma_i32_16x16x32_i8(ao, bo, z4, 0, 0, 0);
#pragma unroll
                    for (int v = 0; v < 4; v++) {
                        float a = 0.0f;
                        a = __builtin_fmaf((float)se[v], P[4 * (2 * jj) + v], a);
                        a = __builtin_fmaf((float)so[v], P[4 * (2 * jj + 1) + v], a);
                        leaf[2 * dd + jj][v] = a;
                    }
                }
            }
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const float q = (leaf[0][v] + leaf[1][v]) + (leaf[2][v] + leaf[3][v]);
                sub[v] = qd == 0 ? q : sub[v] + q;
            }
        }
    };

    // One output per thread and iteration: (row group slot, token, row).
    const int nout = g.RG * M * kMvRows;
    const int o = threadIdx.x < nout ? (int)threadIdx.x : 0;
    const int os = o / (M * kMvRows);
    const int ot = (o - os * M * kMvRows) >> 4;
    const int orr = o & 15;
    const int osrc = os * g.nch;                              // first chunk wave of the slot
    const int ooff = (orr & 3) * kMvCombV + 16 * (orr >> 2) + ot;   // (v, lane) of the output in a chunk's record
    const __amdgpu_buffer_rsrc_t ry = mv_rsrc(y, (uint32_t)((int64_t)M * n * 4));
    auto finish = [&](int i, int cb) {
        const float *cw = comb + cb * (kMvWaves * kMvCombWave) + osrc * kMvCombWave + ooff;
        float cv[kMvChunkPairs];
#pragma unroll
        for (int cc = 0; cc < kMvChunkPairs; cc++) {
            const float vcc = cw[(cc < g.nch ? cc : 0) * kMvCombWave];
            cv[cc] = cc < g.nch ? vcc : 0.0f;
        }
        const float sum = ((cv[0] + cv[1]) + (cv[2] + cv[3])) + ((cv[4] + cv[5]) + (cv[6] + cv[7]));
        const int64_t row = ((int64_t)((int)blockIdx.x + (int)gridDim.x * i) * g.RG + os) * kMvRows + orr;
        const bool ok = (int)threadIdx.x < nout && row < n;
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, sum), ry,
                                              ok ? (uint32_t)(((int64_t)ot * n + row) * 4) : kMvNoOffset, 0, 0);
    };

    auto step = [&](int i, int cb) {
        float sub[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (active) compute(sub);
        float *cw = comb + cb * (kMvWaves * kMvCombWave) + wave * kMvCombWave + lane;
#pragma unroll
        for (int v = 0; v < 4; v++) cw[v * kMvCombV] = sub[v];
        __syncthreads();
        finish(i, cb);
    };

    // Activations first: at most two (token, pair) items per thread (m*K/64 <=
    // 15*64 <= 2*512), loaded before the weight chunks so that waiting for
    // them does not wait for the chunks too, then written to LDS permuted for
    // the B operand (see the head of the file).  Items past the activations
    // load from past the resources (zeros) and are not written.
    const __amdgpu_buffer_rsrc_t rq = mv_rsrc(xq, (uint32_t)(M * k));
    const __amdgpu_buffer_rsrc_t rd = mv_rsrc(xds, (uint32_t)(M * g.nb * 8));
    u32x4 ac[2][4], ad[2];
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const int e = (int)threadIdx.x + kMvThreads * h;
        const int t = e / g.P, p = e - (e / g.P) * g.P;
        const bool ok = e < M * g.P;
        const uint32_t qo = ok ? (uint32_t)(t * k + 64 * p) : (uint32_t)(M * k);
#pragma unroll
        for (int c = 0; c < 4; c++)
            ac[h][c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, qo + 16 * c, 0, 0));
        ad[h] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                              rd, ok ? (uint32_t)((t * g.nb + 2 * p) * 8) : (uint32_t)(M * g.nb * 8), 0, 0));
    }
    u32x4 bufA[kMvSlots], bufB[kMvSlots];
    issue(bufA, 0);
    issue(bufB, 1);
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const int e = (int)threadIdx.x + kMvThreads * h;
        if (e < M * g.P) {
            const int t = e / g.P, p = e - (e / g.P) * g.P;
            uint8_t *dst = act_q + t * g.ts + 64 * p;
#pragma unroll
            for (int q = 0; q < 4; q++) {
                u32x4 v;
                v[0] = ac[h][0][q];
                v[1] = ac[h][1][q];
                v[2] = ac[h][2][q];
                v[3] = ac[h][3][q];
                *reinterpret_cast<u32x4 *>(dst + 16 * q) = v;
            }
            // each element is copied to a scalar before the bit cast: clang
            // lowers a bit cast of a vector-element expression to a read of
            // element 0
            const uint32_t d0 = ad[h][0], d1 = ad[h][2];
            act_d[t * g.ds + 2 * p] = __builtin_bit_cast(float, d0);
            act_d[t * g.ds + 2 * p + 1] = __builtin_bit_cast(float, d1);
        }
    }
    __syncthreads();
    // Both halves of the loop body always run, so on every path into a stage
    // the other buffer's loads were issued after this buffer's (a path that
    // skipped a half would make the compiler wait for the other buffer too).
    int i = 0;
    for (; i + 1 < my_iters; i += 2) {
        stage(bufA);
        issue(bufA, i + 2);
        step(i, 0);
        stage(bufB);
        issue(bufB, i + 3);
        step(i + 1, 1);
    }
    if (i < my_iters) {
        stage(bufA);
        step(i, 0);
    }
}

template <int M>
static int launch_mma(const uint8_t *w, int64_t w_row_bytes, const int8_t *xq, const float *xds, float *y, int k, int n,
                      const MvGeom &g, hipStream_t stream) {
    const int lds_bytes = g.act_bytes + kMvWaves * kMvTileBytes + kMvCombBytes;
    static LaunchCache cache;
    const int rc = raise_lds_limit(cache, reinterpret_cast<const void *>(&q8_0_gemv_mma_kernel<M>), 160 * 1024);
    if (rc != BQM_OK) return rc;
    // persistent workgroups, one per CU, as few as give each the same number of iterations
    int grid = device_cus();
    if (g.iters < grid) grid = g.iters;
    const int per = (g.iters + grid - 1) / grid;
    grid = (g.iters + per - 1) / per;
    hipLaunchKernelGGL((q8_0_gemv_mma_kernel<M>), dim3(grid), dim3(kMvThreads), lds_bytes, stream, w, w_row_bytes, xq,
                       xds, y, k, n, g);
    return launch_status();
}

bool gemv_mma_applies(int m, int k, int n) {
    if (m < 3 || m > 15 || k > 4096 || k % 256 != 0) return false;
    if ((int64_t)m * n * 4 > 0x7FFFFFF0ll) return false;
    const int64_t act = (int64_t)m * (k + 32) + (int64_t)m * (k / 32 + 4) * 4;
    return ((act + 15) & ~15ll) + kMvWaves * kMvTileBytes + kMvCombBytes <= 160 * 1024;
}

int gemv_mma(const uint8_t *w, int64_t w_row_bytes, const int8_t *xq, const float *xds, float *y, int m, int k, int n,
             hipStream_t s) {
    MvGeom g;
    g.nb = k / kQK;
    g.P = k / 64;
    g.nch = (g.P + kMvChunkPairs - 1) / kMvChunkPairs;
    g.RG = kMvWaves / g.nch;
    if (g.RG > 32 / m) g.RG = 32 / m;
    g.nrg = (n + kMvRows - 1) / kMvRows;
    g.iters = (g.nrg + g.RG - 1) / g.RG;
    g.ts = k + 32;
    g.ds = g.nb + 4;
    g.act_bytes = (m * g.ts + m * g.ds * 4 + 15) & ~15;
    switch (m) {
        case 3: return launch_mma<3>(w, w_row_bytes, xq, xds, y, k, n, g, s);
        case 4: return launch_mma<4>(w, w_row_bytes, xq, xds, y, k, n, g, s);
        case 5: return launch_mma<5>(w, w_row_bytes, xq, xds, y, k, n, g, s);
        case 6: return launch_mma<6>(w, w_row_bytes, xq, xds, y, k, n, g, s);
        case 7: return launch_mma<7>(w, w_row_bytes, xq, xds, y, k, n, g, s);
        case 8: return launch_mma<8>(w, w_row_bytes, xq, xds, y, k, n, g, s);
        case 9: return launch_mma<9>(w, w_row_bytes, xq, xds, y, k, n, g, s);
        case 10: return launch_mma<10>(w, w_row_bytes, xq, xds, y, k, n, g, s);
        case 11: return launch_mma<11>(w, w_row_bytes, xq, xds, y, k, n, g, s);
        case 12: return launch_mma<12>(w, w_row_bytes, xq, xds, y, k, n, g, s);
        case 13: return launch_mma<13>(w, w_row_bytes, xq, xds, y, k, n, g, s);
        case 14: return launch_mma<14>(w, w_row_bytes, xq, xds, y, k, n, g, s);
        case 15: return launch_mma<15>(w, w_row_bytes, xq, xds, y, k, n, g, s);
        default: return BQM_EINVAL;
    }
}

}  // namespace bqm
