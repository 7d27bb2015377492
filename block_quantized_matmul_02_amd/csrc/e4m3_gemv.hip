// e4m3 decode GEMV for gfx950: raw e4m3 weight rows (one byte per weight,
// per-tensor f32 scale) against f32 activations, m = 1..16.
//
// What it computes ("fp8_ffi.rs" page, memra-engine 0.70.0, st_e4m3_enabled
// doc: decode reads the checkpoint's own e4m3 bytes through
// qmatvec_e4m3_mmvq, the scalar-scale class): y[t][r] = w_scale *
// sum_k x[t][k] * dec(w[r][k]).  The page does not give that kernel's
// activation format; the activation is used as the f32 values it is.
//
// Design (HBM-bound: every weight byte is read exactly once per token group):
//  * A row is CPR = k/16 chunks of 16 bytes.  L lanes share a row (64 when
//    k >= 1024, else the next power of two >= CPR), lane i of the row owns
//    chunks i, i+L, ... (J of them), and a wave covers G = 64/L rows per
//    work item.  With L = 64 every load instruction reads 1 KiB of one row.
//  * Items are streamed with 16-byte range-checked buffer loads into three
//    register buffers that rotate, so two items are in flight while one is
//    computed; every refill is issued unconditionally (past the wave's last
//    item the resource is empty) so the compiler's waits are exact.  The
//    weights need no realignment, so they go from the loads straight into the
//    arithmetic, with no LDS pass.
//  * Decode: v_cvt_pk_f32_fp8 turns two OCP e4m3 bytes into two exact f32
//    values (every e4m3 value is exact in f32).
//  * Per-row order, the same for every token count: a leaf is 16 fma over one
//    chunk in k order, starting from +0; a lane sums its J slot leaves by the
//    perfect binary tree over the slot index (padded with +0 to a power of
//    two); the L lane sums are added by a fixed DPP / permlane-swap butterfly,
//    the perfect binary tree over the lane index; y = w_scale * sum.  A leaf
//    is never -0, so the +0 padding changes nothing, and decode and verify
//    agree bitwise whatever the kernel below.  Rounding: at most 16 fma, 3
//    slot levels and 6 lane levels per output, (16 + 9) * 2^-24 of
//    sum|terms|.
//  * One token (k <= 4096): a lane's chunks are the same on every row, so
//    their 16*J activations sit in registers, loaded before the first weight
//    tiles.
//  * Two or more tokens at k > 1024 (J >= 2): the slot-split kernel below,
//    with each wave owning one chunk slot and the tokens' values of that
//    chunk in registers.
//  * Otherwise (k <= 1024, or a launch too large for 32-bit output offsets)
//    the tokens are staged in LDS, one workgroup-shared copy per token group
//    (as many tokens as the LDS holds), each chunk's four 16-byte pieces
//    rotated by (c + c/4) % 4 so the 16 lanes of a read phase, on 16
//    consecutive chunks, hit distinct banks.  Token groups of the same rows
//    run together on one XCD, so their re-reads of a weight tile are served
//    by that XCD's L2.
#include "bqmm_internal.h"

namespace bqm {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kE8Threads = 256;       // workgroup of the one-token kernel and of staged tokens up to 2
constexpr int kE8GroupThreads = 512;  // staged-token workgroup for three or more tokens
constexpr int kE8SlotsMinM = 2;       // fewest tokens for the slot-split kernel
constexpr int kE8MaxK = 8192;
constexpr int kE8LdsBytes = 160 * 1024;

struct E8Geom {
    int CPR;       // 16-byte chunks per row
    int L;         // lanes per row
    int Llog2;
    int G;         // rows per item
    int J;         // chunks per lane per row
    int n_items;   // ceil(n / G)
    int tgsz;      // tokens per group (the last group may hold fewer)
    int ngroups;   // token groups
    int xcd_map;   // token groups of the same rows on one XCD (see the kernel)
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t e8_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 e4m3 bytes -> 16 f32, in byte order
__device__ __forceinline__ void e8_decode16(const u32x4 c, float (&f)[16]) {
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[q], false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[q], true);
        f[4 * q + 0] = lo[0];
        f[4 * q + 1] = lo[1];
        f[4 * q + 2] = hi[0];
        f[4 * q + 3] = hi[1];
    }
}

// float offset of piece i (four floats) of chunk c inside a staged token row
__device__ __forceinline__ int e8_piece(int c, int i) { return 16 * c + 4 * ((i + c + (c >> 2)) & 3); }

// Perfect binary tree over N (a power of two) values in index order.  Slots
// past a row's last chunk hold +0, and a chain that starts from +0 never ends
// at -0, so padding with +0 to any larger power of two gives the same value.
template <int N>
__device__ __forceinline__ float e8_tree(const float *v) {
    if constexpr (N == 1) return v[0];
    else return e8_tree<N / 2>(v) + e8_tree<N / 2>(v + N / 2);
}

// Sum of one value over the L lanes of a row (lanes li = 0..L-1 of a group
// of L): the perfect binary tree over li, formed by a fixed DPP /
// permlane-swap butterfly (xor 1, xor 2, half-row mirror, row mirror, then
// rows and halves swapped).
__device__ __forceinline__ float e8_row_sum(float v, int L) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
    if (L >= 32) v = swap16_sum(v);
    if (L >= 64) v = swap32_sum(v);
    return v;
}

// JM: chunk slots per lane (>= J); XREG: one token, activations in registers;
// NT: threads per workgroup (all of them share the staged tokens).
template <int JM, bool XREG, int NT>
__global__ __launch_bounds__(NT) void e4m3_gemv_kernel(const uint8_t *__restrict__ w,
                                                             const float *__restrict__ x, float w_scale,
                                                             float *__restrict__ y, int m, int k, int n,
                                                             E8Geom g) {
    extern __shared__ __attribute__((aligned(16))) float xs[];   // [TG][k], pieces rotated
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // With several token groups, the groups that stream the same rows are
    // placed on one XCD (workgroups reach the 8 XCDs round-robin, id % 8) at
    // consecutive slots, so they run together and all but the first read
    // the weights from that XCD's L2 instead of from memory.
    int tg, rwg;
    if (g.xcd_map) {
        const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
        tg = slot % g.ngroups;
        rwg = (slot / g.ngroups) * 8 + xcd;
    } else {
        tg = blockIdx.x % g.ngroups;
        rwg = blockIdx.x / g.ngroups;
    }
    const int t0 = tg * g.tgsz;
    const int tcount = min(g.tgsz, m - t0);
    const int nwaves = (gridDim.x / g.ngroups) * (NT / 64);
    const int wid = rwg * (NT / 64) + wave;
    const int Q = wid < g.n_items ? (g.n_items - 1 - wid) / nwaves + 1 : 0;

    const int li = lane & (g.L - 1);
    const int gr = lane >> g.Llog2;
    // this lane's chunk of each slot, and its byte offset in an item
    bool valid[JM];
    uint32_t voff[JM];
#pragma unroll
    for (int j = 0; j < JM; j++) {
        const int c = li + g.L * j;
        valid[j] = j < g.J && c < g.CPR;
        voff[j] = valid[j] ? (uint32_t)(gr * k + 16 * c) : 0xFFFFFFF0u;
    }

    // Activations in registers (one token, k <= 4096), loaded ahead of the
    // weight tiles so that waiting for them does not wait for the tiles.
    float xr[XREG ? JM : 1][16];
    if (XREG) {
        const __amdgpu_buffer_rsrc_t rx = e8_rsrc(x + (int64_t)t0 * k, (uint32_t)k * 4u);
#pragma unroll
        for (int j = 0; j < (XREG ? JM : 1); j++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const uint32_t off = valid[j] ? (uint32_t)(64 * (li + g.L * j) + 16 * i) : 0xFFFFFFF0u;
                // whole-vector cast (a bit cast of one vector element would
                // read element 0)
                const v4f v = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
#pragma unroll
                for (int e = 0; e < 4; e++) xr[j][4 * i + e] = v[e];
            }
    }

    // Item q of this wave: G rows starting at (wid + nwaves*q) * G.  Past the
    // last item the resource is empty and the loads return zeros.
    auto issue = [&](u32x4 (&buf)[JM], int q) {
        const int64_t row0 = (int64_t)(wid + nwaves * q) * g.G;
        const int64_t rem = (int64_t)(n - row0) * k;
        const uint32_t bytes = q >= Q ? 0u : (rem > 0x7FFFFFF0ll ? 0x7FFFFFF0u : (uint32_t)rem);
        const uint8_t *base = q >= Q ? w : w + row0 * k;
        const __amdgpu_buffer_rsrc_t rs = e8_rsrc(base, bytes);
#pragma unroll
        for (int j = 0; j < JM; j++)
            buf[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff[j], 0, 2));
    };

    // one token's lane partials summed over the row's L lanes, then scaled
    auto finish = [&](float v, int t, int row, bool store) {
        v = e8_row_sum(v, g.L);
        if (store && li == 0 && row < n) y[(int64_t)(t0 + t) * n + row] = w_scale * v;
    };

    // No branch on a slot's validity: an invalid slot's weights are the zeros
    // of an out-of-range load (its activations zeros too, or chunk 0 from
    // LDS), so it adds exact zeros; a branch here would let the compiler sink
    // the activation loads behind the tiles.
    auto compute = [&](const u32x4 (&buf)[JM], int q) {
        const int row = (wid + nwaves * q) * g.G + gr;
        if (XREG) {
            float lf[JM];
#pragma unroll
            for (int j = 0; j < JM; j++) {
                float f[16];
                e8_decode16(buf[j], f);
                lf[j] = 0.0f;
#pragma unroll
                for (int e = 0; e < 16; e++) lf[j] = __builtin_fmaf(xr[XREG ? j : 0][e], f[e], lf[j]);
            }
            finish(e8_tree<JM>(lf), 0, row, true);
            return;
        }
        // Staged tokens, two at a time (the second repeats the first when the
        // group's count is odd, and is not stored), each with its slot leaves
        // and trees as above.  Up to 4 slots the chunks are decoded once for
        // all tokens.
        constexpr bool PRE = JM <= 4;
        float fw[PRE ? JM : 1][16];
        if (PRE) {
#pragma unroll
            for (int j = 0; j < JM; j++) e8_decode16(buf[j], fw[PRE ? j : 0]);
        }
#pragma unroll 1
        for (int t = 0; t < tcount; t += 2) {
            const int t1 = t + 1 < tcount ? t + 1 : t;
            const float *x0 = xs + t * k, *x1 = xs + t1 * k;
            // activations of slot j+1 are read while slot j is computed; the
            // scheduling barriers keep the compiler from reading every slot
            // ahead (which needs 64 registers per slot and token pair)
            float v0[2][16], v1[2][16];
            auto fetch = [&](int j, float (&d0)[16], float (&d1)[16]) {
                const int c = valid[j] ? li + g.L * j : 0;
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const float4 p0 = *reinterpret_cast<const float4 *>(x0 + e8_piece(c, i));
                    const float4 p1 = *reinterpret_cast<const float4 *>(x1 + e8_piece(c, i));
                    d0[4 * i + 0] = p0.x; d0[4 * i + 1] = p0.y; d0[4 * i + 2] = p0.z; d0[4 * i + 3] = p0.w;
                    d1[4 * i + 0] = p1.x; d1[4 * i + 1] = p1.y; d1[4 * i + 2] = p1.z; d1[4 * i + 3] = p1.w;
                }
            };
            fetch(0, v0[0], v1[0]);
            float a0[JM], a1[JM];
#pragma unroll
            for (int j = 0; j < JM; j++) {
                a0[j] = 0.0f;
                a1[j] = 0.0f;
                if (j + 1 < JM) fetch(j + 1 < JM ? j + 1 : j, v0[(j + 1) & 1], v1[(j + 1) & 1]);
                float f[16];
                if (PRE) {
#pragma unroll
                    for (int e = 0; e < 16; e++) f[e] = fw[PRE ? j : 0][e];
                } else {
                    // decoded per token pair: the empty asm keeps the compiler
                    // from hoisting all slots' decodes out of the token loop
                    u32x4 bj = buf[j];
                    asm volatile("" : "+v"(bj));
                    e8_decode16(bj, f);
                }
#pragma unroll
                for (int e = 0; e < 16; e++) {
                    a0[j] = __builtin_fmaf(v0[j & 1][e], f[e], a0[j]);
                    a1[j] = __builtin_fmaf(v1[j & 1][e], f[e], a1[j]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            finish(e8_tree<JM>(a0), t, row, true);
            finish(e8_tree<JM>(a1), t1, row, t + 1 < tcount);
        }
    };

    u32x4 bA[JM], bB[JM], bC[JM];
    issue(bA, 0);
    issue(bB, 1);
    issue(bC, 2);
    if (!XREG) {
        // stage the group's tokens (after the first tiles are in flight)
        const int quads = tcount * k / 4;
        for (int p = threadIdx.x; p < quads; p += NT) {
            const int t = p / (k / 4);
            const int r = p - t * (k / 4);
            const int c = r >> 2, i = r & 3;
            const float4 v = *reinterpret_cast<const float4 *>(x + (int64_t)(t0 + t) * k + 4 * r);
            *reinterpret_cast<float4 *>(xs + t * k + e8_piece(c, i)) = v;
        }
        __syncthreads();
    }
    for (int q = 0; q < Q; q += 3) {
        compute(bA, q);
        issue(bA, q + 3);
        if (q + 1 < Q) compute(bB, q + 1);
        issue(bB, q + 4);
        if (q + 2 < Q) compute(bC, q + 2);
        issue(bC, q + 5);
    }
}

// Verify batches at K > 1024 (two or more chunk slots per lane).  The staged-
// token kernel above reads 64 bytes of activations from LDS for every 16 fma,
// which made the LDS as busy as the VALU.  Here the row's chunk slots are
// spread over the waves of a workgroup: wave j owns slot j (chunk li + 64*j of
// every row), so a lane needs only its one chunk of each token, 16*MT floats,
// held in registers for the whole launch.  A workgroup streams items of JP
// rows; wave j loads slot j of all JP rows (1 KiB per row, one load
// instruction), computes each token's slot leaf, and parks it in LDS; after
// one barrier wave r sums row r of the item: the slot tree, then the lane
// butterfly, the same operations in the same order as the one-token kernel.
// JP: chunk slots per lane rounded up to a power of two (waves per workgroup,
// rows per item); MT: token capacity.
template <int JP, int MT>
__global__ __launch_bounds__(64 * JP) void e4m3_gemv_slots_kernel(const uint8_t *__restrict__ w,
                                                                  const float *__restrict__ x, float w_scale,
                                                                  float *__restrict__ y, int m, int k, int n,
                                                                  E8Geom g) {
    constexpr int R = JP;                       // rows per item
    constexpr int EX = R * MT * JP * 64;        // floats of one exchange buffer
    extern __shared__ __attribute__((aligned(16))) float ex[];   // [2][R][MT][JP][64]
    const int lane = threadIdx.x & 63;
    const int j = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int tg, rwg;
    if (g.xcd_map) {
        const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
        tg = slot % g.ngroups;
        rwg = (slot / g.ngroups) * 8 + xcd;
    } else {
        tg = blockIdx.x % g.ngroups;
        rwg = blockIdx.x / g.ngroups;
    }
    const int t0 = tg * g.tgsz;
    const int tcount = min(g.tgsz, m - t0);
    const int nrwg = gridDim.x / g.ngroups;
    const int n_items = (n + R - 1) / R;
    const int Q = rwg < n_items ? (n_items - 1 - rwg) / nrwg + 1 : 0;

    const int c = lane + 64 * j;
    const bool valid = c < g.CPR;
    uint32_t off[R];
#pragma unroll
    for (int r = 0; r < R; r++) off[r] = valid ? (uint32_t)(r * k + 16 * c) : 0xFFFFFFF0u;

    // this lane's chunk of every token (zeros past the group or the row)
    float xr[MT][16];
    {
        const __amdgpu_buffer_rsrc_t rx = e8_rsrc(x + (int64_t)t0 * k, (uint32_t)tcount * (uint32_t)k * 4u);
#pragma unroll
        for (int t = 0; t < MT; t++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const uint32_t o = (valid && t < tcount) ? (uint32_t)((t * k + 16 * c) * 4 + 16 * i) : 0xFFFFFFF0u;
                const v4f v = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rx, o, 0, 0));
#pragma unroll
                for (int e = 0; e < 4; e++) xr[t][4 * i + e] = v[e];
            }
    }
    const __amdgpu_buffer_rsrc_t ry = e8_rsrc(y, (uint32_t)m * (uint32_t)n * 4u);

    // item q: rows (rwg + nrwg*q)*R ..+R; past the last item the resource is empty
    auto issue = [&](u32x4 (&buf)[R], int q) {
        const int64_t row0 = (int64_t)(rwg + nrwg * q) * R;
        const int64_t rem = ((int64_t)n - row0) * k;
        const uint32_t bytes = q >= Q ? 0u : (rem > 0x7FFFFFF0ll ? 0x7FFFFFF0u : (uint32_t)rem);
        const uint8_t *base = q >= Q ? w : w + row0 * k;
        const __amdgpu_buffer_rsrc_t rs = e8_rsrc(base, bytes);
#pragma unroll
        for (int r = 0; r < R; r++)
            buf[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off[r], 0, 2));
    };

    auto step = [&](const u32x4 (&buf)[R], int q) {
        float *e = ex + (q & 1) * EX;
        // slot leaves: one 16-fma chain per row and token, from +0
#pragma unroll
        for (int r = 0; r < R; r++) {
            float f[16];
            e8_decode16(buf[r], f);
#pragma unroll
            for (int t = 0; t < MT; t++) {
                if (t >= tcount) break;
                float lf = 0.0f;
#pragma unroll
                for (int i = 0; i < 16; i++) lf = __builtin_fmaf(xr[t][i], f[i], lf);
                e[((r * MT + t) * JP + j) * 64 + (lane ^ (4 * (t & 3)))] = lf;
            }
        }
        __syncthreads();
        // Wave j finishes row j of the item.  The wave's lanes are split into
        // TP token slots of LPT = 64/TP lanes; lane l takes token l/LPT and the
        // 64/LPT consecutive lane leaves li from 64/LPT*(l%LPT) on: for each li
        // the slot tree, then the tree over its li, then log2(LPT) DPP levels
        // over the token's lanes (xor 1, xor 2, half-row mirror, row mirror):
        // the same perfect tree over li as the butterfly.  In the exchange
        // buffer lane li of token t sits at li ^ 4*(t%4), so the 16 lanes of
        // a b128 read phase hit 16 distinct 4-bank groups.  Exactly one store
        // per wave and item (out-of-range offsets for the other lanes), so
        // the compiler's waits before the next item stay exact.
        {
            constexpr int TP = MT <= 4 ? 4 : MT <= 8 ? 8 : 16;   // token slots of the sum
            constexpr int LPT = 64 / TP;                         // lanes per token
            constexpr int NC = 16 / LPT;                         // groups of 4 li per lane
            const int64_t row = (int64_t)(rwg + nrwg * q) * R + j;
            const int tt = lane / LPT, bq = lane % LPT;
            const int tr = tt < MT ? tt : MT - 1;   // lanes past MT repeat a token and store nothing
            const float *sp = e + (j * MT + tr) * JP * 64;
            const int sw = 4 * (tr & 3);
            float cs[NC];
#pragma unroll
            for (int cq = 0; cq < NC; cq++) {
                float v[JP][4];
#pragma unroll
                for (int jj = 0; jj < JP; jj++) {
                    const float4 p4 = *reinterpret_cast<const float4 *>(sp + jj * 64 + ((4 * NC * bq + 4 * cq) ^ sw));
                    v[jj][0] = p4.x;
                    v[jj][1] = p4.y;
                    v[jj][2] = p4.z;
                    v[jj][3] = p4.w;
                }
                float lv[4];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    float sl[JP];
#pragma unroll
                    for (int jj = 0; jj < JP; jj++) sl[jj] = v[jj][i];
                    lv[i] = e8_tree<JP>(sl);
                }
                cs[cq] = e8_tree<4>(lv);
            }
            float sum = e8_tree<NC>(cs);
            sum += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, sum), 0xB1, 0xF, 0xF, false));
            sum += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, sum), 0x4E, 0xF, 0xF, false));
            if (LPT >= 8)
                sum += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, sum), 0x141, 0xF, 0xF, false));
            if (LPT >= 16)
                sum += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, sum), 0x140, 0xF, 0xF, false));
            const uint32_t o = (bq == 0 && tt < tcount && row < n) ? (uint32_t)(((int64_t)(t0 + tt) * n + row) * 4)
                                                                 : 0xFFFFFFF0u;
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, w_scale * sum), ry, o, 0, 0);
        }
    };

    u32x4 bA[R], bB[R], bC[R];
    issue(bA, 0);
    issue(bB, 1);
    issue(bC, 2);
    for (int q = 0; q < Q; q += 3) {
        step(bA, q);
        issue(bA, q + 3);
        if (q + 1 < Q) step(bB, q + 1);
        issue(bB, q + 4);
        if (q + 2 < Q) step(bC, q + 2);
        issue(bC, q + 5);
    }
}

static bool e8_geom(int m, int k, int n, int tgsz, E8Geom &g) {
    g.CPR = k / 16;
    int L = 16;
    while (L < g.CPR && L < 64) L *= 2;
    g.L = L;
    g.Llog2 = __builtin_ctz(L);
    g.G = 64 / L;
    g.J = (g.CPR + L - 1) / L;
    g.n_items = (n + g.G - 1) / g.G;
    g.tgsz = tgsz;
    g.ngroups = (m + tgsz - 1) / tgsz;
    return g.J <= 8;
}

template <int JM, bool XREG, int NT>
static int e8_launch(const uint8_t *w, const float *x, float w_scale, float *y, int m, int k, int n,
                     const E8Geom &g, hipStream_t stream) {
    const int lds = XREG ? 0 : g.tgsz * k * 4;
    static LaunchCache cache;
    const void *fn = reinterpret_cast<const void *>(&e4m3_gemv_kernel<JM, XREG, NT>);
    const int rc = raise_lds_limit(cache, fn, kE8LdsBytes);
    if (rc != BQM_OK) return rc;
    const int cus = device_cus();
    // resident workgroups per CU (registers and LDS), at most 4
    const int per_cu = blocks_per_cu(cache, fn, NT, lds, 4);
    // Workgroups per token group: no more than fit at once, and few enough
    // that each wave has at least four items (two in the large workgroups,
    // whose staged tokens are shared by 8 or 16 waves).
    const int waves = NT / 64;
    const int min_items = NT > kE8Threads ? 2 : 4;
    int rwgs = (g.n_items + min_items * waves - 1) / (min_items * waves);
    int cap = cus * per_cu / g.ngroups;
    if (cap < 1) cap = 1;
    if (rwgs > cap) rwgs = cap;
    if (rwgs < 1) rwgs = 1;
    E8Geom gg = g;
    gg.xcd_map = 0;
    if (g.ngroups > 1 && rwgs >= 8) {
        rwgs -= rwgs % 8;   // every XCD holds whole sets of token groups
        gg.xcd_map = 1;
    }
    hipLaunchKernelGGL((e4m3_gemv_kernel<JM, XREG, NT>), dim3(rwgs * g.ngroups), dim3(NT), lds, stream, w, x,
                       w_scale, y, m, k, n, gg);
    return launch_status();
}

template <int JP, int MT>
static int e8_launch_slots(const uint8_t *w, const float *x, float w_scale, float *y, int m, int k, int n,
                           const E8Geom &g, hipStream_t stream) {
    constexpr int NT = 64 * JP;
    const int lds = 2 * JP * MT * JP * 64 * 4;
    static LaunchCache cache;
    const void *fn = reinterpret_cast<const void *>(&e4m3_gemv_slots_kernel<JP, MT>);
    const int rc = raise_lds_limit(cache, fn, kE8LdsBytes);
    if (rc != BQM_OK) return rc;
    const int per_cu = blocks_per_cu(cache, fn, NT, lds, 4);
    // row workgroups per token group: all that fit at once, but at least 4
    // items each (every workgroup also loads the group's activations once)
    const int n_items = (n + JP - 1) / JP;
    int rwgs = (n_items + 3) / 4;
    int cap = device_cus() * per_cu / g.ngroups;
    if (cap < 1) cap = 1;
    if (rwgs > cap) rwgs = cap;
    if (rwgs < 1) rwgs = 1;
    E8Geom gg = g;
    gg.xcd_map = 0;
    if (g.ngroups > 1 && rwgs >= 8) {
        rwgs -= rwgs % 8;
        gg.xcd_map = 1;
    }
    hipLaunchKernelGGL((e4m3_gemv_slots_kernel<JP, MT>), dim3(rwgs * g.ngroups), dim3(NT), lds, stream, w, x, w_scale,
                       y, m, k, n, gg);
    return launch_status();
}

}  // namespace bqm

extern "C" int bqm_e4m3_gemv(const uint8_t *w, const float *x, float w_scale, float *y, int m, int k, int n,
                             void *stream) {
    using namespace bqm;
    if (!w || !x || !y) return BQM_EINVAL;
    if (m < 1 || m > BQM_E4M3_GEMV_MAX_M || k < 256 || n < 1) return BQM_EINVAL;
    if (!(w_scale == w_scale) || w_scale - w_scale != 0.0f) return BQM_EINVAL;   // NaN or infinite
    if (k % 256 != 0 || k > kE8MaxK) return BQM_EUNSUPPORTED;
    if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 4)) return BQM_EUNSUPPORTED;
    if ((int64_t)n * k > 0x7FFFFFFFll * 64) return BQM_EUNSUPPORTED;
    hipStream_t s = as_stream(stream);
    E8Geom g;
    if (!e8_geom(m, k, n, m, g)) return BQM_EUNSUPPORTED;
    if (m >= kE8SlotsMinM && g.J >= 2 && (int64_t)m * n * 4 <= 0x7FFFFFF0ll) {
        // chunk slots spread over the waves of a workgroup, tokens in registers
        // token capacity: 2 for two tokens, 4 up to 4 tokens (and always with
        // 8 slots), 10 for 9..10 tokens at 3..4 slots, which then run as one
        // group instead of two, else 8 (the larger capacities cost registers,
        // so occupancy, and idle token slots)
        const int JP = g.J <= 2 ? 2 : g.J <= 4 ? 4 : 8;
        const int MT = m <= 2 ? 2 : JP == 8 ? 4 : (JP == 4 && m > 8 && m <= 10) ? 10 : (m <= 4 ? 4 : 8);
        const int ng = (m + MT - 1) / MT;
        g.tgsz = (m + ng - 1) / ng;
        g.ngroups = ng;
        if (MT == 2) {
            if (JP == 2) return e8_launch_slots<2, 2>(w, x, w_scale, y, m, k, n, g, s);
            if (JP == 4) return e8_launch_slots<4, 2>(w, x, w_scale, y, m, k, n, g, s);
            return e8_launch_slots<8, 2>(w, x, w_scale, y, m, k, n, g, s);
        }
        if (JP == 2 && MT == 4) return e8_launch_slots<2, 4>(w, x, w_scale, y, m, k, n, g, s);
        if (JP == 2) return e8_launch_slots<2, 8>(w, x, w_scale, y, m, k, n, g, s);
        if (JP == 4 && MT == 4) return e8_launch_slots<4, 4>(w, x, w_scale, y, m, k, n, g, s);
        if (JP == 4 && MT == 10) return e8_launch_slots<4, 10>(w, x, w_scale, y, m, k, n, g, s);
        if (JP == 4) return e8_launch_slots<4, 8>(w, x, w_scale, y, m, k, n, g, s);
        return e8_launch_slots<8, 4>(w, x, w_scale, y, m, k, n, g, s);
    }
    if (m <= 2) {
        if (m == 1 && g.J <= 4) return e8_launch<4, true, kE8Threads>(w, x, w_scale, y, m, k, n, g, s);
        if (g.J <= 4) return e8_launch<4, false, kE8Threads>(w, x, w_scale, y, m, k, n, g, s);
        return e8_launch<8, false, kE8Threads>(w, x, w_scale, y, m, k, n, g, s);
    }
    int fit = kE8LdsBytes / (k * 4);
    if (fit > 16) fit = 16;
    const int ngroups = (m + fit - 1) / fit;
    if (!e8_geom(m, k, n, (m + ngroups - 1) / ngroups, g)) return BQM_EUNSUPPORTED;
    if (g.J <= 4) return e8_launch<4, false, kE8GroupThreads>(w, x, w_scale, y, m, k, n, g, s);
    return e8_launch<8, false, kE8Threads>(w, x, w_scale, y, m, k, n, g, s);
}
