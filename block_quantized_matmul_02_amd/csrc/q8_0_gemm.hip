// Q8_0 x q8_1 prefill GEMM (MMQ) for gfx950 on int8 matrix cores.
//
// y[t][r] = sum_b d_w[r][b] * d_x[t][b] * S[t][r][b]: every 32-block dot
// product is an int32 sum from the matrix cores, folded into an f32
// accumulator by the product of the two block scales ("accprobe_bench.rs"
// module doc: int8 MMA with an s32 accumulator per k32 block, folded every
// k32; "fp8_ffi.rs" module doc: the m >= 16 prefill arm).
//
// gfx950 mapping:
//  * v_mfma_i32_32x32x32_i8 has K = 32, exactly one Q8_0 block, so one MFMA
//    gives the int32 block sums S of a 32x32 output tile.
//  * The fold is per output element and block: acc = fma(float(S),
//    d_x * d_w, acc).  The scale products come from the matrix core (see
//    scale2), which leaves two VALU ops per element and block.  Per 32x32
//    tile and block that is 32 cycles of int8 MFMA, 32 of scale-product MFMA
//    (64 per block pair) and 32 VALU instructions of 4 cycles each (wave64
//    on 16 lanes; no packed f32).  Counters of the full kernels at m=512,
//    K=4096, N=20480: VALU busy is exactly 4 cycles per VALU instruction and
//    the matrix core is busy exactly its instructions' cycles.  For the wide
//    tile the two add up to 97-98% of the SQ busy cycles (per shader engine), so
//    its SIMDs hardly ever wait and the fold is the bound; those launches ran
//    at 1.8-2.1 GHz (SQ_BUSY_CYCLES over the 32 shader engines against the
//    kernel time; 2.4 GHz is the peak), the chip's power limit under this
//    load.  The 128 x 64 tile's come to 109% (a little overlap at four waves
//    per SIMD) with 7% more VALU instructions.
//  * Three tile shapes share the fold; the launch picks one by the time of
//    the busiest CU (launch_mmq).  The wide one (256 tokens x 160 rows, one
//    workgroup per CU, below q8_0_gemm_kernel) is taken where it fills the CUs
//    in whole rounds (m = 512, N = 20480 on MI355X); the 128 x 96 one where
//    128 x 64 workgroups would give some CUs a second one in a round (N = 5152
//    and 6144); the 128 x 64 one everywhere else.  All give bitwise the same y.
//  * The 128 x 64 and 128 x 96 tiles (q8_0_gemm_kernel<F8ACC, WN>, WN = 2 or
//    3).  Workgroup: 4 x WN waves over a 128-token x 32*WN-row output tile of
//    32x32 wave tiles.  The 64-row tile runs two workgroups per CU (four waves
//    per SIMD, at most 128 VGPRs each), which wait at their own barriers, out
//    of step, so one keeps the SIMDs busy while the other waits; the 96-row
//    tile one workgroup of 12 waves (three per SIMD, at most 170 VGPRs), so
//    that no SIMD has more than three tiles at N = 5152.  Each workgroup runs
//    the whole k loop in 128-k stages.
//  * LDS holds two stages per workgroup (the one computed and the one being
//    filled), 30 KB each.  The next stage's global loads are in registers
//    while a stage is computed; they are stored to the other buffer during
//    the stage (activations after block 0, weights and scales after block 2,
//    so the LDS writes overlap the fold) and refilled right after, so every
//    load has a whole stage to land.
//  * One barrier per stage, after block 2: block 3's operands are already in
//    registers, so the next stage's first operands and scales are read under
//    block 3's MFMA and fold instead of after a barrier at the end.
//  * The loop runs two stages per trip, so the LDS buffer index is a
//    compile-time constant and every LDS address a per-lane base plus an
//    immediate (this removed about 20 address instructions per stage).
//  * Weight rows are 34-byte blocks whose quants are 2-byte aligned.  Every
//    thread loads one half-block (16 quants) from its 68-byte block pair
//    (4-byte aligned) with a 16-byte and a 4-byte load; an even block's half
//    is realigned from the five dwords with v_alignbit.  Dense quants and f32
//    scales go to LDS.
//  * Quant tiles are stored with a padded row stride of 144 bytes (128 + 16),
//    so the MFMA operand reads of 8 consecutive rows at the same k hit
//    distinct banks.
//  * XCD-aware tile order (below), and range-checked buffer loads: ragged m
//    and n tails read zeros (zero scales), and only in-range outputs are
//    stored.
//  * Measured with the 128 x 64 tile at every N, before the other two tiles
//    existed (m=512, K=4096, weights rotated past the cache, interleaved on
//    one box): N=20480 140 us against 167 for a 16-wave, one-workgroup-per-CU
//    version (two k-groups over alternate stages, their partial sums added in
//    LDS at the end), N=5152 52 against 58, N=4096 34 against 35.  Ablations
//    of that tile at N=20480: without the global loads 126 us, also without
//    the LDS stores 106, also without the barriers 102 (the register-only
//    floor is about 75).  Tried and not kept: direct global-to-LDS loads of
//    the activation tile (XOR-swizzled 128-byte rows) and its d values, which
//    removed two of the three 16-byte LDS stores per thread and stage:
//    bitwise the same, but 152 us against 140.  The wide tile below now
//    takes N=20480 (120-123 us) and the 96-row tile N=5152 (40-41 us).
//
// The same kernel with its accumulator as the one free variable is the
// accumulator instrument ("accprobe_bench.rs" page, memra-engine 0.124.1,
// module doc): the F8ACC arm reads every quant byte as an OCP e4m3 code and
// replaces the int8 MFMA of a block by two v_mfma_f32_32x32x16_fp8_fp8 that
// accumulate in f32 (the low and high 8 bytes of each lane's 16-byte operand,
// the same k set for both operands).  Tiles, LDS, loads, launch and fold count
// are unchanged; the fold skips the int32 -> f32 convert, since the block sum
// already is f32.
#include <type_traits>

#include "bqmm_internal.h"

namespace bqm {

constexpr int kMmqBM = 128;                  // tokens per workgroup tile
constexpr int kMmqSK = 128;                  // k values per stage = 4 blocks
constexpr int kMmqSB = kMmqSK / kQK;         // 4
constexpr int kMmqStride = kMmqSK + 16;      // 144: padded LDS row of quants
constexpr int kMmqPairBytes = 2 * kQ80Bytes; // 68

__device__ __forceinline__ __amdgpu_buffer_rsrc_t mmq_rsrc(const void *base, int64_t bytes) {
    uint32_t b = bytes <= 0 ? 0u : (bytes > 0x7FFFFFF0ll ? 0x7FFFFFF0u : (uint32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)b, 0x00020000);
}

// One 128-k stage of a workgroup tile in LDS.  Weight rows hold the first 16
// bytes of blocks 0..3 and then their second 16 bytes, so the four lanes that
// store one half of a row write 64 consecutive bytes.  The scale rows are
// padded by 4 floats so the stores of different blocks fall in different
// banks.
template <int WN>
struct MmqStage {
    uint8_t x[kMmqBM * kMmqStride];
    uint8_t w[32 * WN * kMmqStride];
    float dx[kMmqSB][kMmqBM + 4];
    float dw[kMmqSB][32 * WN + 4];
};
// two buffers (the stage computed and the one being filled); two workgroups
// per CU for the 64-row tile, one for the 96-row tile
static_assert(4 * sizeof(MmqStage<2>) <= 160 * 1024 && 2 * sizeof(MmqStage<3>) <= 160 * 1024, "LDS");

// Global loads of one stage (128 k), held in registers until stored to LDS:
// two 16-byte activation chunks, one half-block of weights (16 quants, from a
// 16-byte and a 4-byte load) and one activation scale per thread.
struct MmqRegs {
    u32x4 x[2];
    u32x4 w;
    uint32_t w4;
    float dx;
};

template <bool F8ACC, int WN>
__global__ __launch_bounds__(256 * WN) __attribute__((amdgpu_waves_per_eu(WN == 2 ? 4 : 3, WN == 2 ? 4 : 3))) void
q8_0_gemm_kernel(const uint8_t *__restrict__ w, int64_t w_row_bytes, const int8_t *__restrict__ xq,
                 const float *__restrict__ xds, float *__restrict__ y, int m, int k, int n) {
    static_assert(WN == 2 || WN == 3, "64- or 96-row tile");
    constexpr int kMmqBN = 32 * WN;              // weight rows per workgroup tile
    constexpr int kMmqThreads = 256 * WN;        // 4 x WN output waves
    using MmqStageT = MmqStage<WN>;
    __shared__ __attribute__((aligned(16))) MmqStageT st[2];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: kept in a scalar register
    const int wm = (int)((unsigned)wave / WN), wn = (int)((unsigned)wave % WN);
    // XCD-aware tile order.  Workgroups are handed to the 8 XCDs round-robin
    // (id % 8), and each XCD has its own L2.  Renumber so that XCD x runs a
    // contiguous range of tiles, m-tile fastest: the token tiles that share a
    // weight tile then run together on one XCD and read it once into its L2.
    const int nm = (m + kMmqBM - 1) / kMmqBM;
    const int ntiles = gridDim.x;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int per = ntiles >> 3, extra = ntiles & 7;
    const int tile = xcd * per + min(xcd, extra) + slot;
    const int n0 = (tile / nm) * kMmqBN;
    const int m0 = (tile - (tile / nm) * nm) * kMmqBM;
    const int nb = k / kQK;
    const int nit = k / kMmqSK;

    // Resources covering the valid rows only; out-of-range loads return zeros.
    const __amdgpu_buffer_rsrc_t rX = mmq_rsrc(xq + (int64_t)m0 * k, (int64_t)(m - m0) * k);
    const __amdgpu_buffer_rsrc_t rD = mmq_rsrc(xds + (int64_t)m0 * nb * 2, (int64_t)(m - m0) * nb * 8);
    const __amdgpu_buffer_rsrc_t rW = mmq_rsrc(w + (int64_t)n0 * w_row_bytes, (int64_t)(n - n0) * w_row_bytes);

    // Load slots, fixed for the kernel (the stage's offset is a uniform
    // scalar added by the buffer load).
    //  X: chunk q = tid + kMmqThreads*j of the 128 x 128-byte activation
    //     tile (q < 1024): row q >> 3, 16-byte chunk q & 7.  With 768 threads
    //     the second slot of threads 256.. is empty: it reads nothing (an
    //     offset beyond any range) and stores nothing.
    //  dX: (row tid >> 2, block tid & 3), the d of each (d, s) pair (tid < 512).
    //  W: half-block q = tid of the kMmqBN x 4-block weight tile: row q >> 3,
    //     block bb = (q >> 1) & 3, half h = q & 1.  Blocks pair up into 68-byte
    //     pairs (4-byte aligned): the even block's quants sit 2 bytes into the
    //     pair and are realigned from five dwords, the odd block's are aligned.
    uint32_t xoff[2];
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const int q = tid + kMmqThreads * j;
        const bool live = kMmqThreads * (j + 1) <= 1024 || q < 1024;
        xoff[j] = live ? (uint32_t)((q >> 3) * k + 16 * (q & 7)) : 0x80000000u;
    }
    const bool dlive = kMmqThreads <= 4 * kMmqBM || tid < 4 * kMmqBM;
    const uint32_t doff = dlive ? (uint32_t)(((tid >> 2) * nb + (tid & 3)) * 8) : 0x80000000u;
    const int wrow = tid >> 3, wbb = (tid >> 1) & 3, wh = tid & 1;
    const int wodd = wbb & 1;
    const int wsel = 2 * wodd + wh;           // 0: even h0, 1: even h1, 2: odd h0, 3: odd h1
    const uint32_t wpair = (uint32_t)(wrow * w_row_bytes + kMmqPairBytes * (wbb >> 1));
    const uint32_t woff16 = wpair + (wsel == 0 ? 0u : wsel == 1 ? 16u : wsel == 2 ? 36u : 52u);
    const uint32_t woff4 = wpair + (wsel == 0 ? 16u : wsel == 1 ? 32u : wsel == 2 ? 32u : 48u);

    auto load_x = [&](MmqRegs &R, int it) {
        const int sx = it * kMmqSK;
#pragma unroll
        for (int j = 0; j < 2; j++)
            R.x[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rX, xoff[j], sx, 0));
    };
    auto load_wd = [&](MmqRegs &R, int it) {
        const int sw = it * 2 * kMmqPairBytes, sd = it * 4 * 8;
        R.w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rW, woff16, sw, 0));
        R.w4 = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rW, woff4, sw, 0);
        R.dx = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rD, doff, sd, 0));
    };
    auto load_iter = [&](MmqRegs &R, int it) {
        load_x(R, it);
        load_wd(R, it);
    };
    auto store_x = [&](MmqStageT &S, const MmqRegs &R) {
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int q = tid + kMmqThreads * j;
            if (kMmqThreads * (j + 1) <= 1024 || q < 1024)
                *reinterpret_cast<u32x4 *>(S.x + (q >> 3) * kMmqStride + 16 * (q & 7)) = R.x[j];
        }
    };
    auto store_wd = [&](MmqStageT &S, const MmqRegs &R) {
        // even block: quants = bytes 2.. of dwords (w[0..3], w4); odd: w itself
        u32x4 qv;
        qv[0] = __builtin_amdgcn_alignbit(R.w[1], R.w[0], 16u);
        qv[1] = __builtin_amdgcn_alignbit(R.w[2], R.w[1], 16u);
        qv[2] = __builtin_amdgcn_alignbit(R.w[3], R.w[2], 16u);
        qv[3] = __builtin_amdgcn_alignbit(R.w4, R.w[3], 16u);
        if (wodd) qv = R.w;
        *reinterpret_cast<u32x4 *>(S.w + wrow * kMmqStride + 64 * wh + 16 * wbb) = qv;
        if (wh == 0) S.dw[wbb][wrow] = half_bits_to_float(wodd ? (R.w4 >> 16) : (R.w[0] & 0xFFFFu));
        if (dlive) S.dx[tid & 3][tid >> 2] = R.dx;
    };
    auto store_iter = [&](MmqStageT &S, const MmqRegs &R) {
        store_x(S, R);
        store_wd(S, R);
    };

    v16f acc;
#pragma unroll
    for (int v = 0; v < 16; v++) acc[v] = 0.0f;

    const int arow = wm * 32 + (lane & 31);   // A operand row (token) of this lane
    const int brow = wn * 32 + (lane & 31);   // B operand row (weight row) of this lane
    const int khalf = lane >> 5;
    using BlockSum = typename std::conditional<F8ACC, v16f, v16i>::type;
    // the block sums of one 32x32 tile: int32 from the int8 MFMA, or f32 from
    // two fp8 MFMAs over the same bytes (the instrument's f32 arm)
    auto block_sum = [&](const v4i &a, const v4i &b) -> BlockSum {
        if constexpr (F8ACC) {
            typedef long v2l __attribute__((ext_vector_type(2)));
            const v16f zf = {0};
            const v2l av = __builtin_bit_cast(v2l, a), bv = __builtin_bit_cast(v2l, b);
            const v16f lo = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(av[0], bv[0], zf, 0, 0, 0);
            return __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(av[1], bv[1], lo, 0, 0, 0);
        } else {
            const v16i z = {0};
            return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, z, 0, 0, 0);
        }
    };
    struct Ops { v4i A, B; };
    auto rd = [&](const MmqStageT &S, int b) -> Ops {
        Ops o;
        o.A = *reinterpret_cast<const v4i *>(S.x + arow * kMmqStride + 16 * khalf + 32 * b);
        o.B = *reinterpret_cast<const v4i *>(S.w + brow * kMmqStride + 64 * khalf + 16 * b);
        return o;
    };
    auto rs = [&](const MmqStageT &S, int p, float &sa, float &sb) {
        sa = S.dx[2 * p + khalf][arow];
        sb = S.dw[2 * p + khalf][brow];
    };
    // The scale products d_x[t][b] * d_w[r][b] come from the matrix core: one
    // v_mfma_f32_32x32x1_2b_f32 forms the 32x32 outer products of two blocks
    // (lanes 0-31 carry block b, lanes 32-63 block b+1; each result element is
    // one correctly rounded f32 product, as a VALU multiply would give), in the
    // block sums' register layout.
    auto scale2 = [&](float sa, float sb) -> v32f {
        const v32f z32 = {0};
        return __builtin_amdgcn_mfma_f32_32x32x1f32(sa, sb, z32, 0, 0, 0);
    };
    auto fold = [&](const BlockSum &Sb, const v32f &P, int e) {
#pragma unroll
        for (int v = 0; v < 16; v++) {
            if constexpr (F8ACC)
                acc[v] = __builtin_fmaf(Sb[v], P[16 * e + v], acc[v]);
            else
                acc[v] = __builtin_fmaf((float)Sb[v], P[16 * e + v], acc[v]);
        }
        asm volatile("" : "+v"(acc) :: "memory");
    };

    // Prologue: stage 0 into st[0], stage 1's loads into the registers, and
    // stage 0's first operands and scales read.
    MmqRegs R;
    const int last = nit - 1;
    load_iter(R, 0);
    store_iter(st[0], R);
    load_iter(R, min(1, last));
    __syncthreads();
    Ops o0 = rd(st[0], 0);
    float sa01, sb01;
    rs(st[0], 0, sa01, sb01);
    // One stage: compute st[cur] while stage it + 1's loads go from the
    // registers into st[cur ^ 1] and stage it + 2's are issued in their place
    // (unconditional: past the end they repeat the last stage, so the
    // compiler's count of loads in flight stays exact, and the next block's
    // operand reads, issued before the stores, are waited for without them).
    // The barrier follows block 2: block 3's operands are in registers, and
    // the next stage's first operands and scales are read under its MFMA and
    // fold.  The loop runs two stages per trip (the stage count is even), so
    // the buffer index is a compile-time constant and every LDS address a
    // per-lane base plus an immediate.
    auto stage = [&](int it, int cur) {
        const int nx = min(it + 2, last);
        const MmqStageT &S = st[cur];
        const v32f P01 = scale2(sa01, sb01);
        const BlockSum S0 = block_sum(o0.A, o0.B);
        const Ops o1 = rd(S, 1);
        const Ops o2 = rd(S, 2);
        float sa23, sb23;
        rs(S, 1, sa23, sb23);
        fold(S0, P01, 0);
        store_x(st[cur ^ 1], R);
        load_x(R, nx);
        const BlockSum S1 = block_sum(o1.A, o1.B);
        const Ops o3 = rd(S, 3);
        fold(S1, P01, 1);
        const v32f P23 = scale2(sa23, sb23);
        const BlockSum S2 = block_sum(o2.A, o2.B);
        fold(S2, P23, 0);
        store_wd(st[cur ^ 1], R);
        load_wd(R, nx);
        __syncthreads();
        const MmqStageT &Sn = st[cur ^ 1];
        o0 = rd(Sn, 0);
        rs(Sn, 0, sa01, sb01);
        const BlockSum S3 = block_sum(o3.A, o3.B);
        fold(S3, P23, 1);
    };
#pragma unroll 1
    for (int it = 0; it < nit; it += 2) {
        stage(it, 0);
        stage(it + 1, 1);
    }

    // Output element (row 8*(v/4) + 4*khalf + v%4, column lane%32) of the
    // wave tile.
    // The lane is read again (mbcnt) rather than kept live across the loop.
    const int elane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int col = n0 + wn * 32 + (elane & 31);
    if (col < n) {
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int row = m0 + wm * 32 + 8 * (v >> 2) + 4 * (elane >> 5) + (v & 3);
            if (row < m) y[(int64_t)row * n + col] = acc[v];
        }
    }
}

// Wide tile: each wave owns 32 tokens and five 32-row weight tiles.
//
//  * Workgroup: 8 waves, one workgroup per CU (two waves per SIMD, up to 256
//    VGPRs each), over 256 tokens x 160 weight rows.  At m = 512, N = 20480
//    that is 256 workgroups, one round on the 256 CUs.
//  * A wave's activations go straight from global memory into its MFMA operand
//    registers (16 bytes of one block per lane); nothing else reads them, so
//    they skip LDS.  The pair of blocks 2p, 2p + 1 is reloaded with the next
//    stage's as soon as the stage is done with it, so one register set covers
//    a stage and each load has a stage to land.
//  * The 160 weight rows are shared by the 8 waves through LDS, in stages of
//    256 k (8 blocks).  They are loaded in chunks of 4 blocks, each half-block
//    read from its 2-byte-aligned place with one unaligned 16-byte load (the
//    driver runs gfx9 in unaligned access mode) and its scale with a 2-byte
//    load, then stored without realignment.
//  * Three LDS buffers (47.6 KB each).  A stage's second chunk store is
//    followed by the stage's one barrier, mid-stage.  After it, the next stage
//    is complete in LDS, so its first operands are read before this stage
//    ends.  The store into the third buffer at the start of a stage only needs
//    every wave past the previous stage's barrier, which means done with the
//    stage before it.
//  * The loop runs three stages per trip, so the buffer indices are
//    compile-time constants (one or two stages follow the loop), and the
//    epilogue stores through a range-checked resource over the workgroup's
//    rows of y, one address add per store and no branch (about 1% together).
//  * Per wave and stage, 40 tile-blocks against 12 vector-memory loads, 2-3
//    LDS writes and 20 LDS operand reads.  The loop's VALU work is the fold
//    plus about 2%.  Fetch is 1.20x the algorithmic reads at N = 20480,
//    against 1.89x for the 128 x 64 tile: the two token halves of a weight
//    tile run together on one XCD, and the activations stay in its L2.
//  * The same fold order per output as the 128 x 64 kernel, so the two give
//    bitwise the same y.
constexpr int kWideWaves = 8;
constexpr int kWideThreads = 64 * kWideWaves;
constexpr int kWideBM = 32 * kWideWaves;   // 256 tokens per workgroup: 32 per wave
constexpr int kWideR = 5;                  // 32-row weight tiles per wave
constexpr int kWideBN = 32 * kWideR;       // 160 weight rows per workgroup
constexpr int kWideSB = 8;                 // blocks per stage
constexpr int kWideSK = kQK * kWideSB;     // 256 k per stage
constexpr int kWideStride = kWideSK + 16;  // 272: padded LDS row of quants
constexpr int kWideNC = kWideSB / 4;       // weight chunks (4 blocks) per stage
constexpr int kWideNW = (2 * 4 * kWideBN + kWideThreads - 1) / kWideThreads;   // half-block slots per thread and chunk
constexpr int kWideRS = kWideThreads / 8;  // rows between a thread's slots

// The three 256-k stages of the weight tile in LDS.  A stage's quants: per
// row the first 16 bytes of blocks 0..7, then their second 16 bytes.  Its
// scale rows, padded by 4 floats, sit with the other stages' at the start
// (15.4 KB), so one per-lane base with an immediate offset reaches every
// scale of every stage.
struct WideLds {
    float dw[3][kWideSB][kWideBN + 4];
    uint8_t w[3][kWideBN * kWideStride];
};
static_assert(sizeof(WideLds) <= 160 * 1024 && sizeof(float) * 3 * kWideSB * (kWideBN + 4) < 65536, "LDS");

template <bool F8ACC>
__global__ __launch_bounds__(kWideThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void q8_0_gemm_wide_kernel(
    const uint8_t *__restrict__ w, int64_t w_row_bytes, const int8_t *__restrict__ xq, const float *__restrict__ xds,
    float *__restrict__ y, int m, int k, int n) {
    __shared__ __attribute__((aligned(16))) WideLds lds;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: kept in a scalar register
    // the same XCD-aware order as the 128 x 64 kernel: the token tiles of a
    // weight tile run together on one XCD
    const int nm = (m + kWideBM - 1) / kWideBM;
    const int ntiles = gridDim.x;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int per = ntiles >> 3, extra = ntiles & 7;
    const int tile = xcd * per + min(xcd, extra) + slot;
    const int n0 = (tile / nm) * kWideBN;
    const int m0 = (tile - (tile / nm) * nm) * kWideBM;
    const int nb = k / kQK;
    const int nit = k / kWideSK;

    // Resources covering the valid rows only; out-of-range loads return zeros.
    const __amdgpu_buffer_rsrc_t rX = mmq_rsrc(xq + (int64_t)m0 * k, (int64_t)(m - m0) * k);
    const __amdgpu_buffer_rsrc_t rD = mmq_rsrc(xds + (int64_t)m0 * nb * 2, (int64_t)(m - m0) * nb * 8);
    const __amdgpu_buffer_rsrc_t rW = mmq_rsrc(w + (int64_t)n0 * w_row_bytes, (int64_t)(n - n0) * w_row_bytes);

    const int t = lane & 31, khalf = lane >> 5;
    // this lane's token row and k half: the A operand of block b at aoff + 32 b;
    // the d of block 2p + khalf at doff + 16 p
    const uint32_t aoff = (uint32_t)((32 * wave + t) * k + 16 * khalf);
    const uint32_t doff = (uint32_t)(((32 * wave + t) * nb + khalf) * 8);

    // Weight slots of a chunk: half-block q = tid + 512 j of the 160 x 4-block
    // chunk, i.e. row (tid >> 3) + 64 j, block (tid >> 1) & 3, half tid & 1.
    const int row0 = tid >> 3, bb0 = (tid >> 1) & 3, hh0 = tid & 1;
    const uint32_t woq = (uint32_t)(row0 * w_row_bytes + kQ80Bytes * bb0 + 2 + 16 * hh0);   // 2-byte aligned
    const uint32_t wod = (uint32_t)(row0 * w_row_bytes + kQ80Bytes * bb0);
    const uint32_t wlds = (uint32_t)(row0 * kWideStride + 16 * kWideSB * hh0 + 16 * bb0);
    const int wdw = bb0 * (kWideBN + 4) + row0;
    struct WRegs {
        u32x4 q[kWideNW];
        uint32_t d[kWideNW];
    };
    // chunk c (blocks 4c .. 4c + 3) of stage it
    auto load_w = [&](WRegs &Wr, int it, int c) {
        const int sw = it * kWideSB * kQ80Bytes + c * 4 * kQ80Bytes;
#pragma unroll
        for (int j = 0; j < kWideNW; j++) {
            // slots past the 1280 of a chunk (waves 4..7, last slot) read
            // nothing: an offset beyond any range
            const bool live = kWideThreads * (j + 1) <= 8 * kWideBN || tid + kWideThreads * j < 8 * kWideBN;
            const uint32_t dead = live ? 0u : 0x80000000u;
            // the row step stays in the per-lane offset, which the range check covers
            const uint32_t ro = (uint32_t)(kWideRS * j) * (uint32_t)w_row_bytes;
            Wr.q[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rW, (woq + ro) | dead, sw, 0));
            Wr.d[j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rW, (wod + ro) | dead, sw, 0);
        }
    };
    auto store_w = [&](int b, const WRegs &Wr, int c) {
#pragma unroll
        for (int j = 0; j < kWideNW; j++) {
            if (tid + kWideThreads * j < 8 * kWideBN) {
                *reinterpret_cast<u32x4 *>(lds.w[b] + wlds + kWideRS * kWideStride * j + 64 * c) = Wr.q[j];
                if (hh0 == 0) (&lds.dw[b][0][0])[wdw + kWideRS * j + 4 * c * (kWideBN + 4)] = half_bits_to_float(Wr.d[j]);
            }
        }
    };

    v4i A[kWideSB];
    float D[kWideSB / 2];
    auto load_a = [&](int p, int it) {
#pragma unroll
        for (int b = 2 * p; b < 2 * p + 2; b++)
            A[b] = __builtin_bit_cast(v4i,
                                      __builtin_amdgcn_raw_buffer_load_b128(rX, aoff + 32 * b, it * kWideSK, 0));
        D[p] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rD, doff + 16 * p, it * kWideSB * 8, 0));
    };

    v16f acc[kWideR];
#pragma unroll
    for (int j = 0; j < kWideR; j++)
#pragma unroll
        for (int v = 0; v < 16; v++) acc[j][v] = 0.0f;

    using BlockSum = typename std::conditional<F8ACC, v16f, v16i>::type;
    auto block_sum = [&](const v4i &a, const v4i &b) -> BlockSum {
        if constexpr (F8ACC) {
            typedef long v2l __attribute__((ext_vector_type(2)));
            const v16f zf = {0};
            const v2l av = __builtin_bit_cast(v2l, a), bv = __builtin_bit_cast(v2l, b);
            const v16f lo = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(av[0], bv[0], zf, 0, 0, 0);
            return __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(av[1], bv[1], lo, 0, 0, 0);
        } else {
            const v16i z = {0};
            return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, z, 0, 0, 0);
        }
    };
    // the scale products of two blocks in the block sums' layout, as in the
    // 128 x 64 kernel
    auto scale2 = [&](float sa, float sb) -> v32f {
        const v32f z32 = {0};
        return __builtin_amdgcn_mfma_f32_32x32x1f32(sa, sb, z32, 0, 0, 0);
    };
    auto fold = [&](v16f &ac, const BlockSum &Sb, const v32f &P, int e) {
#pragma unroll
        for (int v = 0; v < 16; v++) {
            if constexpr (F8ACC)
                ac[v] = __builtin_fmaf(Sb[v], P[16 * e + v], ac[v]);
            else
                ac[v] = __builtin_fmaf((float)Sb[v], P[16 * e + v], ac[v]);
        }
    };
    // B operands (weight rows 32 j + lane % 32) of blocks 2p, 2p + 1 and the
    // weight scale of block 2p + khalf
    struct BOps {
        v4i b0, b1;
        float sb;
    };
    auto rdb = [&](int b, int p, int j) -> BOps {
        BOps o;
        const int brow = 32 * j + t;
        o.b0 = *reinterpret_cast<const v4i *>(lds.w[b] + brow * kWideStride + 16 * kWideSB * khalf + 16 * (2 * p));
        o.b1 = *reinterpret_cast<const v4i *>(lds.w[b] + brow * kWideStride + 16 * kWideSB * khalf + 16 * (2 * p + 1));
        o.sb = lds.dw[b][2 * p + khalf][brow];
        return o;
    };

    // Prologue: stage 0 into st[0] (both chunks loaded before either is
    // stored: one wait for memory instead of two), its activations into the
    // registers, and the first chunk of stage 1 into the weight registers.
    WRegs Wr;
    const int last = nit - 1;
    {
        WRegs W1;
        load_w(Wr, 0, 0);
        load_w(W1, 0, 1);
#pragma unroll
        for (int p = 0; p < kWideSB / 2; p++) load_a(p, 0);
        store_w(0, Wr, 0);
        store_w(0, W1, 1);
    }
    load_w(Wr, min(1, last), 0);
    __syncthreads();

    // One stage: compute st[cur]; chunk c of stage it + 1 goes from the
    // registers into st[nxt] at pair 2c, and the next chunk's loads are issued
    // in its place (past the end they repeat the last stage, so the compiler's
    // count of loads in flight stays exact).
    BOps o = rdb(0, 0, 0);
    auto stage = [&](int it, int cur, int nxt) {
#pragma unroll
        for (int p = 0; p < kWideSB / 2; p++) {
#pragma unroll
            for (int j = 0; j < kWideR; j++) {
                const BOps c = o;
                if (j + 1 < kWideR) o = rdb(cur, p, j + 1);
                else if (p + 1 < kWideSB / 2) o = rdb(cur, p + 1, 0);
                else o = rdb(nxt, 0, 0);   // complete since this stage's barrier
                const v32f P = scale2(D[p], c.sb);
                const BlockSum S0 = block_sum(A[2 * p], c.b0);
                const BlockSum S1 = block_sum(A[2 * p + 1], c.b1);
                fold(acc[j], S0, P, 0);
                fold(acc[j], S1, P, 1);
                asm volatile("" : "+v"(acc[j]) :: "memory");
                // Each tile step is scheduled on its own: interleaving steps
                // made the compiler spill (6 VGPRs in the int8 arm, 14 in the
                // f32 arm, each reload waiting for every load in flight).
                __builtin_amdgcn_sched_barrier(0);
                if (j == kWideR - 1) load_a(p, min(it + 1, last));
                if (j == 0 && (p & 1) == 0) {
                    const int ch = p / 2;
                    store_w(nxt, Wr, ch);
                    if (ch + 1 < kWideNC) load_w(Wr, min(it + 1, last), ch + 1);
                    else load_w(Wr, min(it + 2, last), 0);
                    if (ch + 1 == kWideNC) __syncthreads();
                }
            }
        }
    };
    // three stages per trip, so the buffer indices are compile-time
    // constants; one or two stages after the loop
    int it = 0;
#pragma unroll 1
    for (; it + 3 <= nit; it += 3) {
        stage(it, 0, 1);
        stage(it + 1, 1, 2);
        stage(it + 2, 2, 0);
    }
    if (it < nit) stage(it, 0, 1);
    if (it + 1 < nit) stage(it + 1, 1, 2);

    // Output element (row 8*(v/4) + 4*khalf + v%4, column lane%32) of each
    // wave tile: token row, weight-row column.
    // Stores through a resource over this workgroup's rows of y (m0 .. m - 1):
    // rows past m fall outside it, and columns past n get an offset beyond any
    // range, so no store needs a branch (the launch keeps every offset below
    // 2^31).  The lane is read again (mbcnt) rather than kept live across the
    // loop.
    const int elane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const __amdgpu_buffer_rsrc_t rY = mmq_rsrc(y + (int64_t)m0 * n, (int64_t)(m - m0) * n * 4);
    const uint32_t n4 = (uint32_t)n * 4u;
    const uint32_t ybase = ((uint32_t)(32 * wave + 4 * (elane >> 5)) * (uint32_t)n + (uint32_t)(n0 + (elane & 31))) * 4u;
#pragma unroll
    for (int j = 0; j < kWideR; j++) {
        const uint32_t cb = n0 + 32 * j + (elane & 31) < n ? ybase + 128u * j : 0x80000000u;
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const uint32_t ro = (uint32_t)(8 * (v >> 2) + (v & 3)) * n4;
            // copied to a scalar first: a bit cast of a vector-element
            // expression is lowered to a read of element 0
            const float val = acc[j][v];
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, val), rY, cb + ro, 0, 0);
        }
    }
}

template <bool F8ACC>
static int launch_mmq(const uint8_t *w, int64_t w_row_bytes, const int8_t *xq, const float *xds, float *y, int m,
                      int k, int n, void *stream) {
    if (!w || !xq || !xds || !y) return BQM_EINVAL;
    if (m < 1 || k < 256 || n < 1) return BQM_EINVAL;
    if (k % 256 != 0) return BQM_EUNSUPPORTED;
    if (w_row_bytes < (int64_t)(k / kQK) * kQ80Bytes || w_row_bytes % 16 != 0) return BQM_EUNSUPPORTED;
    if (!aligned(w, 16) || !aligned(xq, 16) || !aligned(xds, 8) || !aligned(y, 4)) return BQM_EUNSUPPORTED;
    // per-workgroup offsets are 32-bit: up to 256 rows of activations and 160
    // of weights (an offset with bit 31 set marks a load that reads nothing)
    if ((int64_t)kWideBM * k > 0x7FFFFFF0ll || (int64_t)kWideBN * w_row_bytes > 0x7FFFFFF0ll) return BQM_EUNSUPPORTED;
    const int64_t mt = (m + kMmqBM - 1) / kMmqBM;
    const int64_t tiles64 = (int64_t)((n + 63) / 64) * mt;
    const int64_t tiles96 = (int64_t)((n + 95) / 96) * mt;
    const int64_t wide = (int64_t)((n + 160 - 1) / 160) * ((m + 256 - 1) / 256);
    if (tiles64 > 0x7FFFFFFF) return BQM_EUNSUPPORTED;
    // Tile choice by the busiest CU's time: workgroups per CU (rounded up) x
    // 32 x 32 tiles per SIMD per workgroup x the measured time of one such
    // tile for all of K=4096 (in 0.1 us at m=512; the ratios are what count):
    //  * 128 x 64 (8 waves, two workgroups per CU): 2 tiles per SIMD, 15.5
    //    with one workgroup on the CU, 13 with two;
    //  * 128 x 96 (12 waves, one per CU): 3 tiles per SIMD, 14.5;
    //  * 256 x 160 (8 waves, one per CU): 10 tiles per SIMD, 12.3.
    // The 96-row tile takes shapes whose 64-row workgroups would leave some
    // CUs a second workgroup in one round (N = 5152 or 6144 at m = 512: 42.8
    // and 45.7 us against 53.5 and 55.7), the wide tile whole rounds of large
    // N (20480).  All three fold in the same order: bitwise the same y.
    const int64_t cus = device_cus();
    const int64_t r64 = (tiles64 + cus - 1) / cus, r96 = (tiles96 + cus - 1) / cus, rw = (wide + cus - 1) / cus;
    const int64_t cost64 = r64 == 1 ? 2 * 155 : r64 * 2 * 130;
    const int64_t cost96 = r96 * 3 * 145;
    const int64_t costw = rw * 10 * 123;
    // the wide tile's output offsets ((256 + 32) rows of y, and a dead column
    // offset of 2^31 plus 27 rows) stay in 32 bits
    const bool wide_ok = (int64_t)(256 + 32) * n * 4 <= 0x7FFFFFF0ll;
    if (wide_ok && costw < cost64 && costw < cost96) {
        hipLaunchKernelGGL((q8_0_gemm_wide_kernel<F8ACC>), dim3((unsigned)wide), dim3(512), 0, as_stream(stream), w,
                           w_row_bytes, xq, xds, y, m, k, n);
    } else if (cost96 < cost64) {
        hipLaunchKernelGGL((q8_0_gemm_kernel<F8ACC, 3>), dim3((unsigned)tiles96), dim3(768), 0, as_stream(stream), w,
                           w_row_bytes, xq, xds, y, m, k, n);
    } else {
        hipLaunchKernelGGL((q8_0_gemm_kernel<F8ACC, 2>), dim3((unsigned)tiles64), dim3(512), 0, as_stream(stream), w,
                           w_row_bytes, xq, xds, y, m, k, n);
    }
    return launch_status();
}

}  // namespace bqm

extern "C" int bqm_q8_0_gemm(const uint8_t *w, int64_t w_row_bytes, const int8_t *xq, const float *xds, float *y,
                             int m, int k, int n, void *stream) {
    return bqm::launch_mmq<false>(w, w_row_bytes, xq, xds, y, m, k, n, stream);
}

extern "C" int bqm_q8_0_gemm_f8acc(const uint8_t *w, int64_t w_row_bytes, const int8_t *xq, const float *xds,
                                   float *y, int m, int k, int n, void *stream) {
    return bqm::launch_mmq<true>(w, w_row_bytes, xq, xds, y, m, k, n, stream);
}
