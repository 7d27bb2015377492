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
//    compute_stage), which leaves two VALU ops per element and block.
//    Without packed f32 the VALU retires a wave64 op every 4 clk, so the fold
//    takes 128 clk per 32x32 tile and block against about 32 clk of int8 MFMA.
//    The MFMA of block b+1 is issued before the fold of block b, and the LDS
//    operands are read two blocks ahead, so the matrix core, the LDS and the
//    VALU overlap.  MFMA results stay in ordinary VGPRs (the build asks for
//    the VGPR form), so the fold reads them without copies.
//  * Workgroup tile BM tokens x 64 weight rows, BM/16 waves of 32x32; k is
//    staged 256 values (8 blocks) at a time into double-buffered LDS, and the
//    global loads run two stages ahead in a register double buffer to cover
//    L2 and Infinity Cache latency (one barrier per stage).  BM = 128 (8
//    waves, one workgroup per CU) loads a quarter less per output than BM =
//    64 (4 waves, two workgroups per CU): per output a workgroup reads 1/64
//    of a weight row plus 1/BM of an activation row, and the vector memory
//    pipeline, not the matrix cores, is what the loads contend for.  The
//    taller tile is used when its workgroups fill whole rounds of the CUs
//    (measured: 10% faster at m=512, N=4096 and 20480, but slower wherever a
//    partial last round or fewer tiles than CUs remain).
//  * Weight rows are 34-byte blocks whose quants are 2-byte aligned.  A
//    68-byte block pair (4-byte aligned) is loaded by two threads straight
//    into registers: one takes dwords 0..8 and realigns the even block with
//    v_alignbit, the other dwords 8..16 (the odd block, already aligned);
//    each writes dense quants plus its f32 scale to LDS.
//  * Quant tiles are stored with a padded row stride of 272 bytes (256 + 16),
//    so the MFMA operand reads of 8 consecutive rows at the same k hit
//    distinct banks and every LDS address is a per-lane base plus a
//    compile-time offset.
//  * Global loads are range-checked buffer loads: ragged m and n tails read
//    zeros (zero scales), and only in-range outputs are stored.
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

constexpr int kMmqBN = 64;
constexpr int kMmqKB = 256;                  // k values per stage = 8 blocks
constexpr int kMmqBlocks = kMmqKB / kQK;     // 8
constexpr int kMmqPairBytes = 2 * kQ80Bytes; // 68
constexpr int kMmqRowStride = kMmqKB + 16;   // 272: padded LDS row of quants

__device__ __forceinline__ __amdgpu_buffer_rsrc_t mmq_rsrc(const void *base, int64_t bytes) {
    uint32_t b = bytes <= 0 ? 0u : (bytes > 0x7FFFFFF0ll ? 0x7FFFFFF0u : (uint32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)b, 0x00020000);
}

template <int BM>
struct MmqStage {
    uint8_t x[BM * kMmqRowStride];       // activation quants, padded rows
    uint8_t w[kMmqBN * kMmqRowStride];   // weight quants, padded rows: first halves of the 8 blocks, then second halves
    // d_x / d_w per block and row.  A row of blocks is padded by 4 floats:
    // the stores write 8 blocks of 4 (d_w) or 8 (d_x) rows per 32 lanes, and a
    // ds_write_b32 serves 32 lanes from 32 banks of 4 bytes, so block rows
    // must differ by 4 mod 32 banks (with 8 floats of padding, blocks b and
    // b+4 met in one bank; measured: 27% fewer LDS bank conflicts).
    float dx[kMmqBlocks][BM + 4];
    float dw[kMmqBlocks][kMmqBN + 4];
};
static_assert(2 * sizeof(MmqStage<128>) <= 160 * 1024, "one 128-row workgroup per CU");
static_assert(4 * sizeof(MmqStage<64>) <= 160 * 1024, "two 64-row workgroups per CU");

// Global loads of one stage, held in registers until written to LDS.  The
// 256 block pairs of a stage's weight tile are loaded as 512 halves, WH per
// thread.
template <int WH>
struct MmqRegs {
    u32x4 x[4];         // 4 activation chunks
    u32x4 w[WH][2];     // half a 68-byte weight block pair: dwords 0..7, or 9..16
    uint32_t w8[WH];    // and dword 8 (the odd block's scale sits in its high half)
    float dx[2];        // 2 (row, block) activation scales
};

template <int BM, bool F8ACC>
__global__ __launch_bounds__(4 * BM) void q8_0_gemm_kernel(const uint8_t *__restrict__ w, int64_t w_row_bytes,
                                                              const int8_t *__restrict__ xq,
                                                              const float *__restrict__ xds, float *__restrict__ y,
                                                              int m, int k, int n) {
    constexpr int kMmqThreads = 4 * BM;
    constexpr int WH = 512 / kMmqThreads;   // weight half-pairs per thread
    using Stage = MmqStage<BM>;
    using Regs = MmqRegs<WH>;
    __shared__ __attribute__((aligned(16))) Stage st[2];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    // XCD-aware tile order.  Workgroups are handed to the 8 XCDs round-robin
    // (id % 8), and each XCD has its own L2.  Renumber so that XCD x runs a
    // contiguous range of tiles, m-tile fastest: the token tiles that share a
    // weight tile then run together on one XCD and read it once into its L2.
    const int nm = (m + BM - 1) / BM;
    const int ntiles = gridDim.x;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int per = ntiles >> 3, extra = ntiles & 7;
    const int tile = xcd * per + min(xcd, extra) + slot;
    const int n0 = (tile / nm) * kMmqBN;
    const int m0 = (tile - (tile / nm) * nm) * BM;
    const int nb = k / kQK;
    const int nstage = k / kMmqKB;

    // Resources covering the valid rows only; out-of-range loads return zeros.
    const __amdgpu_buffer_rsrc_t rX = mmq_rsrc(xq + (int64_t)m0 * k, (int64_t)(m - m0) * k);
    const __amdgpu_buffer_rsrc_t rD = mmq_rsrc(xds + (int64_t)m0 * nb * 2, (int64_t)(m - m0) * nb * 8);
    const __amdgpu_buffer_rsrc_t rW = mmq_rsrc(w + (int64_t)n0 * w_row_bytes, (int64_t)(n - n0) * w_row_bytes);

    // This thread's load slots, as byte offsets fixed for the whole kernel; the
    // stage offset is a uniform scalar added by the buffer load (soffset).
    // X: 4 chunks (row q>>4, chunk q&15).  W: half-pairs h = tid + 4*BM*j,
    // half h&1 (0 the even block, 1 the odd one) of pair p = h>>1 (row p>>2,
    // pair p&3).  dX: 2 (row q>>3, block q&7), the d of each pair.
    int wrow[WH], wpair[WH], odd[WH];
    uint32_t wo0[WH], wo1[WH], wo2[WH];
#pragma unroll
    for (int j = 0; j < WH; j++) {
        const int h = tid + kMmqThreads * j;
        // the two halves of a pair sit in adjacent lanes, so a load instruction
        // covers 32 consecutive pairs densely (measured 6-10% faster than
        // even halves in one wave and odd halves in another)
        const int wp = h >> 1;
        odd[j] = h & 1;
        wrow[j] = wp >> 2;
        wpair[j] = wp & 3;
        const uint32_t wbase = (uint32_t)(wrow[j] * w_row_bytes + kMmqPairBytes * wpair[j]);
        // even: b128 at +0 and +16 (dwords 0..7), b32 at +32 (dword 8)
        // odd:  b128 at +36 and +52 (dwords 9..16), b32 at +32 (dword 8)
        wo0[j] = wbase + (odd[j] ? 36u : 0u);
        wo1[j] = wbase + (odd[j] ? 52u : 16u);
        wo2[j] = wbase + 32u;
    }
    uint32_t xoff[4], doff[2];
#pragma unroll
    for (int s = 0; s < 4; s++) {
        const int q = tid + kMmqThreads * s;
        xoff[s] = (uint32_t)((q >> 4) * k + 16 * (q & 15));
    }
#pragma unroll
    for (int s = 0; s < 2; s++) {
        const int q = tid + kMmqThreads * s;
        doff[s] = (uint32_t)(((q >> 3) * nb + (q & 7)) * 8);
    }
    auto load_stage = [&](Regs &R, int kc) {
        const int sx = kc * kMmqKB, sw = kc * (kMmqBlocks * kQ80Bytes), sd = kc * kMmqBlocks * 8;
#pragma unroll
        for (int s = 0; s < 4; s++)
            R.x[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rX, xoff[s], sx, 0));
#pragma unroll
        for (int j = 0; j < WH; j++) {
            R.w[j][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rW, wo0[j], sw, 0));
            R.w[j][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rW, wo1[j], sw, 0));
            R.w8[j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rW, wo2[j], sw, 0);
        }
#pragma unroll
        for (int s = 0; s < 2; s++)
            R.dx[s] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rD, doff[s], sd, 0));
    };
    auto store_stage = [&](Stage &S, const Regs &R) {
#pragma unroll
        for (int s = 0; s < 4; s++) {
            int q = tid + kMmqThreads * s;
            int row = q >> 4, c = q & 15;
            *reinterpret_cast<u32x4 *>(S.x + row * kMmqRowStride + 16 * c) = R.x[s];
        }
#pragma unroll
        for (int j = 0; j < WH; j++) {
            // the even block's quants start 2 bytes into dword 0: realign them
            // (an odd half's realigned words are computed too and not used)
            const uint32_t d[9] = {R.w[j][0][0], R.w[j][0][1], R.w[j][0][2], R.w[j][0][3],
                                   R.w[j][1][0], R.w[j][1][1], R.w[j][1][2], R.w[j][1][3], R.w8[j]};
            u32x4 qa0, qa1;
            qa0[0] = __builtin_amdgcn_alignbit(d[1], d[0], 16u);
            qa0[1] = __builtin_amdgcn_alignbit(d[2], d[1], 16u);
            qa0[2] = __builtin_amdgcn_alignbit(d[3], d[2], 16u);
            qa0[3] = __builtin_amdgcn_alignbit(d[4], d[3], 16u);
            qa1[0] = __builtin_amdgcn_alignbit(d[5], d[4], 16u);
            qa1[1] = __builtin_amdgcn_alignbit(d[6], d[5], 16u);
            qa1[2] = __builtin_amdgcn_alignbit(d[7], d[6], 16u);
            qa1[3] = __builtin_amdgcn_alignbit(d[8], d[7], 16u);
            // weight tile rows hold the first 16 bytes of blocks 0..7, then the
            // second 16 bytes of blocks 0..7: the 8 lanes of a row then store
            // 128 consecutive bytes per instruction (block-contiguous rows
            // made these stores 4-way bank-conflicted)
            const int b = 2 * wpair[j] + odd[j];
            uint8_t *wr = S.w + wrow[j] * kMmqRowStride + 16 * b;
            *reinterpret_cast<u32x4 *>(wr) = odd[j] ? R.w[j][0] : qa0;
            *reinterpret_cast<u32x4 *>(wr + 128) = odd[j] ? R.w[j][1] : qa1;
            S.dw[b][wrow[j]] = half_bits_to_float(odd[j] ? (R.w8[j] >> 16) : (d[0] & 0xFFFFu));
        }
#pragma unroll
        for (int s = 0; s < 2; s++) {
            int q = tid + kMmqThreads * s;
            S.dx[q & 7][q >> 3] = R.dx[s];
        }
    };

    v16f acc;
#pragma unroll
    for (int v = 0; v < 16; v++) acc[v] = 0.0f;

    // EARLY (the int8 128-row tile) moves the workgroup barrier into the
    // stage (below; measured N=4096 37.6 -> 35.5 us, N=20480 164.8 -> 162.0
    // us, bitwise the same).  The 64-row tile and the fp8 accumulator arm keep
    // the barrier after the stage: the state the early barrier keeps live
    // across it does not fit their registers (257 VGPRs or scratch).
    constexpr bool EARLY = BM == 128 && !F8ACC;
    if constexpr (EARLY) {
        const int arow = wm * 32 + (lane & 31);   // A operand row (token) of this lane
        const int brow = wn * 32 + (lane & 31);   // B operand row (weight row) of this lane
        const int khalf = lane >> 5;

        // One stage: 8 blocks.  Quant operands are read two blocks ahead and the
        // int8 MFMA runs one block ahead of the fold.  The scale products
        // d_x[t][b] * d_w[r][b] come from the matrix core as well: one
        // v_mfma_f32_32x32x1_2b_f32 forms the 32x32 outer products of two blocks
        // (lanes 0-31 carry block b, lanes 32-63 block b+1; each result element
        // is one correctly rounded f32 product, as a VALU multiply would give),
        // in the same register layout as the int32 block sums.  That leaves two
        // VALU ops per output and block: convert S, then fma into the
        // accumulator.  The outer products of a pair are issued one pair ahead.
        //
        // The workgroup barrier sits before the fold of blocks 6 and 7: the next
        // stage's stores are issued before it, and after it the next stage's
        // scales, first two blocks' operands and first MFMAs are issued under
        // those two folds, so no stage starts by waiting for its own LDS reads.
        // The operand slots, scales, partial products and block sums are kept
        // across stages.
        using BlockSum = typename std::conditional<F8ACC, v16f, v16i>::type;
        v4i A[3], B[3];
        float SA[kMmqBlocks / 2], SB[kMmqBlocks / 2];   // d_x[b + khalf][token], d_w[b + khalf][weight row] per pair
        v32f P[2];
        BlockSum Sn;
        const v32f z32 = {0};
        auto rd = [&](const Stage &S, int b, int slot) {
            A[slot] = *reinterpret_cast<const v4i *>(S.x + arow * kMmqRowStride + 16 * khalf + 32 * b);
            B[slot] = *reinterpret_cast<const v4i *>(S.w + brow * kMmqRowStride + 128 * khalf + 16 * b);
        };
        auto read_scales = [&](const Stage &S) {
    #pragma unroll
            for (int p = 0; p < kMmqBlocks / 2; p++) {
                SA[p] = S.dx[2 * p + khalf][arow];
                SB[p] = S.dw[2 * p + khalf][brow];
            }
        };
        // the block sums of one 32x32 tile: int32 from the int8 MFMA, or f32
        // from two fp8 MFMAs over the same bytes
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
        // the first block's MFMAs and operands of a stage (before its fold loop)
        auto start_stage = [&](const Stage &S) {
            read_scales(S);
            rd(S, 0, 0);
            rd(S, 1, 1);
            P[0] = __builtin_amdgcn_mfma_f32_32x32x1f32(SA[0], SB[0], z32, 0, 0, 0);
            Sn = block_sum(A[0], B[0]);
        };
        // block b of stage S; in blocks 6 and 7 the first reads and MFMAs of the
        // next stage (buffer N) are issued under the fold
        auto block = [&](const Stage &S, const Stage &N, int b) {
            if (b + 2 < kMmqBlocks) rd(S, b + 2, (b + 2) % 3);
            if (b == 6) {
                read_scales(N);   // pair 3's scale product was issued at block 4
                rd(N, 0, 0);      // slot 0 was last read by block 6's MFMA (issued at block 5)
            }
            const BlockSum Sc = Sn;
            if (b + 1 < kMmqBlocks) Sn = block_sum(A[(b + 1) % 3], B[(b + 1) % 3]);
            if ((b & 1) == 0 && b + 2 < kMmqBlocks)
                P[((b + 2) >> 1) & 1] = __builtin_amdgcn_mfma_f32_32x32x1f32(SA[(b + 2) >> 1], SB[(b + 2) >> 1], z32, 0, 0, 0);
            if (b == 7) {
                rd(N, 1, 1);      // slot 1 was last read by block 7's MFMA (issued at block 6)
                P[0] = __builtin_amdgcn_mfma_f32_32x32x1f32(SA[0], SB[0], z32, 0, 0, 0);   // P[0] held pair 2
            }
            // Issue those MFMAs before the fold below (they then run under the
            // fold's VALU work instead of stalling the next block's fold): the
            // empty asm claims to modify the accumulators, so no fold instruction
            // can move above it, and it reads Sn, so the block-sum MFMA cannot
            // move below it.
            asm volatile("" : "+v"(Sn), "+v"(acc));
            const v32f &Pc = P[(b >> 1) & 1];
            const int h = 16 * (b & 1);
    #pragma unroll
            for (int v = 0; v < 16; v++) {
                if constexpr (F8ACC)
                    acc[v] = __builtin_fmaf(Sc[v], Pc[h + v], acc[v]);
                else
                    acc[v] = __builtin_fmaf((float)Sc[v], Pc[h + v], acc[v]);
            }
            if (b == 7) Sn = block_sum(A[0], B[0]);   // the next stage's block 0
            // Keep each block's group (reads for b+2, MFMAs for b+1, fold of b) in
            // this order: an empty asm that reads and writes the accumulators stops
            // the compiler from hoisting every block's loads and MFMAs to the top
            // (which costs registers and serializes the fold behind them).  The
            // empty asm emits no instruction.
            asm volatile("" : "+v"(acc) :: "memory");
        };
        auto pre = [&](const Stage &S, const Stage &N) {
    #pragma unroll
            for (int b = 0; b < kMmqBlocks - 2; b++) block(S, N, b);
        };
        auto post = [&](const Stage &S, const Stage &N) {
            block(S, N, kMmqBlocks - 2);
            block(S, N, kMmqBlocks - 1);
        };

        // The loads are unconditional (past the last stage they re-read it, an L2
        // hit): with a branch around them the compiler cannot count the loads in
        // flight, and its wait before writing the older register buffer to LDS
        // would then also wait for the loads just issued.  Past the last stage
        // the next-stage reads of blocks 6 and 7 read a stale buffer; their
        // results are never folded.
        Regs R0, R1;
        const int last = nstage - 1;
        load_stage(R0, 0);
        load_stage(R1, min(1, last));
        store_stage(st[0], R0);
        __syncthreads();
        start_stage(st[0]);
        for (int kc = 0; kc < nstage; kc += 2) {
            // st[0] holds stage kc; R1 holds stage kc+1 (in flight)
            load_stage(R0, min(kc + 2, last));
            pre(st[0], st[1]);
            if (kc + 1 < nstage) store_stage(st[1], R1);
            __syncthreads();
            post(st[0], st[1]);
            if (kc + 1 < nstage) {
                load_stage(R1, min(kc + 3, last));
                pre(st[1], st[0]);
                if (kc + 2 < nstage) store_stage(st[0], R0);
                __syncthreads();
                post(st[1], st[0]);
            }
        }

    } else {
        const int arow = wm * 32 + (lane & 31);   // A operand row (token) of this lane
        const int brow = wn * 32 + (lane & 31);   // B operand row (weight row) of this lane
        const int khalf = lane >> 5;

        // One stage: 8 blocks.  Quant operands are read two blocks ahead and the
        // int8 MFMA runs one block ahead of the fold.  The scale products
        // d_x[t][b] * d_w[r][b] come from the matrix core as well: one
        // v_mfma_f32_32x32x1_2b_f32 forms the 32x32 outer products of two blocks
        // (lanes 0-31 carry block b, lanes 32-63 block b+1; each result element
        // is one correctly rounded f32 product, as a VALU multiply would give),
        // in the same register layout as the int32 block sums.  That leaves two
        // VALU ops per output and block: convert S, then fma into the
        // accumulator.  The outer products of a pair are issued one pair ahead.
        auto compute_stage = [&](const Stage &S) {
            v4i A[3], B[3];
            const uint8_t *xa = S.x + arow * kMmqRowStride + 16 * khalf;
            const uint8_t *wb = S.w + brow * kMmqRowStride + 128 * khalf;
            auto rd = [&](int b, int slot) {
                A[slot] = *reinterpret_cast<const v4i *>(xa + 32 * b);
                B[slot] = *reinterpret_cast<const v4i *>(wb + 16 * b);
            };
            // scale operands of the 4 block pairs: d_x[b + khalf][token], d_w[b + khalf][weight row]
            float SA[kMmqBlocks / 2], SB[kMmqBlocks / 2];
    #pragma unroll
            for (int p = 0; p < kMmqBlocks / 2; p++) {
                SA[p] = S.dx[2 * p + khalf][arow];
                SB[p] = S.dw[2 * p + khalf][brow];
            }
            const v32f z32 = {0};
            v32f P[2];
            rd(0, 0);
            rd(1, 1);
            P[0] = __builtin_amdgcn_mfma_f32_32x32x1f32(SA[0], SB[0], z32, 0, 0, 0);
            // the block sums of one 32x32 tile: int32 from the int8 MFMA, or f32
            // from two fp8 MFMAs over the same bytes
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
            BlockSum Sn = block_sum(A[0], B[0]);
    #pragma unroll
            for (int b = 0; b < kMmqBlocks; b++) {
                if (b + 2 < kMmqBlocks) rd(b + 2, (b + 2) % 3);
                const BlockSum Sc = Sn;
                if (b + 1 < kMmqBlocks) Sn = block_sum(A[(b + 1) % 3], B[(b + 1) % 3]);
                if ((b & 1) == 0 && b + 2 < kMmqBlocks)
                    P[((b + 2) >> 1) & 1] =
                        __builtin_amdgcn_mfma_f32_32x32x1f32(SA[(b + 2) >> 1], SB[(b + 2) >> 1], z32, 0, 0, 0);
                // Issue those MFMAs before the fold below (they then run under the
                // fold's VALU work instead of stalling the next block's fold): the
                // empty asm claims to modify the accumulators, so no fold
                // instruction can move above it, and it reads Sn, so the block-sum
                // MFMA cannot move below it.
                asm volatile("" : "+v"(Sn), "+v"(acc));
                const v32f &Pc = P[(b >> 1) & 1];
                const int h = 16 * (b & 1);
    #pragma unroll
                for (int v = 0; v < 16; v++) {
                    if constexpr (F8ACC)
                        acc[v] = __builtin_fmaf(Sc[v], Pc[h + v], acc[v]);
                    else
                        acc[v] = __builtin_fmaf((float)Sc[v], Pc[h + v], acc[v]);
                }
                // Keep each block's group (reads for b+2, MFMAs for b+1, fold of
                // b) in this order: an empty asm that reads and writes the
                // accumulators stops the compiler from hoisting every block's loads
                // and MFMAs to the top (which costs registers and serializes the
                // fold behind them).  The empty asm emits no instruction.
                asm volatile("" : "+v"(acc) :: "memory");
            }
        };

        // The loads are unconditional (past the last stage they re-read it, an L2
        // hit): with a branch around them the compiler cannot count the loads in
        // flight, and its wait before writing the older register buffer to LDS
        // would then also wait for the loads just issued.
        Regs R0, R1;
        const int last = nstage - 1;
        load_stage(R0, 0);
        load_stage(R1, min(1, last));
        store_stage(st[0], R0);
        __syncthreads();
        for (int kc = 0; kc < nstage; kc += 2) {
            // st[0] holds stage kc; R1 holds stage kc+1 (in flight)
            load_stage(R0, min(kc + 2, last));
            compute_stage(st[0]);
            if (kc + 1 < nstage) store_stage(st[1], R1);
            __syncthreads();
            if (kc + 1 < nstage) {
                load_stage(R1, min(kc + 3, last));
                compute_stage(st[1]);
                if (kc + 2 < nstage) store_stage(st[0], R0);
                __syncthreads();
            }
        }

    }

    // Output element (row 8*(v/4) + 4*khalf + v%4, column lane%32) of the wave tile.
    const int khalf = lane >> 5;
    const int col = n0 + wn * 32 + (lane & 31);
    if (col < n) {
#pragma unroll
        for (int v = 0; v < 16; v++) {
            int row = m0 + wm * 32 + 8 * (v >> 2) + 4 * khalf + (v & 3);
            if (row < m) y[(int64_t)row * n + col] = acc[v];
        }
    }
}

template <int BM, bool F8ACC>
static int launch_tiles(const uint8_t *w, int64_t w_row_bytes, const int8_t *xq, const float *xds, float *y, int m,
                        int k, int n, int64_t tiles, hipStream_t s) {
    if (tiles > 0x7FFFFFFF) return BQM_EUNSUPPORTED;
    hipLaunchKernelGGL((q8_0_gemm_kernel<BM, F8ACC>), dim3((unsigned)tiles), dim3(4 * BM), 0, s, w, w_row_bytes, xq,
                       xds, y, m, k, n);
    return launch_status();
}

// Checks shared by both arms, the tile height, then the launch.  The
// 128-row tile runs one workgroup per CU, so it is taken only when its
// workgroups fill whole rounds of the CUs, the last round at least 3/4 full.
template <bool F8ACC>
static int launch_mmq(const uint8_t *w, int64_t w_row_bytes, const int8_t *xq, const float *xds, float *y, int m,
                      int k, int n, void *stream) {
    if (!w || !xq || !xds || !y) return BQM_EINVAL;
    if (m < 1 || k < 256 || n < 1) return BQM_EINVAL;
    if (k % 256 != 0) return BQM_EUNSUPPORTED;
    if (w_row_bytes < (int64_t)(k / kQK) * kQ80Bytes || w_row_bytes % 16 != 0) return BQM_EUNSUPPORTED;
    if (!aligned(w, 16) || !aligned(xq, 16) || !aligned(xds, 8) || !aligned(y, 4)) return BQM_EUNSUPPORTED;
    // per-workgroup offsets are 32-bit: 128 rows of activations, 64 of weights
    if ((int64_t)128 * k > 0x7FFFFFF0ll || (int64_t)kMmqBN * w_row_bytes > 0x7FFFFFF0ll) return BQM_EUNSUPPORTED;
    const int64_t ntiles = (n + kMmqBN - 1) / kMmqBN;
    const int64_t tall = ntiles * ((m + 127) / 128);
    const int64_t cus = device_cus();
    const int64_t last = tall % cus;
    hipStream_t s = as_stream(stream);
    if (tall >= cus && (last == 0 || 4 * last >= 3 * cus))
        return launch_tiles<128, F8ACC>(w, w_row_bytes, xq, xds, y, m, k, n, tall, s);
    return launch_tiles<64, F8ACC>(w, w_row_bytes, xq, xds, y, m, k, n, ntiles * ((m + 63) / 64), s);
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
