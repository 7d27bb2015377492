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
//    Measured on gfx950: with four waves per SIMD a wave64 f32 fma issues
//    about every 2.9 clk (two VALU instructions of different waves can issue
//    together) but v_cvt_f32_i32 only every 4.4 clk, so the fold costs about
//    90 clk per 32x32 tile and block, the int8 MFMA 35 and the scale-product
//    MFMA 32 (per block, two blocks per instruction); in a register-only
//    probe the three take 142 clk together, the floor of this design (83 us
//    at m=512, K=4096, N=20480 with a 2.2 GHz shader clock).
//  * Workgroup: 16 waves, one per CU (four per SIMD, at most 128 VGPRs each),
//    over a 128-token x 64-row output tile.  Waves 0-7 and 8-15 form two
//    k-groups with the same eight 32x32 wave tiles: in iteration i k-group g
//    computes the 128-k stage 2i + g, and at the end group 1's partial sums
//    meet group 0's in LDS in a fixed order.  Four waves per SIMD keep the
//    VALU issuing while some wait on LDS or the barrier (with two waves per
//    SIMD, one stalled wave halves the VALU rate).
//  * LDS holds two iterations (the one computed and the one being filled)
//    of two stages each, 30 KB per stage.  One iteration's global loads are
//    in registers while the previous one is computed; they are stored to the
//    other buffer during the stage (activations after block 0, weights and
//    scales after block 2, so the LDS writes overlap the fold), and one
//    barrier ends an iteration.
//  * Weight rows are 34-byte blocks whose quants are 2-byte aligned.  Every
//    thread loads one quarter-block (16 quants) from its 68-byte block pair
//    (4-byte aligned) with a 16-byte and a 4-byte load; an even block's
//    quarter is realigned from the five dwords with v_alignbit.  Dense quants
//    and f32 scales go to LDS.
//  * Quant tiles are stored with a padded row stride of 144 bytes (128 + 16),
//    so the MFMA operand reads of 8 consecutive rows at the same k hit
//    distinct banks and every LDS address is a per-lane base plus a
//    compile-time offset.
//  * XCD-aware tile order (below), and range-checked buffer loads: ragged m
//    and n tails read zeros (zero scales), and only in-range outputs are
//    stored.
//  * Measured against the previous design (8 waves, two per SIMD, 128 x 64
//    tiles, 256-k stages, loads two stages ahead), interleaved on one box:
//    N=20480 152.8 against 163.3 us, N=4096 36.1 against 37.8; N=5152 63 against
//    58 (81 column tiles leave a ragged second round either way).  Ablations
//    of this kernel at N=20480: without the global loads 141.5 us, also
//    without the LDS stores 115, also without the barriers 108: the compute
//    from LDS is 108 us against the 83 us register-only floor.
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
constexpr int kMmqBN = 64;                   // weight rows per workgroup tile
constexpr int kMmqSK = 128;                  // k values per stage = 4 blocks
constexpr int kMmqSB = kMmqSK / kQK;         // 4
constexpr int kMmqThreads = 1024;            // 16 waves: 2 k-groups x (4 x 2) output waves
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
struct MmqStage {
    uint8_t x[kMmqBM * kMmqStride];
    uint8_t w[kMmqBN * kMmqStride];
    float dx[kMmqSB][kMmqBM + 4];
    float dw[kMmqSB][kMmqBN + 4];
};
// two buffers (the iteration computed and the one being filled) x two k-groups
static_assert(4 * sizeof(MmqStage) <= 160 * 1024, "LDS");
static_assert(kMmqBM * kMmqBN * 4 <= 2 * sizeof(MmqStage), "the k-group reduction reuses two stage buffers");

// Global loads of one iteration (two stages, 256 k), held in registers until
// stored to LDS: two 16-byte activation chunks, one quarter-block of weights
// (16 quants, from a 16-byte and a 4-byte load) and one activation scale per
// thread.
struct MmqRegs {
    u32x4 x[2];
    u32x4 w;
    uint32_t w4;
    float dx;
};

template <bool F8ACC>
__global__ __launch_bounds__(kMmqThreads) void q8_0_gemm_kernel(const uint8_t *__restrict__ w, int64_t w_row_bytes,
                                                                const int8_t *__restrict__ xq,
                                                                const float *__restrict__ xds, float *__restrict__ y,
                                                                int m, int k, int n) {
    __shared__ __attribute__((aligned(16))) MmqStage st[2][2];   // [buffer][k-group]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int grp = wave >> 3;                 // k-group: stages 2i + grp of iteration i
    const int wm = (wave >> 1) & 3, wn = wave & 1;
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
    const int nit = k / (2 * kMmqSK);

    // Resources covering the valid rows only; out-of-range loads return zeros.
    const __amdgpu_buffer_rsrc_t rX = mmq_rsrc(xq + (int64_t)m0 * k, (int64_t)(m - m0) * k);
    const __amdgpu_buffer_rsrc_t rD = mmq_rsrc(xds + (int64_t)m0 * nb * 2, (int64_t)(m - m0) * nb * 8);
    const __amdgpu_buffer_rsrc_t rW = mmq_rsrc(w + (int64_t)n0 * w_row_bytes, (int64_t)(n - n0) * w_row_bytes);

    // Load slots, fixed for the kernel (the iteration's offset is a uniform
    // scalar added by the buffer load).
    //  X: chunk q = tid + 1024*j of the 128 x 256-byte activation tile: row
    //     q >> 4, 16-byte chunk q & 15 (chunks 0..7 stage 0, 8..15 stage 1).
    //  dX: (row tid >> 3, block tid & 7), the d of each (d, s) pair.
    //  W: quarter-block q = tid of the 64 x 8-block weight tile: row q >> 4,
    //     block bb = (q >> 1) & 7, half h = q & 1.  Blocks pair up into 68-byte
    //     pairs (4-byte aligned): the even block's quants sit 2 bytes into the
    //     pair and are realigned from five dwords, the odd block's are aligned.
    uint32_t xoff[2];
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const int q = tid + kMmqThreads * j;
        xoff[j] = (uint32_t)((q >> 4) * k + 16 * (q & 15));
    }
    const uint32_t doff = (uint32_t)(((tid >> 3) * nb + (tid & 7)) * 8);
    const int wrow = tid >> 4, wbb = (tid >> 1) & 7, wh = tid & 1;
    const int wodd = wbb & 1;
    const int wsel = 2 * wodd + wh;           // 0: even h0, 1: even h1, 2: odd h0, 3: odd h1
    const uint32_t wpair = (uint32_t)(wrow * w_row_bytes + kMmqPairBytes * (wbb >> 1));
    const uint32_t woff16 = wpair + (wsel == 0 ? 0u : wsel == 1 ? 16u : wsel == 2 ? 36u : 52u);
    const uint32_t woff4 = wpair + (wsel == 0 ? 16u : wsel == 1 ? 32u : wsel == 2 ? 32u : 48u);

    auto load_iter = [&](MmqRegs &R, int it) {
        const int sx = it * 2 * kMmqSK, sw = it * 4 * kMmqPairBytes, sd = it * 8 * 8;
#pragma unroll
        for (int j = 0; j < 2; j++)
            R.x[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rX, xoff[j], sx, 0));
        R.w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rW, woff16, sw, 0));
        R.w4 = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rW, woff4, sw, 0);
        R.dx = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rD, doff, sd, 0));
    };
    auto store_x = [&](MmqStage *S, const MmqRegs &R) {
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int q = tid + kMmqThreads * j;
            const int row = q >> 4, c = q & 15;
            *reinterpret_cast<u32x4 *>(S[c >> 3].x + row * kMmqStride + 16 * (c & 7)) = R.x[j];
        }
    };
    auto store_wd = [&](MmqStage *S, const MmqRegs &R) {
        // even block: quants = bytes 2.. of dwords (w[0..3], w4); odd: w itself
        u32x4 qv;
        qv[0] = __builtin_amdgcn_alignbit(R.w[1], R.w[0], 16u);
        qv[1] = __builtin_amdgcn_alignbit(R.w[2], R.w[1], 16u);
        qv[2] = __builtin_amdgcn_alignbit(R.w[3], R.w[2], 16u);
        qv[3] = __builtin_amdgcn_alignbit(R.w4, R.w[3], 16u);
        if (wodd) qv = R.w;
        const int sg = wbb >> 2, bs = wbb & 3;
        *reinterpret_cast<u32x4 *>(S[sg].w + wrow * kMmqStride + 64 * wh + 16 * bs) = qv;
        if (wh == 0) S[sg].dw[bs][wrow] = half_bits_to_float(wodd ? (R.w4 >> 16) : (R.w[0] & 0xFFFFu));
        S[(tid & 7) >> 2].dx[tid & 3][tid >> 3] = R.dx;
    };
    auto store_iter = [&](MmqStage *S, const MmqRegs &R) {
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
    // One stage of 4 blocks for this wave's 32x32 tile.  The scale products
    // d_x[t][b] * d_w[r][b] come from the matrix core: one
    // v_mfma_f32_32x32x1_2b_f32 forms the 32x32 outer products of two blocks
    // (lanes 0-31 carry block b, lanes 32-63 block b+1; each result element is
    // one correctly rounded f32 product, as a VALU multiply would give), in the
    // block sums' register layout.  That leaves two VALU ops per output and
    // block, convert S then fma, the work that bounds this kernel; four waves
    // per SIMD keep the VALU busy while any one of them waits.
    auto compute_stage = [&](const MmqStage &S, auto &&mid) {
        const uint8_t *xa = S.x + arow * kMmqStride + 16 * khalf;
        const uint8_t *wb = S.w + brow * kMmqStride + 64 * khalf;
        const v32f z32 = {0};
        v4i A = *reinterpret_cast<const v4i *>(xa);
        v4i B = *reinterpret_cast<const v4i *>(wb);
#pragma unroll
        for (int p = 0; p < kMmqSB / 2; p++) {
            const float sa = S.dx[2 * p + khalf][arow], sb = S.dw[2 * p + khalf][brow];
            const v32f P = __builtin_amdgcn_mfma_f32_32x32x1f32(sa, sb, z32, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 2; e++) {
                const int b = 2 * p + e;
                const BlockSum Sb = block_sum(A, B);
                if (b + 1 < kMmqSB) {
                    A = *reinterpret_cast<const v4i *>(xa + 32 * (b + 1));
                    B = *reinterpret_cast<const v4i *>(wb + 16 * (b + 1));
                }
#pragma unroll
                for (int v = 0; v < 16; v++) {
                    if constexpr (F8ACC)
                        acc[v] = __builtin_fmaf(Sb[v], P[16 * e + v], acc[v]);
                    else
                        acc[v] = __builtin_fmaf((float)Sb[v], P[16 * e + v], acc[v]);
                }
                asm volatile("" : "+v"(acc) :: "memory");
                mid(b);
            }
        }
    };

    // Iteration i: k-group g computes stage 2i + g from LDS buffer i % 2 while
    // the registers hold iteration i + 1's loads; those are then stored to the
    // other buffer, iteration i + 2's loads issued (unconditional: past the
    // end they re-read the last iteration, so the compiler's count of loads in
    // flight stays exact), and one barrier ends the iteration.
    MmqRegs R;
    const int last = nit - 1;
    load_iter(R, 0);
    store_iter(st[0], R);
    load_iter(R, min(1, last));
    __syncthreads();
#pragma unroll 1
    for (int it = 0; it < nit; it++) {
        const int cur = it & 1;
        // the next iteration's stores spread over this stage: activations
        // after block 0, weights and scales after block 2 (the other buffer is
        // not read in this iteration)
        const bool more = it + 1 < nit;
        compute_stage(st[cur][grp], [&](int b) {
            if (b == 0 && more) store_x(st[cur ^ 1], R);
            if (b == 2 && more) store_wd(st[cur ^ 1], R);
        });
        load_iter(R, min(it + 2, last));
        __syncthreads();
    }

    // The two k-groups' partial sums meet in LDS: group 1 stores, group 0
    // adds (its own + group 1's, a fixed order) and writes y.  Output element
    // (row 8*(v/4) + 4*khalf + v%4, column lane%32) of the wave tile.
    float *red = reinterpret_cast<float *>(&st[0][0]);
    float *mine = red + ((wm * 2 + wn) * 16) * 64 + lane;
    if (grp == 1) {
#pragma unroll
        for (int v = 0; v < 16; v++) mine[v * 64] = acc[v];
    }
    __syncthreads();
    if (grp == 0) {
        const int col = n0 + wn * 32 + (lane & 31);
        if (col < n) {
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int row = m0 + wm * 32 + 8 * (v >> 2) + 4 * khalf + (v & 3);
                if (row < m) y[(int64_t)row * n + col] = acc[v] + mine[v * 64];
            }
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
    // per-workgroup offsets are 32-bit: 128 rows of activations, 64 of weights
    if ((int64_t)kMmqBM * k > 0x7FFFFFF0ll || (int64_t)kMmqBN * w_row_bytes > 0x7FFFFFF0ll) return BQM_EUNSUPPORTED;
    const int64_t tiles = (int64_t)((n + kMmqBN - 1) / kMmqBN) * ((m + kMmqBM - 1) / kMmqBM);
    if (tiles > 0x7FFFFFFF) return BQM_EUNSUPPORTED;
    hipLaunchKernelGGL((q8_0_gemm_kernel<F8ACC>), dim3((unsigned)tiles), dim3(kMmqThreads), 0, as_stream(stream), w,
                       w_row_bytes, xq, xds, y, m, k, n);
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
