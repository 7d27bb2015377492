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
//    gives S for a 32x32 output tile and one block; its int32 result is
//    folded at once (cvt, scale product, fma).  The fold runs on the VALU
//    and bounds the kernel; the matrix cores are idle most of the time.
//  * Workgroup tile 64 tokens x 64 weight rows, 4 waves of 32x32, K staged
//    256 values (8 blocks) at a time.  Global loads are coalesced 16-byte
//    buffer loads (range-checked in hardware: ragged m and n tails read
//    zeros), prefetched into registers one stage ahead.
//  * Weight rows arrive in 34-byte blocks whose quants are 2-byte aligned;
//    the raw bytes are staged in LDS, then realigned with v_alignbit into a
//    dense quant tile and an f32 scale array.
//  * Quant tiles use a 16-byte-chunk XOR swizzle (chunk ^ (row & 7)) so the
//    MFMA operand reads of 8 consecutive rows hit distinct banks.
#include "bqmm_internal.h"

namespace bqm {

constexpr int kMmqBM = 64;
constexpr int kMmqBN = 64;
constexpr int kMmqKB = 256;                  // k values per stage = 8 blocks
constexpr int kMmqBlocks = kMmqKB / kQK;     // 8
constexpr int kMmqRawRow = kMmqBlocks * kQ80Bytes;   // 272 bytes
constexpr int kMmqThreads = 256;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t mmq_rsrc(const void *base, int64_t bytes) {
    uint32_t b = bytes <= 0 ? 0u : (bytes > 0x7FFFFFF0ll ? 0x7FFFFFF0u : (uint32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)b, 0x00020000);
}

__global__ __launch_bounds__(kMmqThreads) void q8_0_gemm_kernel(const uint8_t *__restrict__ w, int64_t w_row_bytes,
                                                              const int8_t *__restrict__ xq,
                                                              const float *__restrict__ xds, float *__restrict__ y,
                                                              int m, int k, int n) {
    __shared__ __attribute__((aligned(16))) uint8_t sX[kMmqBM * kMmqKB];        // swizzled quants
    __shared__ __attribute__((aligned(16))) uint8_t sW[kMmqBN * kMmqKB];        // swizzled quants
    __shared__ __attribute__((aligned(16))) uint8_t sWraw[kMmqBN * kMmqRawRow];  // raw 34-byte blocks
    __shared__ float sDX[kMmqBlocks][kMmqBM];
    __shared__ float sDW[kMmqBlocks][kMmqBN];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int n0 = blockIdx.x * kMmqBN;
    const int m0 = blockIdx.y * kMmqBM;
    const int nb = k / kQK;
    const int nstage = k / kMmqKB;

    // Resources covering the valid rows only; out-of-range loads return zeros.
    const __amdgpu_buffer_rsrc_t rX = mmq_rsrc(xq + (int64_t)m0 * k, (int64_t)(m - m0) * k);
    const __amdgpu_buffer_rsrc_t rD = mmq_rsrc(xds + (int64_t)m0 * nb * 2, (int64_t)(m - m0) * nb * 8);
    const __amdgpu_buffer_rsrc_t rW = mmq_rsrc(w + (int64_t)n0 * w_row_bytes, (int64_t)(n - n0) * w_row_bytes);

    // Per-thread load slots.  X: 1024 chunks, 4 per thread.  Wraw: 1088 chunks,
    // 5 slots (the fifth for tid < 64).  dX: 512 floats, 2 per thread.
    u32x4 rx[4], rw[5];
    float rdx[2];
    auto load_stage = [&](int kc) {
#pragma unroll
        for (int s = 0; s < 4; s++) {
            int q = tid + 256 * s;
            int row = q >> 4, c = q & 15;
            uint32_t off = (uint32_t)(row * k + kc * kMmqKB + 16 * c);
            rx[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rX, off, 0, 0));
        }
#pragma unroll
        for (int s = 0; s < 5; s++) {
            int q = tid + 256 * s;
            int row = q / 17, c = q - row * 17;
            uint32_t off = (q < kMmqBN * 17) ? (uint32_t)(row * w_row_bytes + kc * kMmqRawRow + 16 * c) : 0xFFFFFFF0u;
            rw[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rW, off, 0, 0));
        }
#pragma unroll
        for (int s = 0; s < 2; s++) {
            int q = tid + 256 * s;
            int row = q >> 3, b = q & 7;
            uint32_t off = (uint32_t)(((int64_t)row * nb + kc * kMmqBlocks + b) * 8);
            rdx[s] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rD, off, 0, 0));
        }
    };
    auto store_stage = [&]() {
#pragma unroll
        for (int s = 0; s < 4; s++) {
            int q = tid + 256 * s;
            int row = q >> 4, c = q & 15;
            *reinterpret_cast<u32x4 *>(sX + row * kMmqKB + 16 * (c ^ (row & 7))) = rx[s];
        }
#pragma unroll
        for (int s = 0; s < 5; s++) {
            int q = tid + 256 * s;
            if (q < kMmqBN * 17) *reinterpret_cast<u32x4 *>(sWraw + 16 * q) = rw[s];
        }
#pragma unroll
        for (int s = 0; s < 2; s++) {
            int q = tid + 256 * s;
            sDX[q & 7][q >> 3] = rdx[s];
        }
    };

    v16f acc;
#pragma unroll
    for (int v = 0; v < 16; v++) acc[v] = 0.0f;

    const int arow = wm * 32 + (lane & 31);   // A operand row (token) of this lane
    const int brow = wn * 32 + (lane & 31);   // B operand row (weight row) of this lane
    const int khalf = lane >> 5;

    load_stage(0);
    for (int kc = 0; kc < nstage; kc++) {
        store_stage();
        __syncthreads();
        if (kc + 1 < nstage) load_stage(kc + 1);
        // realign 64 rows x 8 blocks: 2 (row, block) items per thread
#pragma unroll
        for (int s = 0; s < 2; s++) {
            int it = tid + 256 * s;
            int row = it & 63, b = it >> 6;
            const uint32_t *rp = reinterpret_cast<const uint32_t *>(sWraw + row * kMmqRawRow + 68 * (b >> 1));
            uint32_t q[8];
            uint32_t sbits;
            if ((b & 1) == 0) {
                uint32_t dw[9];
#pragma unroll
                for (int d = 0; d < 9; d++) dw[d] = rp[d];
                sbits = dw[0] & 0xFFFFu;
#pragma unroll
                for (int d = 0; d < 8; d++) q[d] = __builtin_amdgcn_alignbit(dw[d + 1], dw[d], 16u);
            } else {
                sbits = rp[8] >> 16;
#pragma unroll
                for (int d = 0; d < 8; d++) q[d] = rp[9 + d];
            }
            u32x4 lo = {q[0], q[1], q[2], q[3]}, hi = {q[4], q[5], q[6], q[7]};
            *reinterpret_cast<u32x4 *>(sW + row * kMmqKB + 16 * ((2 * b) ^ (row & 7))) = lo;
            *reinterpret_cast<u32x4 *>(sW + row * kMmqKB + 16 * ((2 * b + 1) ^ (row & 7))) = hi;
            sDW[b][row] = half_bits_to_float(sbits);
        }
        __syncthreads();
#pragma unroll 2
        for (int b = 0; b < kMmqBlocks; b++) {
            int c = 2 * b + khalf;
            v4i a = *reinterpret_cast<const v4i *>(sX + arow * kMmqKB + 16 * (c ^ (arow & 7)));
            v4i bb = *reinterpret_cast<const v4i *>(sW + brow * kMmqKB + 16 * (c ^ (brow & 7)));
            v16i z = {0};
            v16i S = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bb, z, 0, 0, 0);
            float dw = sDW[b][brow];
            const float *dxp = &sDX[b][wm * 32 + 4 * khalf];
#pragma unroll
            for (int qd = 0; qd < 4; qd++) {
                float4 dx = *reinterpret_cast<const float4 *>(dxp + 8 * qd);
                acc[4 * qd + 0] = __builtin_fmaf((float)S[4 * qd + 0], dx.x * dw, acc[4 * qd + 0]);
                acc[4 * qd + 1] = __builtin_fmaf((float)S[4 * qd + 1], dx.y * dw, acc[4 * qd + 1]);
                acc[4 * qd + 2] = __builtin_fmaf((float)S[4 * qd + 2], dx.z * dw, acc[4 * qd + 2]);
                acc[4 * qd + 3] = __builtin_fmaf((float)S[4 * qd + 3], dx.w * dw, acc[4 * qd + 3]);
            }
        }
        __syncthreads();
    }

    // Output element (row 8*(v/4) + 4*khalf + v%4, column lane%32) of the wave tile.
    const int col = n0 + wn * 32 + (lane & 31);
    if (col < n) {
#pragma unroll
        for (int v = 0; v < 16; v++) {
            int row = m0 + wm * 32 + 8 * (v >> 2) + 4 * khalf + (v & 3);
            if (row < m) y[(int64_t)row * n + col] = acc[v];
        }
    }
}

}  // namespace bqm

extern "C" int bqm_q8_0_gemm(const uint8_t *w, int64_t w_row_bytes, const int8_t *xq, const float *xds, float *y,
                             int m, int k, int n, void *stream) {
    using namespace bqm;
    if (!w || !xq || !xds || !y) return BQM_EINVAL;
    if (m < 1 || k < 256 || n < 1) return BQM_EINVAL;
    if (k % 256 != 0) return BQM_EUNSUPPORTED;
    if (w_row_bytes < (int64_t)(k / kQK) * kQ80Bytes || w_row_bytes % 16 != 0) return BQM_EUNSUPPORTED;
    if (!aligned(w, 16) || !aligned(xq, 16) || !aligned(xds, 8) || !aligned(y, 4)) return BQM_EUNSUPPORTED;
    // per-workgroup offsets are 32-bit: 64 rows of activations / weights
    if ((int64_t)kMmqBM * k > 0x7FFFFFF0ll || (int64_t)kMmqBN * w_row_bytes > 0x7FFFFFF0ll) return BQM_EUNSUPPORTED;
    dim3 grid((n + kMmqBN - 1) / kMmqBN, (m + kMmqBM - 1) / kMmqBM);
    if (grid.y > 65535) return BQM_EUNSUPPORTED;
    hipLaunchKernelGGL(q8_0_gemm_kernel, grid, dim3(kMmqThreads), 0, as_stream(stream), w, w_row_bytes, xq, xds, y, m,
                       k, n);
    return launch_status();
}
