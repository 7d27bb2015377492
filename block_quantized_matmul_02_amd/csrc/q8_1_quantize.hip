// q8_1 activation quantization for gfx950.
//
// Rule per (token, 32-value block), from the memra-engine pages: d = amax/127
// (f32 division), q = clamp(round_half_away(x/d), -127, 127), and the pair's
// second value s = d * sum(q); a block whose d is 0 (amax == 0, or amax/127
// underflowing) quantizes to zeros ("decode_kernel_census.rs", fn q8: int8 per
// column plus a per-32 scale pair; "f16_ffi.rs", fn try_f16_gemm, W8A8 arm:
// the int8 rule with Rust's round).
//
// Mapping: 8 lanes per block, one float4 per lane, so a wave covers 8 blocks
// (1 KiB of x) with fully coalesced 16-byte loads; the block amax and quant
// sum are reduced across the 8 lanes with DPP.  The kernel is HBM-bound
// (4 B read + 1.25 B written per value); the correctly rounded division costs
// ~10 VALU ops per value, far under the VALU budget at HBM speed.
#include "bqmm_internal.h"

namespace bqm {

__device__ __forceinline__ int isum8(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);
    return v;
}

// One thread per 4 values; blocks of 32 values = 8 consecutive lanes.
__global__ __launch_bounds__(256) void q8_1_quantize_kernel(const float4 *__restrict__ x,
                                                          int *__restrict__ xq,
                                                          float2 *__restrict__ xds,
                                                          int64_t nvec) {
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    // Lanes past the end still take part in the DPP reductions (with zeros) so
    // every 8-lane group reduces with its full membership; nvec % 8 == 0, so a
    // group is either entirely valid or entirely past the end.
    bool valid = i < nvec;
    float4 v = valid ? x[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    const Q81Lane r = q8_1_block_lane(v);
    int sum = isum8(r.qsum);
    if (valid) {
        xq[i] = (int)r.packed;
        if ((threadIdx.x & 7) == 0) xds[i >> 3] = make_float2(r.d, r.d * (float)sum);
    }
}

}  // namespace bqm

extern "C" int bqm_q8_1_quantize(const float *x, int8_t *xq, float *xds, int m, int k, void *stream) {
    using namespace bqm;
    if (!x || !xq || !xds) return BQM_EINVAL;
    if (m < 1 || k < kQK) return BQM_EINVAL;
    if (k % kQK != 0) return BQM_EUNSUPPORTED;
    if (!aligned(x, 16) || !aligned(xq, 4) || !aligned(xds, 8)) return BQM_EUNSUPPORTED;
    int64_t nvec = (int64_t)m * k / 4;
    int64_t grid = (nvec + 255) / 256;
    if (grid > 0x7FFFFFFF) return BQM_EUNSUPPORTED;
    hipLaunchKernelGGL(q8_1_quantize_kernel, dim3((unsigned)grid), dim3(256), 0, as_stream(stream),
                       reinterpret_cast<const float4 *>(x), reinterpret_cast<int *>(xq),
                       reinterpret_cast<float2 *>(xds), nvec);
    return launch_status();
}
