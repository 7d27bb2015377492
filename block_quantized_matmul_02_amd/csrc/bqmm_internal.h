// Internal helpers shared by the gfx950 kernels of libbqmm.  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "bqmm.h"

namespace bqm {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v32f __attribute__((ext_vector_type(32)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kQK = 32;          // values per quantization block
constexpr int kQ80Bytes = 34;    // Q8_0 block: fp16 scale + 32 int8

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Map the launch status to the library's return code.  The status is read
// with hipPeekAtLastError, which leaves it in place: an error the caller left
// pending before the call is reported (it is indistinguishable from a failed
// launch) but not consumed.
inline int launch_status() {
    hipError_t e = hipPeekAtLastError();
    return e == hipSuccess ? BQM_OK : BQM_EHIP_BASE + (int)e;
}

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

// Host-side facts that the launches need are queried once per device and
// kept in per-device slots (a device ordinal beyond the table shares the last
// slot and is re-queried whenever its value differs).
constexpr int kMaxDevices = 64;

inline int current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    return dev < kMaxDevices ? dev : kMaxDevices - 1;
}

// Compute units of the current device (256 on MI355X, also the fallback).
inline int device_cus() {
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    const int slot = dev < kMaxDevices ? dev : kMaxDevices - 1;
    int cus = dev < kMaxDevices ? cache[slot].load(std::memory_order_relaxed) : 0;
    if (cus > 0) return cus;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    if (dev < kMaxDevices) cache[slot].store(cus, std::memory_order_relaxed);
    return cus;
}

// Per-kernel launch facts: whether the dynamic LDS limit has been raised on a
// device, and the last occupancy answer (for one LDS size) on each device.
// One static instance per kernel instantiation.
struct LaunchCache {
    std::atomic<int> lds_raised[kMaxDevices];
    std::atomic<uint64_t> occupancy[kMaxDevices];   // (lds bytes << 8) | blocks per CU, 0 = none
};

// Allow `bytes` of dynamic LDS for kernel `fn` on the current device (once).
inline int raise_lds_limit(LaunchCache &c, const void *fn, int bytes) {
    const int dev = current_device();
    if (c.lds_raised[dev].load(std::memory_order_relaxed)) return BQM_OK;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return BQM_EHIP_BASE + (int)e;
    c.lds_raised[dev].store(1, std::memory_order_relaxed);
    return BQM_OK;
}

// Resident workgroups per CU of `fn` with `threads` threads and `lds` bytes of
// dynamic LDS, at least 1 and at most `cap`; asked of the runtime only when the
// LDS size differs from the last one asked on this device.
inline int blocks_per_cu(LaunchCache &c, const void *fn, int threads, int lds, int cap) {
    const int dev = current_device();
    const uint64_t hit = c.occupancy[dev].load(std::memory_order_relaxed);
    if (hit != 0 && (hit >> 8) == (uint64_t)(uint32_t)lds) return (int)(hit & 0xFF);
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, lds) != hipSuccess || per_cu < 1) per_cu = 1;
    if (per_cu > cap) per_cu = cap;
    c.occupancy[dev].store(((uint64_t)(uint32_t)lds << 8) | (uint64_t)per_cu, std::memory_order_relaxed);
    return per_cu;
}

// The matrix-core GEMV for 3..15 tokens (q8_0_gemv_mma.hip): whether it takes
// a shape, and its launch (arguments already checked by the GEMV entry).
bool gemv_mma_applies(int m, int k, int n);
int gemv_mma(const uint8_t *w, int64_t w_row_bytes, const int8_t *xq, const float *xds, float *y, int m, int k, int n,
             hipStream_t s);

// ---------------------------------------------------------------- device side

// IEEE binary16 bits -> f32 (exact; hardware conversion handles subnormals).
__device__ __forceinline__ float half_bits_to_float(unsigned h) {
    _Float16 v = __builtin_bit_cast(_Float16, (unsigned short)(h & 0xFFFFu));
    return (float)v;
}

// Butterfly sums inside a row of 16 lanes using DPP; every lane of the row ends
// with the same value.  Steps: pair lanes (xor 1), quads (xor 2), the two
// halves of each 8-lane group (half mirror), the two halves of the row (mirror).
__device__ __forceinline__ float dpp_sum16(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
    return v;
}

// The swap builtins return a 2-vector {new vdst, new src0}.  Each element is
// copied to a scalar before any bit cast: clang lowers a __builtin_bit_cast of
// a vector-element expression to a load from the vector's first element.
// Sum of lanes l and l^16 (rows 0/1 and 2/3 exchanged by v_permlane16_swap).
__device__ __forceinline__ float swap16_sum(float v) {
    unsigned u = __builtin_bit_cast(unsigned, v);
    auto s = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    unsigned a = s[0], b = s[1];
    return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// Sum of lanes l and l^32 (the wave's halves exchanged by v_permlane32_swap).
__device__ __forceinline__ float swap32_sum(float v) {
    unsigned u = __builtin_bit_cast(unsigned, v);
    auto s = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    unsigned a = s[0], b = s[1];
    return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// Max of lanes l, l^16 and of lanes l, l^32.
__device__ __forceinline__ float swap16_max(float v) {
    unsigned u = __builtin_bit_cast(unsigned, v);
    auto s = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    unsigned a = s[0], b = s[1];
    return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}

__device__ __forceinline__ float swap32_max(float v) {
    unsigned u = __builtin_bit_cast(unsigned, v);
    auto s = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    unsigned a = s[0], b = s[1];
    return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}

// The q8_1 rule for one 32-value block held by 8 consecutive lanes, four
// values per lane: d = amax/127 (f32 division), q = clamp(round_half_away(
// x/d), -127, 127) with a correctly rounded division, all zeros when d is 0.
// Returns the lane's four quants packed little-endian into a dword and sets
// d.  Every lane of the 8-lane group must execute it together (DPP).
__device__ __forceinline__ float q8_1_max8(float v) {
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)));
    return v;
}

__device__ __forceinline__ int q8_1_quant1(float x, float d, bool nz) {
    if (!nz) return 0;
    float r = __builtin_roundf(x / d);   // correctly rounded f32 division, ties away from zero
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

struct Q81Lane {
    unsigned packed;   // quants 0..3 of this lane, byte i = quant i
    int qsum;          // sum of this lane's four quants
    float d;           // the block scale
};

__device__ __forceinline__ Q81Lane q8_1_block_lane(float4 v) {
    const float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    const float amax = q8_1_max8(a);
    const float d = amax / 127.0f;
    const bool nz = d > 0.0f;   // amax == 0, or amax/127 underflowing to 0: an all-zero block
    const int q0 = q8_1_quant1(v.x, d, nz), q1 = q8_1_quant1(v.y, d, nz);
    const int q2 = q8_1_quant1(v.z, d, nz), q3 = q8_1_quant1(v.w, d, nz);
    Q81Lane r;
    r.packed = (unsigned)(q0 & 0xFF) | ((unsigned)(q1 & 0xFF) << 8) | ((unsigned)(q2 & 0xFF) << 16) | ((unsigned)q3 << 24);
    r.qsum = q0 + q1 + q2 + q3;
    r.d = d;
    return r;
}

}  // namespace bqm
