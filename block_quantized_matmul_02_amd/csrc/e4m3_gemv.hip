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
//  * Activations: for one token and k <= 4096 a lane's chunks are the same on
//    every row, so their 16*J values sit in registers, loaded before the
//    first weight tiles.  Otherwise a token group (up to 4 tokens) is staged
//    in LDS with each chunk's four 16-byte pieces rotated by (c + c/4) % 4, so
//    the 16 lanes of a read phase, on 16 consecutive chunks, hit distinct
//    banks.  More than 4 tokens run as several token groups; the groups of
//    the same rows run together on one XCD, so their re-reads of a weight
//    tile are served by that XCD's L2.  Past 4 tokens the kernel is bound by
//    its f32 FMAs (one per weight byte and token), not by memory.
//  * Arithmetic: per chunk and token, 16 fma in k order into one f32 partial
//    per lane; the L partials of a row are summed by a fixed DPP /
//    permlane-swap butterfly; y = w_scale * sum.  A token's operation order
//    does not depend on m or its group, so decode and verify agree bitwise.
#include "bqmm_internal.h"

namespace bqm {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kE8Threads = 256;
constexpr int kE8Waves = kE8Threads / 64;
constexpr int kE8MaxTG = 4;          // tokens per group
constexpr int kE8MaxK = 8192;

struct E8Geom {
    int CPR;       // 16-byte chunks per row
    int L;         // lanes per row
    int Llog2;
    int G;         // rows per item
    int J;         // chunks per lane per row
    int n_items;   // ceil(n / G)
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

// TG: token-group capacity; JM: chunk slots per lane (>= J); XREG: one token,
// activations in registers.
template <int TG, int JM, bool XREG>
__global__ __launch_bounds__(kE8Threads) void e4m3_gemv_kernel(const uint8_t *__restrict__ w,
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
    const int t0 = tg * TG;
    const int tcount = min(TG, m - t0);
    const int nwaves = (gridDim.x / g.ngroups) * kE8Waves;
    const int wid = rwg * kE8Waves + wave;
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

    auto compute = [&](const u32x4 (&buf)[JM], int q) {
        float acc[TG];
#pragma unroll
        for (int t = 0; t < TG; t++) acc[t] = 0.0f;
        // No branch on the slot's validity: an invalid slot's weights are the
        // zeros of an out-of-range load (its activations zeros too, or chunk 0
        // from LDS), so it adds exact zeros; a branch here would let the
        // compiler sink the activation loads behind the tiles.
#pragma unroll
        for (int j = 0; j < JM; j++) {
            float f[16];
            e8_decode16(buf[j], f);
            const int c = valid[j] ? li + g.L * j : 0;
#pragma unroll
            for (int t = 0; t < TG; t++) {
                if (!XREG && t >= tcount) break;
                float xv[16];
                if (XREG) {
#pragma unroll
                    for (int e = 0; e < 16; e++) xv[e] = xr[XREG ? j : 0][e];
                } else {
                    const float *xt = xs + t * k;
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        const float4 v = *reinterpret_cast<const float4 *>(xt + e8_piece(c, i));
                        xv[4 * i + 0] = v.x;
                        xv[4 * i + 1] = v.y;
                        xv[4 * i + 2] = v.z;
                        xv[4 * i + 3] = v.w;
                    }
                }
#pragma unroll
                for (int e = 0; e < 16; e++) acc[t] = __builtin_fmaf(xv[e], f[e], acc[t]);
            }
        }
        const int row = (wid + nwaves * q) * g.G + gr;
#pragma unroll
        for (int t = 0; t < TG; t++) {
            if (!XREG && t >= tcount) break;
            float v = acc[t];
            v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
            v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
            v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
            v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
            if (g.L >= 32) v = swap16_sum(v);
            if (g.L >= 64) v = swap32_sum(v);
            if (li == 0 && row < n) y[(int64_t)(t0 + t) * n + row] = w_scale * v;
        }
    };

    u32x4 bA[JM], bB[JM], bC[JM];
    issue(bA, 0);
    issue(bB, 1);
    issue(bC, 2);
    if (!XREG) {
        // stage the group's tokens (after the first tiles are in flight)
        const int quads = tcount * k / 4;
        for (int p = threadIdx.x; p < quads; p += kE8Threads) {
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

static bool e8_geom(int m, int k, int n, E8Geom &g) {
    g.CPR = k / 16;
    int L = 16;
    while (L < g.CPR && L < 64) L *= 2;
    g.L = L;
    g.Llog2 = __builtin_ctz(L);
    g.G = 64 / L;
    g.J = (g.CPR + L - 1) / L;
    g.n_items = (n + g.G - 1) / g.G;
    g.ngroups = (m + kE8MaxTG - 1) / kE8MaxTG;
    return g.J <= 8;
}

template <int TG, int JM, bool XREG>
static int e8_launch(const uint8_t *w, const float *x, float w_scale, float *y, int m, int k, int n,
                     const E8Geom &g, hipStream_t stream) {
    const int lds = XREG ? 0 : TG * k * 4;
    static int attr_done = 0;
    if (!attr_done) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&e4m3_gemv_kernel<TG, JM, XREG>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return BQM_EHIP_BASE + (int)e;
        attr_done = 1;
    }
    const int cus = device_cus();
    // resident workgroups per CU (registers and LDS), at most 4
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(&e4m3_gemv_kernel<TG, JM, XREG>),
                                                     kE8Threads, lds) != hipSuccess || per_cu < 1)
        per_cu = 1;
    if (per_cu > 4) per_cu = 4;
    // Workgroups per token group: no more than fit at once, and few enough
    // that each wave has at least four items (each wave also reads the
    // activations once, which small n would otherwise multiply).
    int rwgs = (g.n_items + 4 * kE8Waves - 1) / (4 * kE8Waves);
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
    hipLaunchKernelGGL((e4m3_gemv_kernel<TG, JM, XREG>), dim3(rwgs * g.ngroups), dim3(kE8Threads), lds, stream, w, x,
                       w_scale, y, m, k, n, gg);
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
    E8Geom g;
    if (!e8_geom(m, k, n, g)) return BQM_EUNSUPPORTED;
    hipStream_t s = as_stream(stream);
    if (m == 1 && g.J <= 4) return e8_launch<1, 4, true>(w, x, w_scale, y, m, k, n, g, s);
    if (g.J <= 4) {
        if (m <= 2) return e8_launch<2, 4, false>(w, x, w_scale, y, m, k, n, g, s);
        return e8_launch<4, 4, false>(w, x, w_scale, y, m, k, n, g, s);
    }
    if (m == 1) return e8_launch<1, 8, false>(w, x, w_scale, y, m, k, n, g, s);
    if (m <= 2) return e8_launch<2, 8, false>(w, x, w_scale, y, m, k, n, g, s);
    return e8_launch<4, 8, false>(w, x, w_scale, y, m, k, n, g, s);
}
