// Traffic twins: measurement kernels for the benchmark, not part of the library's API.
//
// Each twin issues the same global loads and stores as one of the library's kernels, in
// the same launch shape (workgroup size, elements per lane, sub-tiles per wave, XCD
// mapping, cache-policy bits), but replaces the method's arithmetic by a few bitwise
// operations that keep every load live.  Its time is the traffic ceiling of that stream
// mix on this chip: the kernel's time over its twin's says how much of the gap to HBM
// peak is arithmetic and scheduling, and how much is the memory system.  The streaming
// copy (one 16-byte vector per thread in, one out) is the plain ceiling for context.
//
// Built into its own library (libloco_twins.so) with the library's flags; the results
// of a twin are meaningless values.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "loco_device.hpp"

namespace loco {
namespace {

constexpr int kThreads = 256;
constexpr int kTwinMaxPeers = 16;

__device__ __forceinline__ u32x4 fold(u32x4 a, u32x4 b) { return a ^ b; }

// ---- streaming copy ------------------------------------------------------------------

__global__ __launch_bounds__(kThreads) void twin_copy_kernel(const u32x4* src, u32x4* dst, int64_t n16) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < n16) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// ---- compensate-quantize ------------------------------------------------------------
// Per lane and sub-tile: 8 gradient elements (non-temporal) and 8 error elements loaded
// and stored (non-temporal), the 8 codes (non-temporal) and, in lane b < the tile's block
// count, block b's absmax.  The lane layout is the kernel's: two pieces of 4 elements at
// 4l and 256 + 4l when the gradient or the error is fp32 (each instruction then covers a
// contiguous run), else 8 consecutive elements at 8l.  U sub-tiles of 512 elements per
// wave; the kernel's workgroup size per error kind, workgroups renumbered in XCD runs.

template <int N>
struct Raw {
    uint32_t w[N];
};

template <int BYTES, bool NT>
__device__ __forceinline__ Raw<(BYTES + 3) / 4> ldraw(const void* p) {
    Raw<(BYTES + 3) / 4> r;
    if constexpr (BYTES == 16) {
        const u32x4 v = NT ? __builtin_nontemporal_load((const u32x4*)p) : *(const u32x4*)p;
        r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
    } else if constexpr (BYTES == 8) {
        const u32x2 v = NT ? __builtin_nontemporal_load((const u32x2*)p) : *(const u32x2*)p;
        r.w[0] = v.x; r.w[1] = v.y;
    } else {
        r.w[0] = NT ? __builtin_nontemporal_load((const uint32_t*)p) : *(const uint32_t*)p;
    }
    return r;
}

template <int BYTES>
__device__ __forceinline__ void stnt(void* p, const uint32_t* w) {
    if constexpr (BYTES == 16) __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]}, (u32x4*)p);
    else if constexpr (BYTES == 8) __builtin_nontemporal_store(u32x2{w[0], w[1]}, (u32x2*)p);
    else if constexpr (BYTES == 4) __builtin_nontemporal_store(w[0], (uint32_t*)p);
    else if constexpr (BYTES == 2) __builtin_nontemporal_store((uint16_t)w[0], (uint16_t*)p);
    else __builtin_nontemporal_store((uint8_t)w[0], (uint8_t*)p);
}

template <int GB, int EB, int BITS, int U, int RUN, int TPB>
__global__ __launch_bounds__(TPB) void twin_cq_kernel(const void* g, void* e, uint8_t* codes, float* absmax,
                                                      int64_t ntiles, int nb) {
    constexpr bool SPLIT = GB == 4 || EB == 4;
    constexpr int N = SPLIT ? 4 : 8;  // elements per access
    constexpr int PIECES = 8 / N;
    const int lane = lane_id();
    const int64_t wg = xcd_remap<8, RUN>(blockIdx.x, gridDim.x);
    const int64_t t = wg * (TPB / 64) + uniform(threadIdx.x / 64);
    if (t >= ntiles) return;
    Raw<(N * GB + 3) / 4> gw[U][PIECES];
    Raw<(N * EB + 3) / 4> ew[U][PIECES];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int pc = 0; pc < PIECES; ++pc) {
            const int64_t i0 = (t * U + u) * 512 + (SPLIT ? pc * 256 + lane * 4 : lane * 8);
            gw[u][pc] = ldraw<N * GB, true>((const char*)g + i0 * GB);
            ew[u][pc] = ldraw<N * EB, true>((const char*)e + i0 * EB);
        }
    uint32_t x = 0;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int pc = 0; pc < PIECES; ++pc) {
            const int64_t i0 = (t * U + u) * 512 + (SPLIT ? pc * 256 + lane * 4 : lane * 8);
            uint32_t w[(N * EB + 3) / 4];
#pragma unroll
            for (int i = 0; i < (N * EB + 3) / 4; ++i) w[i] = ew[u][pc].w[i] ^ gw[u][pc].w[0];
            stnt<N * EB>((char*)e + i0 * EB, w);
            x ^= w[0];
            uint32_t c[2] = {w[0], w[(N * EB + 3) / 4 - 1]};
            stnt<N * BITS / 8>(codes + (i0 * BITS) / 8, c);
        }
    if (lane < nb) absmax[t * nb + lane] = __uint_as_float(x & 0x3F7FFFFFu);
}

// ---- dequant-reduce (bf16 / fp32 shard, or the fused Adam step) ----------------------
// Per lane and sub-tile, in the kernel's lane layout (8 consecutive outputs for a bf16
// shard; two pieces of 4 at 4l and 256 + 4l for an fp32 shard and the Adam step): every
// peer's codes of the lane's elements (non-temporal) and its block absmax, then the 8
// outputs (non-temporal); or, for the Adam step, theta, m and v loaded and stored and the
// bf16 weight copy stored (all non-temporal).

struct TwinPeers {
    const uint8_t* codes[kTwinMaxPeers];
    const float* absmax[kTwinMaxPeers];
};

// The kernel's workgroup shape per mode: 4-wave workgroups in XCD runs of 16 for a shard,
// one-wave workgroups in runs of 64 for the Adam step.
constexpr int twin_dr_tpb(int mode) { return mode == 2 ? 64 : 256; }
constexpr int twin_dr_run(int mode) { return mode == 2 ? 64 : 16; }

template <int BITS, int MODE, int U, int P>
__global__ __launch_bounds__(twin_dr_tpb(MODE)) void twin_dr_kernel(TwinPeers pp, int64_t ntiles, int lb, void* out,
                                                                    float* theta, float* m, float* v, uint16_t* tb) {
    constexpr bool SPLIT = MODE != 1;
    const int lane = lane_id();
    const int64_t wg = xcd_remap<8, twin_dr_run(MODE)>(blockIdx.x, gridDim.x);
    const int64_t t = wg * (twin_dr_tpb(MODE) / 64) + uniform(threadIdx.x / 64);
    if (t >= ntiles) return;
    auto at = [&](int u, int pc) { return (t * U + u) * 512 + (SPLIT ? pc * 256 + lane * 4 : lane * 8 + pc * 4); };
    f32x4 th[U][2], mo[U][2], ve[U][2];
    if constexpr (MODE == 2) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int pc = 0; pc < 2; ++pc) {
                th[u][pc] = __builtin_nontemporal_load((const f32x4*)(theta + at(u, pc)));
                mo[u][pc] = __builtin_nontemporal_load((const f32x4*)(m + at(u, pc)));
                ve[u][pc] = __builtin_nontemporal_load((const f32x4*)(v + at(u, pc)));
            }
    }
    uint32_t acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u] = 0u;
#pragma unroll
    for (int p = 0; p < P; ++p) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            uint32_t w;
            if constexpr (SPLIT) {
                w = __builtin_nontemporal_load((const uint16_t*)(pp.codes[p] + at(u, 0) * BITS / 8)) ^
                    __builtin_nontemporal_load((const uint16_t*)(pp.codes[p] + at(u, 1) * BITS / 8));
            } else {
                w = __builtin_nontemporal_load((const uint32_t*)(pp.codes[p] + at(u, 0) * BITS / 8));
            }
            acc[u] ^= w ^ __float_as_uint(pp.absmax[p][at(u, 0) >> lb]);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t a = acc[u] & 0x3F7FFFFFu;
        if constexpr (MODE == 1) {
            __builtin_nontemporal_store(u32x4{a, a, a, a}, (u32x4*)((uint16_t*)out + at(u, 0)));
        } else if constexpr (MODE == 0) {
            const f32x4 x = __builtin_bit_cast(f32x4, u32x4{a, a, a, a});
            __builtin_nontemporal_store(x, (f32x4*)((float*)out + at(u, 0)));
            __builtin_nontemporal_store(x, (f32x4*)((float*)out + at(u, 1)));
        } else {
            const float s = __uint_as_float(a);
            const f32x4 d = {s, s, s, s};
#pragma unroll
            for (int pc = 0; pc < 2; ++pc) {
                __builtin_nontemporal_store(th[u][pc] + d, (f32x4*)(theta + at(u, pc)));
                __builtin_nontemporal_store(mo[u][pc] + d, (f32x4*)(m + at(u, pc)));
                __builtin_nontemporal_store(ve[u][pc] + d, (f32x4*)(v + at(u, pc)));
                if (tb) __builtin_nontemporal_store(u32x2{a, a}, (u32x2*)(tb + at(u, pc)));
            }
        }
    }
}

// ---- Top-k ---------------------------------------------------------------------------
// One 256-thread workgroup per 4096-element chunk: thread t loads rows q*1024 + 4t of the
// gradient and the error as 16-byte vectors and stores the error rows back (all
// non-temporal); the first k threads store an index, the first ceil(k*bits/8) a code byte,
// thread 0 the chunk's absmax.

__global__ __launch_bounds__(kThreads) void twin_tk_kernel(const float* g, float* e, uint16_t* idx, uint8_t* codes,
                                                           float* absmax, int64_t nchunks, int k, int nbytes) {
    const int64_t c = blockIdx.x;
    if (c >= nchunks) return;
    const int tid = threadIdx.x;
    const float* gb = g + c * 4096;
    float* eb = e + c * 4096;
    u32x4 gv[4], ev[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        gv[q] = __builtin_nontemporal_load((const u32x4*)(gb + q * 1024 + tid * 4));
        ev[q] = __builtin_nontemporal_load((const u32x4*)(eb + q * 1024 + tid * 4));
    }
    uint32_t x = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const u32x4 y = fold(gv[q], ev[q]);
        __builtin_nontemporal_store(y, (u32x4*)(eb + q * 1024 + tid * 4));
        x ^= y.x;
    }
    if (tid < k) idx[c * k + tid] = (uint16_t)(x & 0xFFFu);
    if (tid < nbytes) codes[c * nbytes + tid] = (uint8_t)x;
    if (tid == 0) absmax[c] = __uint_as_float(x & 0x3F7FFFFFu);
}

// ---- sparse aggregation -----------------------------------------------------------------
// The fp32-output kernel's shape: a pre-read of every peer's payload arrays, then one
// 128-thread workgroup per 4096-element chunk: every peer's k indices, code bytes and
// absmax of the chunk are loaded, then the chunk's 16 KB of fp32 output is stored as
// 16-byte vectors (non-temporal).

struct TwinSparsePeers {
    const uint16_t* idx[kTwinMaxPeers];
    const uint8_t* codes[kTwinMaxPeers];
    const float* absmax[kTwinMaxPeers];
};

template <int P>
__global__ __launch_bounds__(128) void twin_sa_kernel(TwinSparsePeers pp, int64_t nchunks, int k, int nbytes,
                                                      float* out) {
    const int64_t c = blockIdx.x;
    if (c >= nchunks) return;
    const int tid = threadIdx.x;
    uint32_t x = 0;
#pragma unroll
    for (int p = 0; p < P; ++p) {
        if (tid < k) x ^= pp.idx[p][c * k + tid];
        if (tid < nbytes) x ^= pp.codes[p][c * nbytes + tid];
        if (tid == 0) x ^= __float_as_uint(pp.absmax[p][c]);
    }
    const float s = __uint_as_float(x & 0x3F7FFFFFu);
    float* o = out + c * 4096;
#pragma unroll
    for (int r = 0; r < 8; ++r) __builtin_nontemporal_store(f32x4{s, s, s, s}, (f32x4*)(o + (r * 128 + tid) * 4));
}

// The general aggregation kernel's pre-read: every 16-byte vector of the peers' payload
// arrays loaded once (cached loads, so that the aggregation finds them in the caches),
// folded into one word that reaches memory only if it has one particular value (then at
// out[0], which the aggregation overwrites).
__global__ __launch_bounds__(kThreads) void twin_sa_pre_kernel(TwinSparsePeers pp, int npeers, int64_t iv,
                                                               int64_t cv, int64_t av, float* out) {
    const int64_t first = (int64_t)blockIdx.x * kThreads + threadIdx.x, stride = (int64_t)gridDim.x * kThreads;
    uint32_t x = 0;
    for (int p = 0; p < npeers; ++p) {
        for (int64_t i = first; i < iv; i += stride) x ^= ((const u32x4*)pp.idx[p])[i].x;
        for (int64_t i = first; i < cv; i += stride) x ^= ((const u32x4*)pp.codes[p])[i].y;
        for (int64_t i = first; i < av; i += stride) x ^= ((const u32x4*)pp.absmax[p])[i].z;
    }
    if (x == 0x9E3779B9u) out[0] = __uint_as_float(x);
}

int64_t grid_of(int64_t ntiles, int per_wg) { return (ntiles + per_wg - 1) / per_wg; }

}  // namespace
}  // namespace loco

using namespace loco;

// Every entry point returns 0, or -1 for an unsupported shape, or a HIP error code.
extern "C" {

__attribute__((visibility("default"))) int loco_twin_copy(const void* src, void* dst, int64_t bytes, void* stream) {
    const int64_t n16 = bytes / 16;
    if (n16 <= 0) return -1;
    void* args[] = {(void*)&src, (void*)&dst, (void*)&n16};
    return hipLaunchKernel((const void*)&twin_copy_kernel, dim3((unsigned)grid_of(n16, kThreads)), dim3(kThreads),
                           args, 0, (hipStream_t)stream);
}

// g: gradient (gbytes 2 or 4 per element); e: error of kind ekind (0 fp32, 1 bf16, 2 int8);
// n elements (whole tiles only; a ragged tail is left out); bits 2/4/8.
__attribute__((visibility("default"))) int loco_twin_cq(const void* g, void* e, uint8_t* codes, float* absmax,
                                                        int64_t n, int gbytes, int ekind, int bits, int block,
                                                        void* stream) {
    const int U = ekind == 2 ? 2 : 1;
    const int64_t ntiles = n / (512 * U);
    if (ntiles <= 0 || block < 64 || block > 512 || (block & (block - 1)) != 0) return -1;
    const int nb = 512 * U / block;
    const void* k = nullptr;
    int tpb = 0;
    // the kernel's workgroup size and XCD run per error kind
#define LOCO_TWIN_CQ(GB, EK, EB, BI, UU, RUN, TPB)                                       \
    if (gbytes == GB && ekind == EK && bits == BI) {                                      \
        k = (const void*)&twin_cq_kernel<GB, EB, BI, UU, RUN, TPB>;                       \
        tpb = TPB;                                                                        \
    }
    LOCO_TWIN_CQ(2, 0, 4, 4, 1, 128, 64)
    LOCO_TWIN_CQ(2, 0, 4, 8, 1, 128, 64)
    LOCO_TWIN_CQ(2, 1, 2, 4, 1, 32, 256)
    LOCO_TWIN_CQ(2, 2, 1, 4, 2, 64, 128)
    LOCO_TWIN_CQ(4, 0, 4, 4, 1, 128, 64)
#undef LOCO_TWIN_CQ
    if (!k) return -1;
    void* args[] = {(void*)&g, (void*)&e, (void*)&codes, (void*)&absmax, (void*)&ntiles, (void*)&nb};
    return hipLaunchKernel(k, dim3((unsigned)grid_of(ntiles, tpb / 64)), dim3(tpb), args, 0, (hipStream_t)stream);
}

// 8 peers of 4-bit codes; mode 0: fp32 out, 1: bf16 out, 2: Adam step on theta, m, v (+ the
// bf16 copy tb, may be null).
__attribute__((visibility("default"))) int loco_twin_dr(const uint8_t* const* codes, const float* const* absmax,
                                                        int npeers, int64_t n, int bits, int block, int mode,
                                                        void* out, float* theta, float* m, float* v, uint16_t* tb,
                                                        void* stream) {
    if (npeers != 8 || bits != 4 || (block & (block - 1)) != 0 || block < 64) return -1;
    TwinPeers pp{};
    for (int i = 0; i < npeers; ++i) {
        pp.codes[i] = codes[i];
        pp.absmax[i] = absmax[i];
    }
    const int U = mode == 2 ? 1 : 2;
    const int64_t ntiles = n / (512 * U);
    if (ntiles <= 0) return -1;
    const int lb = __builtin_ctz((unsigned)block);
    const void* k = mode == 0 ? (const void*)&twin_dr_kernel<4, 0, 2, 8>
                  : mode == 1 ? (const void*)&twin_dr_kernel<4, 1, 2, 8>
                              : (const void*)&twin_dr_kernel<4, 2, 1, 8>;
    void* args[] = {(void*)&pp, (void*)&ntiles, (void*)&lb, (void*)&out, (void*)&theta, (void*)&m, (void*)&v,
                    (void*)&tb};
    const int tpb = mode == 2 ? twin_dr_tpb(2) : twin_dr_tpb(0);
    return hipLaunchKernel(k, dim3((unsigned)grid_of(ntiles, tpb / 64)), dim3(tpb), args, 0, (hipStream_t)stream);
}

__attribute__((visibility("default"))) int loco_twin_tk(const float* g, float* e, uint16_t* idx, uint8_t* codes,
                                                        float* absmax, int64_t n, int k, int bits, void* stream) {
    const int64_t nchunks = n / 4096;
    if (nchunks <= 0 || k < 1 || k > kThreads) return -1;
    const int nbytes = (k * bits + 7) / 8;
    void* args[] = {(void*)&g, (void*)&e, (void*)&idx, (void*)&codes, (void*)&absmax, (void*)&nchunks, (void*)&k,
                    (void*)&nbytes};
    return hipLaunchKernel((const void*)&twin_tk_kernel, dim3((unsigned)nchunks), dim3(kThreads), args, 0,
                           (hipStream_t)stream);
}

__attribute__((visibility("default"))) int loco_twin_sa(const uint16_t* const* idx, const uint8_t* const* codes,
                                                        const float* const* absmax, int npeers, int64_t n, int k,
                                                        int bits, float* out, void* stream) {
    const int64_t nchunks = n / 4096;
    if (npeers != 8 || nchunks <= 0 || k < 1 || k > 128) return -1;
    TwinSparsePeers pp{};
    for (int i = 0; i < npeers; ++i) {
        pp.idx[i] = idx[i];
        pp.codes[i] = codes[i];
        pp.absmax[i] = absmax[i];
    }
    const int nbytes = (k * bits + 7) / 8;
    const int64_t iv = nchunks * k * 2 / 16, cv = nchunks * nbytes / 16, av = nchunks * 4 / 16;
    void* pre[] = {(void*)&pp, (void*)&npeers, (void*)&iv, (void*)&cv, (void*)&av, (void*)&out};
    const int64_t pb = grid_of(iv + cv + av, kThreads) < 2048 ? grid_of(iv + cv + av, kThreads) : 2048;
    const hipError_t err = hipLaunchKernel((const void*)&twin_sa_pre_kernel, dim3((unsigned)(pb < 1 ? 1 : pb)),
                                           dim3(kThreads), pre, 0, (hipStream_t)stream);
    if (err != hipSuccess) return err;
    void* args[] = {(void*)&pp, (void*)&nchunks, (void*)&k, (void*)&nbytes, (void*)&out};
    return hipLaunchKernel((const void*)&twin_sa_kernel<8>, dim3((unsigned)nchunks), dim3(128), args, 0,
                           (hipStream_t)stream);
}

}  // extern "C"
