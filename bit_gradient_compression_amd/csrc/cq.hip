// Fused compensate -> block absmax -> quantize -> pack -> error update, one HBM pass.
//
// LoCo ("LoCo: Low-Bit Communication Adaptor for Large-scale Model Training"),
// Sec. 3.1 Eqns. (1)-(3) and Sec. 3.2 Eqns. (4)-(5), with a per-block absmax scale:
//   h = g + e;  absmax = max|h| per block;  step = absmax/qmax;  inv = 1/step
//   q = clamp(rint(h*inv));  r = h - q*step;  e' = beta*e + (1-beta)*r
//
// Mapping: a wavefront owns a tile of kCqUnroll sub-tiles of 512 elements; lane l owns
// 8 consecutive elements of each sub-tile, so one bf16 gradient load, two fp32 error
// loads and one 32-bit code store per lane are 16-byte (or 4-byte) coalesced accesses.
// A scale block of B elements is B/8 consecutive lanes; its absmax is reduced with DPP
// row operations (and a permlane swap past 16 lanes).  Every load of a tile is issued
// before any arithmetic.  The grid covers all wave tiles of all segments of the call:
// each wave takes one tile and exits, so the waves in flight sweep the buffers in
// address order (measured on MI355X, a persistent grid-stride loop over the same
// traffic mix runs ~15% slower).

#include "loco_device.hpp"
#include "loco_internal.hpp"

namespace loco {
namespace {

template <bool BF>
__device__ __forceinline__ float load1(const void* p, int64_t i) {
    if constexpr (BF) return __uint_as_float((uint32_t)((const uint16_t*)p)[i] << 16);
    else return ((const float*)p)[i];
}

template <bool BF>
__device__ __forceinline__ void store1(void* p, int64_t i, float v) {
    if constexpr (BF) ((uint16_t*)p)[i] = bf16_rne(v);
    else ((float*)p)[i] = v;
}

// 8 consecutive elements starting at i0 (16-byte aligned).  The gradient is read once:
// non-temporal.
template <bool BF>
__device__ __forceinline__ void load8_nt(const void* p, int64_t i0, float (&x)[8]) {
    if constexpr (BF) {
        u32x4 w = __builtin_nontemporal_load((const u32x4*)((const uint16_t*)p + i0));
        x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
        x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
    } else {
        const f32x4* q = (const f32x4*)((const float*)p + i0);
        f32x4 a = __builtin_nontemporal_load(q);
        f32x4 b = __builtin_nontemporal_load(q + 1);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
}

template <bool BF>
__device__ __forceinline__ void load8(const void* p, int64_t i0, float (&x)[8]) {
    if constexpr (BF) {
        u32x4 w = *(const u32x4*)((const uint16_t*)p + i0);
        x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
        x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
    } else {
        const f32x4* q = (const f32x4*)((const float*)p + i0);
        f32x4 a = q[0];
        f32x4 b = q[1];
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
}

template <bool BF>
__device__ __forceinline__ void store8(void* p, int64_t i0, const float (&x)[8]) {
    if constexpr (BF) {
        u32x4 w;
        w.x = bf16x2_rne(x[0], x[1]); w.y = bf16x2_rne(x[2], x[3]);
        w.z = bf16x2_rne(x[4], x[5]); w.w = bf16x2_rne(x[6], x[7]);
        __builtin_nontemporal_store(w, (u32x4*)((uint16_t*)p + i0));
    } else {
        f32x4* q = (f32x4*)((float*)p + i0);
        f32x4 a = {x[0], x[1], x[2], x[3]};
        f32x4 b = {x[4], x[5], x[6], x[7]};
        __builtin_nontemporal_store(a, q);
        __builtin_nontemporal_store(b, q + 1);
    }
}

template <bool GBF, bool EBF, int BITS, int B, bool FIXED, bool FULL>
__device__ __forceinline__ void cq_tile(const CqSegDev& sg, int64_t base, int lane,
                                        const CqParams& p) {
    constexpr int QMAX = (1 << (BITS - 1)) - 1;
    constexpr int LPB = B / kCqVec;  // lanes per scale block
    constexpr int SUB = 64 * kCqVec;
    float h[kCqUnroll][kCqVec];
    float e[kCqUnroll][kCqVec];

    // Issue every load of the tile first.
#pragma unroll
    for (int u = 0; u < kCqUnroll; ++u) {
        const int64_t i0 = base + u * SUB + lane * kCqVec;
        float g[kCqVec];
        if constexpr (FULL) {
            load8_nt<GBF>(sg.g, i0, g);
            load8<EBF>(sg.e, i0, e[u]);
        } else {
#pragma unroll
            for (int j = 0; j < kCqVec; ++j) {
                const bool ok = i0 + j < sg.n;
                g[j] = ok ? load1<GBF>(sg.g, i0 + j) : 0.0f;
                e[u][j] = ok ? load1<EBF>(sg.e, i0 + j) : 0.0f;
            }
        }
#pragma unroll
        for (int j = 0; j < kCqVec; ++j) h[u][j] = g[j] + e[u][j];  // Eqn. (2)
    }

#pragma unroll
    for (int u = 0; u < kCqUnroll; ++u) {
        const int64_t i0 = base + u * SUB + lane * kCqVec;
        float step, inv, am = 0.0f;
        if constexpr (FIXED) {
            step = p.fixed_step;
            inv = p.fixed_inv;
        } else {
            uint32_t m = 0;
#pragma unroll
            for (int j = 0; j < kCqVec; ++j) m = max(m, __float_as_uint(h[u][j]) & 0x7FFFFFFFu);
            m = group_max_u32<LPB>(m);
            am = __uint_as_float(m);
            step = am / (float)QMAX;
            inv = (m != 0u) ? 1.0f / step : 0.0f;
        }

        float en[kCqVec];
        uint32_t packed_lo = 0, packed_hi = 0;
#pragma unroll
        for (int j = 0; j < kCqVec; ++j) {
            const float x = h[u][j] * inv;
            const float rq = __builtin_amdgcn_fmed3f(__builtin_rintf(x), (float)(-QMAX - 1), (float)QMAX);
            const int q = (int)rq;
            const float d = (float)q * step;                     // decompressor
            const float r = h[u][j] - d;                         // Eqn. (4)
            en[j] = p.beta * e[u][j] + p.omega * r;              // Eqn. (5)
            const uint32_t f = (uint32_t)q & ((1u << BITS) - 1u);
            if constexpr (BITS == 8) {
                if (j < 4) packed_lo |= f << (8 * j);
                else packed_hi |= f << (8 * (j - 4));
            } else {
                packed_lo |= f << (BITS * j);
            }
        }

        if constexpr (FULL) {
            store8<EBF>(sg.e, i0, en);
            uint8_t* c = sg.codes + (i0 * BITS) / 8;
            if constexpr (BITS == 8) {
                u32x2 w = {packed_lo, packed_hi};
                __builtin_nontemporal_store(w, (u32x2*)c);
            } else if constexpr (BITS == 4) {
                __builtin_nontemporal_store(packed_lo, (uint32_t*)c);
            } else {
                __builtin_nontemporal_store((uint16_t)packed_lo, (uint16_t*)c);
            }
            if constexpr (!FIXED) {
                if (lane % LPB == 0) sg.absmax[i0 / B] = am;
            }
        } else {
            const int64_t left = sg.n - i0;
            const int nvalid = left <= 0 ? 0 : (left >= kCqVec ? kCqVec : (int)left);
#pragma unroll
            for (int j = 0; j < kCqVec; ++j)
                if (j < nvalid) store1<EBF>(sg.e, i0 + j, en[j]);
            const int nbytes = (nvalid * BITS + 7) / 8;
            uint8_t* c = sg.codes + (i0 * BITS) / 8;
#pragma unroll
            for (int b = 0; b < kCqVec * BITS / 8; ++b) {
                if (b < nbytes) {
                    const uint32_t w = (b < 4) ? packed_lo : packed_hi;
                    c[b] = (uint8_t)(w >> (8 * (b & 3)));
                }
            }
            if constexpr (!FIXED) {
                if (lane % LPB == 0 && nvalid > 0) sg.absmax[i0 / B] = am;
            }
        }
    }
}

// Segment of wave tile t: the last segment whose first tile is <= t (binary search over
// the launch's segment table; t is wave-uniform, so this runs on the scalar unit).
__device__ __forceinline__ int find_segment(const CqParams& p, int64_t t) {
    int lo = 0, hi = p.nseg - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (p.seg[mid].tile0 <= t) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

template <bool GBF, bool EBF, int BITS, int B, bool FIXED>
__global__ __launch_bounds__(kCqThreads) void cq_kernel(CqParams p) {
    const int lane = lane_id();
    const int64_t nwaves = (int64_t)gridDim.x * (kCqThreads / kWave);
    const int64_t wg = xcd_remap<kXcds, kCqXcdRun>(blockIdx.x, gridDim.x);
    for (int64_t t = wg * (kCqThreads / kWave) + uniform(threadIdx.x / kWave); t < p.ntiles;
         t += nwaves) {
        const CqSegDev sg = p.seg[find_segment(p, t)];
        const int64_t base = (t - sg.tile0) * kCqTile;
        if (base + kCqTile <= sg.n)
            cq_tile<GBF, EBF, BITS, B, FIXED, true>(sg, base, lane, p);
        else
            cq_tile<GBF, EBF, BITS, B, FIXED, false>(sg, base, lane, p);
    }
}

template <bool GBF, bool EBF, int BITS, bool FIXED>
const void* pick_block(int block) {
    if constexpr (FIXED) {
        return (const void*)&cq_kernel<GBF, EBF, BITS, 64, true>;
    } else {
        switch (block) {
            case 64: return (const void*)&cq_kernel<GBF, EBF, BITS, 64, false>;
            case 128: return (const void*)&cq_kernel<GBF, EBF, BITS, 128, false>;
            case 256: return (const void*)&cq_kernel<GBF, EBF, BITS, 256, false>;
            case 512: return (const void*)&cq_kernel<GBF, EBF, BITS, 512, false>;
        }
        return nullptr;
    }
}

template <bool GBF, bool EBF, bool FIXED>
const void* pick_bits(int bits, int block) {
    switch (bits) {
        case 2: return pick_block<GBF, EBF, 2, FIXED>(block);
        case 4: return pick_block<GBF, EBF, 4, FIXED>(block);
        case 8: return pick_block<GBF, EBF, 8, FIXED>(block);
    }
    return nullptr;
}

template <bool GBF, bool EBF>
const void* pick_fixed(bool fixed, int bits, int block) {
    return fixed ? pick_bits<GBF, EBF, true>(bits, block) : pick_bits<GBF, EBF, false>(bits, block);
}

}  // namespace

hipError_t launch_cq(const CqParams& p, bool grad_bf16, bool err_bf16, int bits, int block,
                     bool fixed, hipStream_t stream) {
    const void* k = nullptr;
    if (grad_bf16)
        k = err_bf16 ? pick_fixed<true, true>(fixed, bits, block) : pick_fixed<true, false>(fixed, bits, block);
    else
        k = err_bf16 ? pick_fixed<false, true>(fixed, bits, block) : pick_fixed<false, false>(fixed, bits, block);
    if (!k) return hipErrorInvalidValue;
    const int64_t waves_per_block = kCqThreads / kWave;
    int64_t blocks = (p.ntiles + waves_per_block - 1) / waves_per_block;
    if (blocks > kMaxGrid) blocks = kMaxGrid;
    if (blocks < 1) blocks = 1;
    void* args[] = {(void*)&p};
    return hipLaunchKernel(k, dim3((unsigned)blocks), dim3(kCqThreads), args, 0, stream);
}

}  // namespace loco
