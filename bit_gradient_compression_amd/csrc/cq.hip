// Fused compensate -> block absmax -> quantize -> pack -> error update, one HBM pass.
//
// LoCo ("LoCo: Low-Bit Communication Adaptor for Large-scale Model Training"),
// Sec. 3.1 Eqns. (1)-(3) and Sec. 3.2 Eqns. (4)-(5), with a per-block absmax scale:
//   h = g + e;  absmax = max|h| per block;  step = absmax/qmax;  inv = 1/step (0 where
//   that is not finite: an all-zero block, or one too small for its reciprocal)
//   q = clamp(rint(h*inv));  r = h - q*step;  e' = beta*e + (1-beta)*r
// The error is stored as fp32, bf16, or the paper's 8-bit codes of a fixed scale s_e
// (Sec. 3.2, Eqn. (7): e = e8 * fl(1/s_e) on load, e8' = clamp(rint(e' * s_e)) on store),
// and a step may store e' = 0 instead (the periodic reset of Eqn. (7)).
//
// Mapping: a wavefront owns a tile of sub-tiles of 512 elements (one sub-tile with a
// float error, two with an 8-bit error, whose waves move fewer bytes); lane l owns 8
// consecutive elements of each sub-tile, so one bf16 gradient load, two fp32 error loads
// (one 8-byte load of an 8-bit error) and one 32-bit code store per lane are coalesced.
// A scale block of B elements is B/8 consecutive lanes; its absmax is reduced with DPP
// row operations (and a permlane swap past 16 lanes).  Every load of a tile is issued
// before any arithmetic.  The 8-bit-error kernel is bound by VALU issue as much as by
// HBM, so its per-element work is kept to a minimum: codes are packed from the float q
// with v_cvt_pk_u8_f32, the int8 error is encoded by a magic-number add and v_perm, and
// a wave issues the two divisions of its blocks once for both sub-tiles (each lane
// divides for one block; the results are shuffled to the block's lanes).
// The grid covers all wave tiles of all segments of the call: each wave takes one tile
// and exits, so the waves in flight sweep the buffers in address order (measured on
// MI355X, a persistent grid-stride loop over the same traffic mix runs ~15% slower).

#include "loco_device.hpp"
#include "loco_internal.hpp"

namespace loco {
namespace {

// Element kinds of the gradient (F32, BF16) and of the error (F32, BF16, I8).
enum : int { kF32 = 0, kBF16 = 1, kI8 = 2 };

template <int K>
__device__ __forceinline__ float load1(const void* p, int64_t i, float estep) {
    if constexpr (K == kBF16) return __uint_as_float((uint32_t)((const uint16_t*)p)[i] << 16);
    else if constexpr (K == kI8) return (float)((const int8_t*)p)[i] * estep;
    else return ((const float*)p)[i];
}

// The int8 error code of x: clamp(rint(x * escale), -128, 127), ties to even, as the low
// byte of a float's bits.  Clamping before rounding gives the same integer (the bounds are
// integers), and adding 1.5 * 2^23 to a value in [-128, 127] rounds it to an integer (ties
// to even) held in the low mantissa bits, two's complement in the low byte.
__device__ __forceinline__ uint32_t i8_code_bits(float x, float escale) {
    return __float_as_uint(__builtin_amdgcn_fmed3f(x * escale, -128.0f, 127.0f) + 12582912.0f);
}

template <int K>
__device__ __forceinline__ void store1(void* p, int64_t i, float v, float escale) {
    if constexpr (K == kBF16) ((uint16_t*)p)[i] = bf16_rne(v);
    else if constexpr (K == kI8) ((int8_t*)p)[i] = (int8_t)(i8_code_bits(v, escale) & 0xFFu);
    else ((float*)p)[i] = v;
}

// 4 int8 codes (one word, biased by 0x80) -> e8 * estep, as fma(e8 + 128, estep,
// -128 * estep): its exact value is e8 * estep, rounded once, the same as the product.
__device__ __forceinline__ void i8x4_to_f32(uint32_t w, float estep, float off, float* x) {
    const uint32_t u = w ^ 0x80808080u;
    x[0] = __builtin_fmaf(ubyte_to_f32<0>(u), estep, off);
    x[1] = __builtin_fmaf(ubyte_to_f32<1>(u), estep, off);
    x[2] = __builtin_fmaf(ubyte_to_f32<2>(u), estep, off);
    x[3] = __builtin_fmaf(ubyte_to_f32<3>(u), estep, off);
}

// 8 consecutive elements starting at i0 (16-byte aligned for 2- and 4-byte kinds, 8-byte
// for int8).  NT: non-temporal (the gradient is read once).
template <int K, bool NT>
__device__ __forceinline__ void load8(const void* p, int64_t i0, float (&x)[8], float estep) {
    if constexpr (K == kBF16) {
        const u32x4* q = (const u32x4*)((const uint16_t*)p + i0);
        const u32x4 w = NT ? __builtin_nontemporal_load(q) : *q;
        x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
        x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
    } else if constexpr (K == kI8) {
        const u32x2* q = (const u32x2*)((const int8_t*)p + i0);
        const u32x2 w = NT ? __builtin_nontemporal_load(q) : *q;
        const float off = -128.0f * estep;
        i8x4_to_f32(w.x, estep, off, x);
        i8x4_to_f32(w.y, estep, off, x + 4);
    } else {
        const f32x4* q = (const f32x4*)((const float*)p + i0);
        const f32x4 a = NT ? __builtin_nontemporal_load(q) : q[0];
        const f32x4 b = NT ? __builtin_nontemporal_load(q + 1) : q[1];
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
}

// 8 consecutive elements of the new error; zero: store 0 instead (the error reset).
template <int K>
__device__ __forceinline__ void store8(void* p, int64_t i0, const float (&x)[8], float escale, bool zero) {
    if constexpr (K == kBF16) {
        u32x4 w;
        w.x = bf16x2_rne(x[0], x[1]); w.y = bf16x2_rne(x[2], x[3]);
        w.z = bf16x2_rne(x[4], x[5]); w.w = bf16x2_rne(x[6], x[7]);
        if (zero) w = u32x4{0u, 0u, 0u, 0u};
        __builtin_nontemporal_store(w, (u32x4*)((uint16_t*)p + i0));
    } else if constexpr (K == kI8) {
        u32x2 w = {low_bytes4(i8_code_bits(x[0], escale), i8_code_bits(x[1], escale), i8_code_bits(x[2], escale),
                              i8_code_bits(x[3], escale)),
                   low_bytes4(i8_code_bits(x[4], escale), i8_code_bits(x[5], escale), i8_code_bits(x[6], escale),
                              i8_code_bits(x[7], escale))};
        if (zero) w = u32x2{0u, 0u};
        __builtin_nontemporal_store(w, (u32x2*)((int8_t*)p + i0));
    } else {
        f32x4* q = (f32x4*)((float*)p + i0);
        f32x4 a = {x[0], x[1], x[2], x[3]};
        f32x4 b = {x[4], x[5], x[6], x[7]};
        if (zero) {
            a = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            b = a;
        }
        __builtin_nontemporal_store(a, q);
        __builtin_nontemporal_store(b, q + 1);
    }
}

template <int GK, int EK, int BITS, int B, bool FIXED, bool FULL>
__device__ __forceinline__ void cq_tile(const CqSegDev& sg, int64_t base, int lane,
                                        const CqParams& p) {
    constexpr int QMAX = (1 << (BITS - 1)) - 1;
    constexpr int LPB = B / kCqVec;  // lanes per scale block
    constexpr int SUB = 64 * kCqVec;
    constexpr int U = cq_unroll(EK);
    float h[U][kCqVec];
    float e[U][kCqVec];

    // Issue every load of the tile first.
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t i0 = base + u * SUB + lane * kCqVec;
        float g[kCqVec];
        if constexpr (FULL) {
            load8<GK, true>(sg.g, i0, g, 0.0f);
            load8<EK, false>(sg.e, i0, e[u], p.err_step);
        } else {
#pragma unroll
            for (int j = 0; j < kCqVec; ++j) {
                const bool ok = i0 + j < sg.n;
                g[j] = ok ? load1<GK>(sg.g, i0 + j, 0.0f) : 0.0f;
                e[u][j] = ok ? load1<EK>(sg.e, i0 + j, p.err_step) : 0.0f;
            }
        }
#pragma unroll
        for (int j = 0; j < kCqVec; ++j) h[u][j] = g[j] + e[u][j];  // Eqn. (2)
    }

    // Block scales.  With several sub-tiles per wave, lane b takes the maximum of the
    // tile's b-th block and divides once (step = absmax / qmax, inv = 1 / step); each lane
    // then fetches its own block's pair: the same quotients, one division per block
    // instead of one per lane.
    constexpr int BPS = 64 / LPB;  // blocks per sub-tile
    float step_u[U], inv_u[U], am_u[U];
    if constexpr (FIXED) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            step_u[u] = p.fixed_step;
            inv_u[u] = p.fixed_inv;
            am_u[u] = 0.0f;
        }
    } else {
        uint32_t mu[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // max |h| as a float (|x| is a free source modifier): for finite values the
            // same element, and the same bits, as the largest |h| bit pattern
            float mf = 0.0f;
#pragma unroll
            for (int j = 0; j < kCqVec; ++j) mf = fmaxf(mf, fabsf(h[u][j]));
            mu[u] = group_max_u32<LPB>(__float_as_uint(mf));
            am_u[u] = __uint_as_float(mu[u]);
        }
        if constexpr (U > 1) {
            uint32_t mb = 0;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t v = (uint32_t)__shfl((int)mu[u], (lane % BPS) * LPB, 64);
                mb = (lane / BPS == u) ? v : mb;
            }
            const float stepb = __uint_as_float(mb) / (float)QMAX;
            const float invb = finite_recip(stepb);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int src = u * BPS + lane / LPB;
                step_u[u] = __shfl(stepb, src, 64);
                inv_u[u] = __shfl(invb, src, 64);
            }
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                step_u[u] = am_u[u] / (float)QMAX;
                inv_u[u] = finite_recip(step_u[u]);
            }
        }
    }

#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t i0 = base + u * SUB + lane * kCqVec;
        const float step = step_u[u], inv = inv_u[u], am = am_u[u];

        float en[kCqVec], rq[kCqVec];
#pragma unroll
        for (int j = 0; j < kCqVec; ++j) {
            const float x = h[u][j] * inv;
            rq[j] = __builtin_amdgcn_fmed3f(__builtin_rintf(x), (float)(-QMAX - 1), (float)QMAX);
            const float d = rq[j] * step;                        // decompressor (rq is the integer q)
            const float r = h[u][j] - d;                         // Eqn. (4)
            en[j] = p.beta * e[u][j] + p.omega * r;              // Eqn. (5)
        }
        uint32_t packed_lo, packed_hi;
        pack_codes8<BITS>(rq, packed_lo, packed_hi);
        const bool zero = p.reset;  // Eqn. (7): this step stores a zero error

        if constexpr (FULL) {
            store8<EK>(sg.e, i0, en, p.err_scale, zero);
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
                if (j < nvalid) store1<EK>(sg.e, i0 + j, zero ? 0.0f : en[j], p.err_scale);
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

template <int GK, int EK, int BITS, int B, bool FIXED>
__global__ __launch_bounds__(kCqThreads) void cq_kernel(CqParams p) {
    const int lane = lane_id();
    const int64_t nwaves = (int64_t)gridDim.x * (kCqThreads / kWave);
    constexpr int TILE = cq_tile_elems(EK);
    const int64_t wg = xcd_remap<kXcds, EK == kI8 ? kCqXcdRunI8 : kCqXcdRun>(blockIdx.x, gridDim.x);
    for (int64_t t = wg * (kCqThreads / kWave) + uniform(threadIdx.x / kWave); t < p.ntiles;
         t += nwaves) {
        const CqSegDev sg = p.seg[find_segment(p, t)];
        const int64_t base = (t - sg.tile0) * TILE;
        if (base + TILE <= sg.n)
            cq_tile<GK, EK, BITS, B, FIXED, true>(sg, base, lane, p);
        else
            cq_tile<GK, EK, BITS, B, FIXED, false>(sg, base, lane, p);
    }
}

template <int GK, int EK, int BITS, bool FIXED>
const void* pick_block(int block) {
    if constexpr (FIXED) {
        return (const void*)&cq_kernel<GK, EK, BITS, 64, true>;
    } else {
        switch (block) {
            case 64: return (const void*)&cq_kernel<GK, EK, BITS, 64, false>;
            case 128: return (const void*)&cq_kernel<GK, EK, BITS, 128, false>;
            case 256: return (const void*)&cq_kernel<GK, EK, BITS, 256, false>;
            case 512: return (const void*)&cq_kernel<GK, EK, BITS, 512, false>;
        }
        return nullptr;
    }
}

template <int GK, int EK, bool FIXED>
const void* pick_bits(int bits, int block) {
    switch (bits) {
        case 2: return pick_block<GK, EK, 2, FIXED>(block);
        case 4: return pick_block<GK, EK, 4, FIXED>(block);
        case 8: return pick_block<GK, EK, 8, FIXED>(block);
    }
    return nullptr;
}

template <int GK, int EK>
const void* pick_fixed(bool fixed, int bits, int block) {
    return fixed ? pick_bits<GK, EK, true>(bits, block) : pick_bits<GK, EK, false>(bits, block);
}

template <int GK>
const void* pick_err(int err_kind, bool fixed, int bits, int block) {
    switch (err_kind) {
        case kF32: return pick_fixed<GK, kF32>(fixed, bits, block);
        case kBF16: return pick_fixed<GK, kBF16>(fixed, bits, block);
        case kI8: return pick_fixed<GK, kI8>(fixed, bits, block);
    }
    return nullptr;
}

}  // namespace

hipError_t launch_cq(const CqParams& p, int grad_kind, int err_kind, int bits, int block, bool fixed,
                     hipStream_t stream) {
    const void* k = nullptr;
    if (grad_kind == kBF16) k = pick_err<kBF16>(err_kind, fixed, bits, block);
    else if (grad_kind == kF32) k = pick_err<kF32>(err_kind, fixed, bits, block);
    if (!k) return hipErrorInvalidValue;
    const int64_t waves_per_block = kCqThreads / kWave;
    int64_t blocks = (p.ntiles + waves_per_block - 1) / waves_per_block;
    if (blocks > kMaxGrid) blocks = kMaxGrid;
    if (blocks < 1) blocks = 1;
    void* args[] = {(void*)&p};
    return hipLaunchKernel(k, dim3((unsigned)blocks), dim3(kCqThreads), args, 0, stream);
}

}  // namespace loco
