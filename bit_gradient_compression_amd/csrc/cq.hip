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
// elements of each sub-tile, as two pieces of 4 consecutive elements at 4l and 256 + 4l
// where the gradient or the error is fp32, else as the 8 consecutive elements at 8l, so
// that every load and store instruction of the wave covers one contiguous run of memory
// (CqLayout).  The gradient and the error are loaded and the error stored non-temporally,
// except where a tile's first or last line of a stream is shared with a neighbouring tile.
// A scale block of B <= 256 elements is B/4 consecutive lanes of one piece (B/8 lanes of
// consecutive elements; a block of 512, both pieces of the wave); its absmax is reduced
// with DPP row operations (and permlane swaps past 16 lanes).  Every load of a tile is
// issued before any arithmetic.  The 8-bit-error kernel is bound by VALU issue as much as by
// HBM, so its per-element work is kept to a minimum: codes are packed from the float q
// with v_cvt_pk_u8_f32, the int8 error is encoded by a magic-number add and v_perm, and
// a wave issues the two divisions of its blocks once for all of its blocks (lane b
// divides for block b and stores its absmax; the results are shuffled to the blocks'
// lanes).
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

// Lane layout of a 512-element sub-tile.  Each lane owns 8 elements as two pieces of 4
// consecutive elements.  Split: the pieces sit at 4l and 256 + 4l, so every load and
// store instruction of the wave covers one contiguous run (1 KB of an fp32 stream).
// Contiguous: the lane's 8 elements are consecutive (8l), which already makes each
// instruction contiguous when every stream has at most 2 bytes per element (bf16
// gradient with a bf16 or 8-bit error).  The split layout is taken when the gradient or
// the error is fp32: there, the contiguous layout makes each 16-byte instruction touch
// half of every 32 bytes, and on MI355X the 7B shard's mix (bf16 gradient, fp32 error)
// then streams at 5.67 TB/s in its traffic twin against 6.0 TB/s split.  The 8-bit-error
// kernel is bound by instruction issue, and the split layout's extra reductions and
// narrower accesses cost it 7% (0.663 against 0.622 ms).
template <int GK, int EK>
struct CqLayout {
    static constexpr bool kSplit = GK == kF32 || EK == kF32;
    // element offset, within the sub-tile, of piece pc of lane l
    static __device__ __forceinline__ int piece(int l, int pc) { return kSplit ? pc * 256 + l * 4 : l * 8 + pc * 4; }
};

// Cache policy of the error stream: loaded and stored non-temporally (read once, written
// once per step).  Split layout: 6.0 TB/s in the 7B shard's twin against 5.6 with plain
// loads.  Contiguous layout: the MoE experts (bf16 error) 1.466 against 1.49 ms back to
// back; the 8-bit error unchanged.
#ifndef LOCO_CQ_E_LOAD_NT_SPLIT
#define LOCO_CQ_E_LOAD_NT_SPLIT 1
#endif
#ifndef LOCO_CQ_E_LOAD_NT_CONTIG
#define LOCO_CQ_E_LOAD_NT_CONTIG 1
#endif

template <class T, bool NT>
__device__ __forceinline__ T ld(const void* p) {
    if constexpr (NT) return __builtin_nontemporal_load((const T*)p);
    else return *(const T*)p;
}

constexpr int elem_bytes(int k) { return k == kI8 ? 1 : k == kBF16 ? 2 : 4; }

// The N elements of kind K held in the words w (as loaded from memory) as floats.
template <int K, int N>
__device__ __forceinline__ void words_to_f32(u32x4 w, float* x, float estep, float eoff) {
    if constexpr (K == kBF16) {
        x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
        if constexpr (N == 8) {
            x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
        }
    } else if constexpr (K == kI8) {
        i8x4_to_f32(w.x, estep, eoff, x);
        if constexpr (N == 8) i8x4_to_f32(w.y, estep, eoff, x + 4);
    } else {
        static_assert(N == 4, "fp32 elements come 4 at a time");
        x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y);
        x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
    }
}

// The N * elem_bytes(K) bytes (4, 8 or 16) at byte offset off of a buffer resource, with
// cache policy AUX (0: cached; kLoadNt: non-temporal).
template <int K, int N, int AUX>
__device__ __forceinline__ u32x4 load_words(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    constexpr int BYTES = N * elem_bytes(K);
    if constexpr (BYTES == 16) {
        return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
    } else if constexpr (BYTES == 8) {
        const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX);
        return u32x4{w.x, w.y, 0u, 0u};
    } else {
        static_assert(BYTES == 4, "4, 8 or 16 bytes per lane");
        return u32x4{__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX), 0u, 0u, 0u};
    }
}

// A segment need not start on a 128-byte line: then each stream's first and last line of
// a wave tile also hold elements of the neighbouring tiles.  Accessed non-temporally, such
// a line is fetched, and its halves written, separately for each of the two waves.  The
// lanes whose bytes lie in such a line load them with the cached policy instead, so that
// the two waves meet in L2; all other lanes load non-temporally.  Measured on the 7B
// shard, whose partitions start 64 bytes into a line of the fp32 error: 1.0066 of the
// algorithmic bytes and 1.365 ms, against 1.0118 and 1.380 ms with every load
// non-temporal (partitions padded to start on a line: 0.9997 and 1.35-1.36 ms).  Most of
// the time comes from the error's lines, whose writes then merge in L2.
#ifndef LOCO_CQ_EDGE_CACHED
#define LOCO_CQ_EDGE_CACHED 1
#endif
constexpr bool kEdgeCached = LOCO_CQ_EDGE_CACHED != 0;

template <int K, int N, bool NT>
__device__ __forceinline__ void loadn(const void* p, int64_t i0, float* x, float estep, float eoff);

// N elements of kind K at element i0 of a full wave tile [t0, t1) of stream p, as loadn
// with policy NT, except (EDGE) for the lanes in a shared edge line.  head / tail: this
// load instruction's row holds the tile's first / last element; a row in between has no
// shared edge line and loads as loadn does.  The edge rows load through a buffer resource
// over the tile, whose cache policy is an immediate: two global loads of one address that
// differ only in policy would be merged into one.
template <int K, int N, bool NT, bool EDGE>
__device__ __forceinline__ void loadn_tile(const void* p, int64_t t0, int64_t t1, int64_t i0, bool head, bool tail,
                                           float* x, float estep, float eoff) {
    if constexpr (EDGE && NT) {
        if (!head && !tail) {
            loadn<K, N, NT>(p, i0, x, estep, eoff);
            return;
        }
        constexpr int64_t S = elem_bytes(K);
        const char* tb = (const char*)p + t0 * S;  // wave-uniform
        const uint32_t bytes = (uint32_t)((t1 - t0) * S);
        const auto r = buffer_rsrc(tb, bytes);
        // offsets, within the tile, of its first and last line boundaries
        const uint32_t lo = (uint32_t)((128u - ((uintptr_t)tb & 127u)) & 127u);
        const uint32_t hi = (uint32_t)((((uintptr_t)tb + bytes) & ~(uintptr_t)127) - (uintptr_t)tb);
        const uint32_t off = (uint32_t)((i0 - t0) * S);
        u32x4 w;
        if ((head && off < lo) || (tail && off + (uint32_t)(N * S) > hi)) w = load_words<K, N, 0>(r, off);
        else w = load_words<K, N, kLoadNt>(r, off);
        words_to_f32<K, N>(w, x, estep, eoff);
    } else {
        loadn<K, N, NT>(p, i0, x, estep, eoff);
    }
}

// N = 4 or 8 consecutive elements starting at i0 (i0 a multiple of N).  NT: non-temporal.
template <int K, int N, bool NT>
__device__ __forceinline__ void loadn(const void* p, int64_t i0, float* x, float estep, float eoff) {
    if constexpr (K == kBF16) {
        if constexpr (N == 8) {
            const u32x4 w = ld<u32x4, NT>((const uint16_t*)p + i0);
            x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
            x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
        } else {
            const u32x2 w = ld<u32x2, NT>((const uint16_t*)p + i0);
            x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
        }
    } else if constexpr (K == kI8) {
        if constexpr (N == 8) {
            const u32x2 w = ld<u32x2, NT>((const int8_t*)p + i0);
            i8x4_to_f32(w.x, estep, eoff, x);
            i8x4_to_f32(w.y, estep, eoff, x + 4);
        } else {
            i8x4_to_f32(ld<uint32_t, NT>((const int8_t*)p + i0), estep, eoff, x);
        }
    } else {
#pragma unroll
        for (int v = 0; v < N / 4; ++v) {
            const f32x4 a = ld<f32x4, NT>((const float*)p + i0 + 4 * v);
            x[4 * v] = a.x; x[4 * v + 1] = a.y; x[4 * v + 2] = a.z; x[4 * v + 3] = a.w;
        }
    }
}

// N = 4 or 8 consecutive elements of the new error (non-temporal).  keep is all ones, or
// 0 on a reset step (store 0 instead): a mask on the stored words, so that the step's
// arithmetic stays branch-free.
template <int K, int N>
__device__ __forceinline__ void storen(void* p, int64_t i0, const float* x, float escale, uint32_t keep) {
    if constexpr (K == kBF16) {
        if constexpr (N == 8) {
            const u32x4 w = {bf16x2_rne(x[0], x[1]), bf16x2_rne(x[2], x[3]), bf16x2_rne(x[4], x[5]),
                             bf16x2_rne(x[6], x[7])};
            __builtin_nontemporal_store(w & keep, (u32x4*)((uint16_t*)p + i0));
        } else {
            const u32x2 w = {bf16x2_rne(x[0], x[1]), bf16x2_rne(x[2], x[3])};
            __builtin_nontemporal_store(w & keep, (u32x2*)((uint16_t*)p + i0));
        }
    } else if constexpr (K == kI8) {
        uint32_t w[N / 4];
#pragma unroll
        for (int v = 0; v < N / 4; ++v)
            w[v] = keep & low_bytes4(i8_code_bits(x[4 * v], escale), i8_code_bits(x[4 * v + 1], escale),
                                     i8_code_bits(x[4 * v + 2], escale), i8_code_bits(x[4 * v + 3], escale));
        if constexpr (N == 8) __builtin_nontemporal_store(u32x2{w[0], w[1]}, (u32x2*)((int8_t*)p + i0));
        else __builtin_nontemporal_store(w[0], (uint32_t*)((int8_t*)p + i0));
    } else {
#pragma unroll
        for (int v = 0; v < N / 4; ++v) {
            const u32x4 a = {__float_as_uint(x[4 * v]), __float_as_uint(x[4 * v + 1]), __float_as_uint(x[4 * v + 2]),
                             __float_as_uint(x[4 * v + 3])};
            __builtin_nontemporal_store(a & keep, (u32x4*)((float*)p + i0) + v);
        }
    }
}

// The codes of N = 4 or 8 consecutive elements (N*BITS/8 bytes, low bits of lo:hi first)
// at element i0 (a multiple of N).
template <int BITS, int N>
__device__ __forceinline__ void store_codes(uint8_t* codes, int64_t i0, uint32_t lo, uint32_t hi) {
    uint8_t* c = codes + (i0 * BITS) / 8;
    constexpr int NB = N * BITS / 8;
    if constexpr (NB == 8) __builtin_nontemporal_store(u32x2{lo, hi}, (u32x2*)c);
    else if constexpr (NB == 4) __builtin_nontemporal_store(lo, (uint32_t*)c);
    else if constexpr (NB == 2) __builtin_nontemporal_store((uint16_t)lo, (uint16_t*)c);
    else __builtin_nontemporal_store((uint8_t)lo, c);
}

// U sub-tiles of 512 elements from element `base` of the segment, in the lane layout of
// CqLayout.  Element j < 4 of the lane is piece 0's j, element j >= 4 piece 1's j - 4.
// FULL: all U sub-tiles are inside the segment; otherwise elements past its end are
// neither read nor written.
template <int GK, int EK, int BITS, int B, bool FIXED, bool FULL, int U>
__device__ __forceinline__ void cq_tile(const CqSegDev& sg, int64_t base, int lane,
                                        const CqParams& p) {
    using LY = CqLayout<GK, EK>;
    constexpr bool SPLIT = LY::kSplit;
    constexpr int QMAX = (1 << (BITS - 1)) - 1;
    constexpr int SUB = 64 * kCqVec;
    constexpr bool ENT = SPLIT ? LOCO_CQ_E_LOAD_NT_SPLIT != 0 : LOCO_CQ_E_LOAD_NT_CONTIG != 0;
    float h[U][kCqVec];
    float e[U][kCqVec];
    const float eoff = -128.0f * p.err_step;  // the 8-bit error's decoder offset
    // Not with an 8-bit error: that kernel is bound by instruction issue, and with edge
    // lanes it ran 1% slower back to back on the 7B shard (0.617 against 0.611 ms), though
    // 1.5% faster cache-flushed (0.600 against 0.609).
    constexpr bool EDGE = kEdgeCached && EK != kI8;

    // Issue every load of the tile first.
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float g[kCqVec];
        if constexpr (FULL && !SPLIT) {
            const int64_t i0 = base + u * SUB + LY::piece(lane, 0);
            const bool head = u == 0, tail = u == U - 1;  // rows: the sub-tiles
            loadn_tile<GK, 8, true, EDGE>(sg.g, base, base + U * SUB, i0, head, tail, g, 0.0f, 0.0f);
            loadn_tile<EK, 8, ENT, EDGE>(sg.e, base, base + U * SUB, i0, head, tail, e[u], p.err_step, eoff);
        } else {
#pragma unroll
            for (int pc = 0; pc < 2; ++pc) {
                const int64_t i0 = base + u * SUB + LY::piece(lane, pc);
                if constexpr (FULL) {
                    const bool head = u == 0 && pc == 0, tail = u == U - 1 && pc == 1;  // rows: the pieces
                    loadn_tile<GK, 4, true, EDGE>(sg.g, base, base + U * SUB, i0, head, tail, g + 4 * pc, 0.0f, 0.0f);
                    loadn_tile<EK, 4, ENT, EDGE>(sg.e, base, base + U * SUB, i0, head, tail, e[u] + 4 * pc,
                                                 p.err_step, eoff);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const bool ok = i0 + j < sg.n;
                        g[4 * pc + j] = ok ? load1<GK>(sg.g, i0 + j, 0.0f) : 0.0f;
                        e[u][4 * pc + j] = ok ? load1<EK>(sg.e, i0 + j, p.err_step) : 0.0f;
                    }
                }
            }
        }
#pragma unroll
        for (int j = 0; j < kCqVec; ++j) h[u][j] = g[j] + e[u][j];  // Eqn. (2)
    }

    // Block scales.  In the split layout a block of B <= 256 elements is B/4 consecutive
    // lanes of one piece (a block of 512 is both pieces of all lanes); in the contiguous
    // layout it is B/8 consecutive lanes.  The maxima of |h| are reduced over each block's
    // lanes (DPP, permlane swaps); then lane b takes the tile's b-th block maximum,
    // divides once (step = absmax / qmax, inv = 1 / step, 0 where not finite) and stores
    // that block's absmax, and every lane fetches the step and inverse of its blocks:
    // two divisions per lane per tile, whatever the number of blocks.
    constexpr int BPS = SUB / B;  // blocks per sub-tile
    constexpr int NB = U * BPS;   // blocks per tile (<= 16)
    constexpr int LPB = SPLIT ? (B <= SUB / 2 ? B / 4 : 64) : B / 8;  // a block's lanes in a piece
    float stepA[U], invA[U], stepB[U], invB[U];
    if constexpr (FIXED) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            stepA[u] = stepB[u] = p.fixed_step;
            invA[u] = invB[u] = p.fixed_inv;
        }
    } else {
        uint32_t mA[U], mB[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // max |h| as a float (|x| is a free source modifier): for finite values the
            // same element, and the same bits, as the largest |h| bit pattern
            float fa = 0.0f, fb = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                fa = fmaxf(fa, fabsf(h[u][j]));
                fb = fmaxf(fb, fabsf(h[u][4 + j]));
            }
            if constexpr (SPLIT && B <= SUB / 2) {
                mA[u] = group_max_u32<LPB>(__float_as_uint(fa));
                mB[u] = group_max_u32<LPB>(__float_as_uint(fb));
            } else {
                mA[u] = mB[u] = group_max_u32<LPB>(__float_as_uint(fmaxf(fa, fb)));
            }
        }
        // lane b < NB: block b of the tile, block k = b % BPS of sub-tile b / BPS.  Split:
        // piece 0's block k (k < BPS/2) or piece 1's block k - BPS/2, at lane
        // (k % (BPS/2)) * LPB (a block of 512: lane 0).  Contiguous: lane k * LPB.
        constexpr bool TWO = SPLIT && BPS >= 2;
        const int k = lane % BPS;
        const int src = TWO ? (k % (BPS / 2)) * LPB : k * LPB;
        uint32_t mb = 0u;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t va = (uint32_t)__shfl((int)mA[u], src, 64);
            uint32_t v = va;
            if constexpr (TWO) {
                const uint32_t vb = (uint32_t)__shfl((int)mB[u], src, 64);
                v = k >= BPS / 2 ? vb : va;
            }
            mb = (lane / BPS == u) ? v : mb;
        }
        const float amb = __uint_as_float(mb);
        const float stepb = amb / (float)QMAX;
        const float invb = finite_recip(stepb);
        // the block's absmax, stored by its lane (blocks past a ragged end are skipped)
        if (lane < NB) {
            if (FULL || base + (int64_t)lane * B < sg.n) sg.absmax[base / B + lane] = amb;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int ba = u * BPS + LY::piece(lane, 0) / B;  // piece 0's block in the tile
            stepA[u] = __shfl(stepb, ba, 64);
            invA[u] = __shfl(invb, ba, 64);
            if constexpr (SPLIT && B <= SUB / 2) {
                const int bb = u * BPS + LY::piece(lane, 1) / B;  // piece 1's block
                stepB[u] = __shfl(stepb, bb, 64);
                invB[u] = __shfl(invb, bb, 64);
            } else {
                stepB[u] = stepA[u];
                invB[u] = invA[u];
            }
        }
    }

#pragma unroll
    for (int u = 0; u < U; ++u) {
        float en[kCqVec], rq[kCqVec];
#pragma unroll
        for (int j = 0; j < kCqVec; ++j) {
            const float step = j < 4 ? stepA[u] : stepB[u];
            const float inv = j < 4 ? invA[u] : invB[u];
            const float x = h[u][j] * inv;
            rq[j] = __builtin_amdgcn_fmed3f(__builtin_rintf(x), (float)(-QMAX - 1), (float)QMAX);
            const float d = rq[j] * step;                        // decompressor (rq is the integer q)
            const float r = h[u][j] - d;                         // Eqn. (4)
            en[j] = p.beta * e[u][j] + p.omega * r;              // Eqn. (5)
        }
        // packed codes: element j of the lane at bits [BITS*j, BITS*j + BITS) of lo:hi, so
        // piece 0's 4 codes are the low 4*BITS bits and piece 1's the next 4*BITS
        uint32_t packed_lo, packed_hi;
        pack_codes8<BITS>(rq, packed_lo, packed_hi);
        uint32_t cw[2];
        if constexpr (BITS == 8) {
            cw[0] = packed_lo;
            cw[1] = packed_hi;
        } else {
            cw[0] = packed_lo & ((1u << (4 * BITS)) - 1u);
            cw[1] = packed_lo >> (4 * BITS);
        }
        const bool zero = p.reset;  // Eqn. (7): this step stores a zero error
        const uint32_t keep = zero ? 0u : ~0u;

        if constexpr (FULL && !SPLIT) {
            const int64_t i0 = base + u * SUB + LY::piece(lane, 0);
            storen<EK, 8>(sg.e, i0, en, p.err_scale, keep);
            store_codes<BITS, 8>(sg.codes, i0, packed_lo, packed_hi);
        } else {
#pragma unroll
            for (int pc = 0; pc < 2; ++pc) {
                const int64_t i0 = base + u * SUB + LY::piece(lane, pc);
                if constexpr (FULL) {
                    storen<EK, 4>(sg.e, i0, en + 4 * pc, p.err_scale, keep);
                    store_codes<BITS, 4>(sg.codes, i0, cw[pc], 0u);
                } else {
                    const int64_t left = sg.n - i0;
                    const int nvalid = left <= 0 ? 0 : (left >= 4 ? 4 : (int)left);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (j < nvalid) store1<EK>(sg.e, i0 + j, zero ? 0.0f : en[4 * pc + j], p.err_scale);
                    const int nbytes = (nvalid * BITS + 7) / 8;
                    uint8_t* c = sg.codes + (i0 * BITS) / 8;
#pragma unroll
                    for (int b = 0; b < BITS / 2; ++b)
                        if (b < nbytes) c[b] = (uint8_t)(cw[pc] >> (8 * b));
                }
            }
        }
    }
}

// Segment of wave tile t: the last segment whose first tile is <= t (binary search over
// the launch's segment table; t is wave-uniform, so this runs on the scalar unit).
// (Counting the first tiles <= t over a packed array instead, all loaded at once, measured
// no faster: 1.40 ms on the 7B shard either way, and slower back to back for the 8-bit
// error, 0.665 against 0.627 ms.)
__device__ __forceinline__ int find_segment(const CqParams& p, int64_t t) {
    int lo = 0, hi = p.nseg - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (p.seg[mid].tile0 <= t) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// One wave tile per wave: tile tbase + (the wave's index in the launch).  Nothing is
// carried from tile to tile (33 VGPRs for the 7B shard's kernel, 50 with an 8-bit error).
template <int GK, int EK, int BITS, int B, bool FIXED>
__global__ __launch_bounds__(cq_threads(EK)) void cq_kernel(CqParams p, int64_t tbase) {
    const int lane = lane_id();
    constexpr int TILE = cq_tile_elems(EK);
    const int64_t wg = xcd_remap<kXcds, cq_xcd_run(EK)>(blockIdx.x, gridDim.x);
    const int64_t t = tbase + wg * (cq_threads(EK) / kWave) + uniform(threadIdx.x / kWave);
    if (t >= p.ntiles) return;
    const CqSegDev sg = p.seg[find_segment(p, t)];
    const int64_t base = (t - sg.tile0) * TILE;
    if (base + TILE <= sg.n) {
        cq_tile<GK, EK, BITS, B, FIXED, true, cq_unroll(EK)>(sg, base, lane, p);
    } else {
        // the segment's ragged last tile, one sub-tile at a time (a sub-tile holds whole
        // blocks), so that its bounds checks do not raise the kernel's register count
#pragma unroll 1
        for (int u = 0; u < cq_unroll(EK) && base + u * 64 * kCqVec < sg.n; ++u)
            cq_tile<GK, EK, BITS, B, FIXED, false, 1>(sg, base + u * 64 * kCqVec, lane, p);
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
    // one wave per tile; launches of at most kMaxGrid workgroups
    const int threads = cq_threads(err_kind);
    const int64_t waves_per_block = threads / kWave;
    const int64_t per_launch = kMaxGrid * waves_per_block;
    for (int64_t tbase = 0; tbase < p.ntiles; tbase += per_launch) {
        const int64_t tiles = p.ntiles - tbase < per_launch ? p.ntiles - tbase : per_launch;
        const int64_t blocks = (tiles + waves_per_block - 1) / waves_per_block;
        void* args[] = {(void*)&p, (void*)&tbase};
        const hipError_t err = hipLaunchKernel(k, dim3((unsigned)blocks), dim3(threads), args, 0, stream);
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace loco
