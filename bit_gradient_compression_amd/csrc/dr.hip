// Dequantize and average the peers' low-bit payloads of one partition.
//
// LoCo ("LoCo: Low-Bit Communication Adaptor for Large-scale Model Training"),
// Sec. 3.3, Eqn. (8): each node gathers the N low-bit partitions it owns (all2all) and
// averages their decompressed values in high precision:
//   acc = sum over p = 0..N-1 (in that order) of q_p * step_p;  out = acc * out_scale
//
// Mapping: a wave tile is one or two sub-tiles of 512 outputs; lane l owns 8 outputs of
// each sub-tile as two pieces of 4 consecutive elements (DrLayout): consecutive (8l) for
// a bf16 shard, at 4l and 256 + 4l for an fp32 shard and the fused Adam step, so that
// every load and store instruction of the wave covers one contiguous run.  A piece sits
// in one scale block (blocks are >= 64 elements).  The fp32 accumulator never leaves
// registers; only the reduced shard is written.  One wave tile per wave, the grid
// covering all tiles.
//
// Fused consumer (LoCo, Sec. 4, Eqn. (9)): instead of writing the reduced gradient g,
// the kernel takes one Adam-family step with it on the partition's fp32 weights and
// moments, which it reads and writes in the same pass:
//   m' = (1-b1) m + b1 g;  v' = (1-b2) v + b2 g^2;  u = 1 / sqrt(v' + delta)
//   theta' = theta - lr (m' u)
// and optionally writes a bf16 copy of theta'.  The reduced gradient never reaches HBM.

#include "loco_device.hpp"
#include "loco_internal.hpp"

namespace loco {
namespace {

// Codes of N = 4 or 8 consecutive elements (N*BITS/8 bytes) at byte offset off of a
// peer's tile, in the low bits.
template <int BITS, int N>
__device__ __forceinline__ u32x2 load_codes_at(__amdgpu_buffer_rsrc_t tile, uint32_t off) {
    constexpr int NB = N * BITS / 8;
    if constexpr (NB == 1) return u32x2{(uint32_t)__builtin_amdgcn_raw_buffer_load_b8(tile, off, 0, kLoadNt), 0u};
    else if constexpr (NB == 2) return u32x2{(uint32_t)__builtin_amdgcn_raw_buffer_load_b16(tile, off, 0, kLoadNt), 0u};
    else if constexpr (NB == 4) return u32x2{__builtin_amdgcn_raw_buffer_load_b32(tile, off, 0, kLoadNt), 0u};
    else return __builtin_amdgcn_raw_buffer_load_b64(tile, off, 0, kLoadNt);
}

// Signed code j (0..7) of the 8 held in w.
template <int BITS>
__device__ __forceinline__ int code_of(u32x2 w, int j) {
    if constexpr (BITS == 8) return __builtin_amdgcn_sbfe(j < 4 ? w.x : w.y, (j & 3) * 8, 8);
    else return __builtin_amdgcn_sbfe(w.x, j * BITS, BITS);
}

// Decoding of 4- and 8-bit codes.  A code is biased to unsigned (c = q + 2^(b-1), one xor
// for a word of codes) and fl(q*step) is formed as fma(c, step, -2^(b-1)*step): the fma's
// exact value is q*step, rounded once, so the result is bit-identical to rounding q*step
// (2^(b-1)*step is exact).  1: c enters the fma as a binary16 subnormal, c * 2^-24, taken
// straight from the low or high half of a word of masked codes by the mixed-precision fma
// (v_fma_mix_f32), against a step scaled by 2^24 (exact); a 4-bit code masked at bits 4-7
// of a half reads as 16c * 2^-24 and meets the step scaled by 2^20.  Per code: 5/8 (4-bit)
// or 3/4 (8-bit) of a bias-mask-shift instruction, one fma, one add.  0: c is converted
// with the byte converts (v_cvt_f32_ubyteN).
#ifndef LOCO_DR_DECODE_F16
#define LOCO_DR_DECODE_F16 1
#endif
constexpr bool kDecodeF16 = LOCO_DR_DECODE_F16 != 0;
constexpr float kF16SubScale = 0x1p24f;  // 2^24: a binary16 subnormal m is m * 2^-24

// The binary16 value of the low / high half of x (m * 2^-24 for m < 1024).
__device__ __forceinline__ float half_lo(uint32_t x) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(x & 0xFFFFu));
}
__device__ __forceinline__ float half_hi(uint32_t x) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(x >> 16));
}

template <int N>
__device__ __forceinline__ void acc_byte(float& a, uint32_t x, float step, float off) {
    a = a + __builtin_fmaf(ubyte_to_f32<N>(x), step, off);
}

// acc[j] += fl(q_j * step) for the 8 codes held in w: codes 0-3 with the scale (sa, oa),
// codes 4-7 with (sb, ob) (the lane's two pieces may sit in different scale blocks).
// w.x holds codes 0-3 in its low and 4-7 in its high 16 bits at 4 bits (2 bits: low and
// high byte); at 8 bits w.x holds codes 0-3 and w.y codes 4-7.
// 2 bits: acc + (float)q * step.  4 and 8 bits: s is step * 2^24 (LOCO_DR_DECODE_F16) or
// step, o = -2^(b-1) * step, with |step| < 2^100 so that neither overflows; s16 (4 bits,
// LOCO_DR_DECODE_F16) is step * 2^20, for the codes held at bits 4-7 of a half.
template <int BITS>
__device__ __forceinline__ void accumulate8(float (&acc)[kDrVec], u32x2 w, float sa, float oa, float sb, float ob,
                                            float sa16, float sb16) {
    if constexpr (BITS == 2) {
#pragma unroll
        for (int j = 0; j < kDrVec; ++j) acc[j] = acc[j] + (float)code_of<BITS>(w, j) * (j < 4 ? sa : sb);
    } else if constexpr (kDecodeF16 && BITS == 4) {
        // Codes j and j + 4 sit in nibble j of the low and the high half.  Nibbles 0 and
        // 1 of each half are masked in place (nibble 1 reads as 16c * 2^-24, against
        // s16); one shift brings nibbles 2 and 3 down to the same places: 5 instructions
        // (4 xor-and, 1 shift) bias and mask 8 codes, where shifting every nibble down
        // took 8.
        const uint32_t y = w.x >> 8;
        const uint32_t c04 = (w.x ^ 0x88888888u) & 0x000F000Fu, c15 = (w.x ^ 0x88888888u) & 0x00F000F0u;
        const uint32_t c26 = (y ^ 0x88888888u) & 0x000F000Fu, c37 = (y ^ 0x88888888u) & 0x00F000F0u;
        acc[0] = acc[0] + __builtin_fmaf(half_lo(c04), sa, oa);
        acc[1] = acc[1] + __builtin_fmaf(half_lo(c15), sa16, oa);
        acc[2] = acc[2] + __builtin_fmaf(half_lo(c26), sa, oa);
        acc[3] = acc[3] + __builtin_fmaf(half_lo(c37), sa16, oa);
        acc[4] = acc[4] + __builtin_fmaf(half_hi(c04), sb, ob);
        acc[5] = acc[5] + __builtin_fmaf(half_hi(c15), sb16, ob);
        acc[6] = acc[6] + __builtin_fmaf(half_hi(c26), sb, ob);
        acc[7] = acc[7] + __builtin_fmaf(half_hi(c37), sb16, ob);
    } else if constexpr (kDecodeF16 && BITS == 8) {
        const uint32_t x0 = w.x ^ 0x80808080u, x1 = w.y ^ 0x80808080u;
        const uint32_t c02 = x0 & 0x00FF00FFu, c13 = (x0 >> 8) & 0x00FF00FFu;
        const uint32_t c46 = x1 & 0x00FF00FFu, c57 = (x1 >> 8) & 0x00FF00FFu;
        acc[0] = acc[0] + __builtin_fmaf(half_lo(c02), sa, oa);
        acc[1] = acc[1] + __builtin_fmaf(half_lo(c13), sa, oa);
        acc[2] = acc[2] + __builtin_fmaf(half_hi(c02), sa, oa);
        acc[3] = acc[3] + __builtin_fmaf(half_hi(c13), sa, oa);
        acc[4] = acc[4] + __builtin_fmaf(half_lo(c46), sb, ob);
        acc[5] = acc[5] + __builtin_fmaf(half_lo(c57), sb, ob);
        acc[6] = acc[6] + __builtin_fmaf(half_hi(c46), sb, ob);
        acc[7] = acc[7] + __builtin_fmaf(half_hi(c57), sb, ob);
    } else if constexpr (BITS == 4) {
        const uint32_t x = w.x ^ 0x88888888u;
        const uint32_t lo = x & 0x0F0F0F0Fu;         // codes 0, 2, 4, 6
        const uint32_t hi = (x >> 4) & 0x0F0F0F0Fu;  // codes 1, 3, 5, 7
        acc_byte<0>(acc[0], lo, sa, oa);
        acc_byte<0>(acc[1], hi, sa, oa);
        acc_byte<1>(acc[2], lo, sa, oa);
        acc_byte<1>(acc[3], hi, sa, oa);
        acc_byte<2>(acc[4], lo, sb, ob);
        acc_byte<2>(acc[5], hi, sb, ob);
        acc_byte<3>(acc[6], lo, sb, ob);
        acc_byte<3>(acc[7], hi, sb, ob);
    } else {
        const uint32_t x0 = w.x ^ 0x80808080u, x1 = w.y ^ 0x80808080u;
        acc_byte<0>(acc[0], x0, sa, oa);
        acc_byte<1>(acc[1], x0, sa, oa);
        acc_byte<2>(acc[2], x0, sa, oa);
        acc_byte<3>(acc[3], x0, sa, oa);
        acc_byte<0>(acc[4], x1, sb, ob);
        acc_byte<1>(acc[5], x1, sb, ob);
        acc_byte<2>(acc[6], x1, sb, ob);
        acc_byte<3>(acc[7], x1, sb, ob);
    }
}

// Lane layout of a 512-element sub-tile: lane l owns 8 outputs as two pieces of 4
// consecutive elements.  Split (fp32 output, and the fused Adam step with its fp32
// weights and moments): the pieces sit at 4l and 256 + 4l, so every load and store
// instruction of a 4-byte stream covers one contiguous 1 KB run.  Contiguous (bf16
// output): the lane's 8 outputs are consecutive (a 16-byte store each, already
// contiguous across the wave).  In the Adam step's traffic twin the split layout with
// non-temporal state loads and stores streams at 6.0 TB/s, against 5.4 for consecutive
// elements with plain ones.
template <int MODE>
struct DrLayout {
    static constexpr bool kSplit = MODE != kDrOutBf16;
    static __device__ __forceinline__ int piece(int l, int pc) { return kSplit ? pc * 256 + l * 4 : l * 8 + pc * 4; }
};

template <int BITS, int B, bool FIXED>
__device__ __forceinline__ float peer_step(const DrPeerDev& pe, int64_t i0, float fixed_step) {
    constexpr int QMAX = (1 << (BITS - 1)) - 1;
    if constexpr (FIXED) return fixed_step;
    else return pe.absmax[i0 / B] / (float)QMAX;  // 0 for an all-zero block
}

// The lane's 8 outputs of a sub-tile, pieces at elements i0 and i1 (i1 = i0 + 4 in the
// contiguous layout).
template <int MODE>
__device__ __forceinline__ void store_out8(void* out, int64_t i0, int64_t i1, const float (&acc)[kDrVec], float scale) {
    if constexpr (MODE == kDrOutBf16) {
        u32x4 s;
        s.x = bf16x2_rne(acc[0] * scale, acc[1] * scale);
        s.y = bf16x2_rne(acc[2] * scale, acc[3] * scale);
        s.z = bf16x2_rne(acc[4] * scale, acc[5] * scale);
        s.w = bf16x2_rne(acc[6] * scale, acc[7] * scale);
        __builtin_nontemporal_store(s, (u32x4*)((uint16_t*)out + i0));
    } else {
        f32x4 a = {acc[0] * scale, acc[1] * scale, acc[2] * scale, acc[3] * scale};
        f32x4 b = {acc[4] * scale, acc[5] * scale, acc[6] * scale, acc[7] * scale};
        __builtin_nontemporal_store(a, (f32x4*)((float*)out + i0));
        __builtin_nontemporal_store(b, (f32x4*)((float*)out + i1));
    }
}

// The Adam-family step on one element (Eqn. (9)), in the oracle's order of roundings.
__device__ __forceinline__ void adam1(const DrParams& p, float g, float& th, float& m, float& v) {
    m = p.omb1 * m + p.beta1 * g;
    v = p.omb2 * v + p.beta2 * (g * g);
    const float u = 1.0f / sqrtf(v + p.delta);
    th = th - p.lr * (m * u);
}

// 4 consecutive fp32 of the optimizer state, non-temporal (read once, written once).
__device__ __forceinline__ void load4f(const float* src, int64_t i0, float* x) {
    const f32x4 a = __builtin_nontemporal_load((const f32x4*)(src + i0));
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
}

__device__ __forceinline__ void store4f(float* dst, int64_t i0, const float* x) {
    __builtin_nontemporal_store(f32x4{x[0], x[1], x[2], x[3]}, (f32x4*)(dst + i0));
}

// The fused Adam step holds the optimizer state of its sub-tile in registers besides the
// payload codes: 87 VGPRs, 5 waves per SIMD (capped at 6 it spills).
#ifndef LOCO_DRA_WAVES_PER_EU
#define LOCO_DRA_WAVES_PER_EU 5
#endif
constexpr int dr_waves_per_eu(int mode) { return mode == kDrOutAdam ? LOCO_DRA_WAVES_PER_EU : 1; }

template <int BITS, int B, bool FIXED, int MODE>
__global__ __launch_bounds__(dr_threads(MODE)) __attribute__((amdgpu_waves_per_eu(dr_waves_per_eu(MODE))))
void dr_kernel(DrParams p, int64_t tbase) {
    using LY = DrLayout<MODE>;
    constexpr bool SPLIT = LY::kSplit;
    constexpr int U = dr_unroll(MODE);
    constexpr int TILE = dr_tile_elems(MODE);
    constexpr bool ADAM = MODE == kDrOutAdam;
    static_assert(TILE % B == 0, "a wave tile spans whole scale blocks");
    constexpr int SUB = 64 * kDrVec;
    const int lane = lane_id();
    const int64_t wg = xcd_remap<kXcds, dr_xcd_run(MODE)>(blockIdx.x, gridDim.x);
    // element offsets, within the tile, of the lane's pieces in each sub-tile
    int pos[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int pc = 0; pc < 2; ++pc) pos[u][pc] = u * SUB + LY::piece(lane, pc);
    const int64_t t = tbase + wg * (dr_threads(MODE) / kWave) + uniform(threadIdx.x / kWave);
    if (t >= p.ntiles) return;
    {
        const int64_t tb = t * TILE;  // the tile's first element
        float acc[U][kDrVec];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < kDrVec; ++j) acc[u][j] = 0.0f;

        bool whole = tb + TILE <= p.n;  // false: the element-wise path below takes the tile
        if (whole) {
            // The optimizer state is loaded first, so its latency overlaps the payloads'.
            float th[ADAM ? U : 1][kDrVec], mo[ADAM ? U : 1][kDrVec], ve[ADAM ? U : 1][kDrVec];
            if constexpr (ADAM) {
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int pc = 0; pc < 2; ++pc) {
                        load4f(p.theta, tb + pos[u][pc], th[u] + 4 * pc);
                        load4f(p.m, tb + pos[u][pc], mo[u] + 4 * pc);
                        load4f(p.v, tb + pos[u][pc], ve[u] + 4 * pc);
                    }
            }
            // whole wave tile in range.  The tile spans BPT scale blocks; the steps of G
            // peers x BPT blocks are computed one per lane (lane l divides peer l / BPT's
            // block l % BPT: one division per lane per G peers) and each lane fetches its
            // pieces' steps with ds_bpermute.  Every payload load goes through a buffer
            // resource over the peer's part of the tile (its base in SGPRs, a 32-bit lane
            // offset).
            constexpr int BPT = TILE / B;
            constexpr int G = 64 / BPT;
            // the two pieces of a lane lie in different blocks (split layout, blocks of at
            // most 256 elements)
            constexpr bool TWO = SPLIT && B <= SUB / 2;
            const int64_t blk0 = t * (TILE / B);
            const int64_t cbase = t * (int64_t)(TILE * BITS / 8);
            const uint32_t aoff = (uint32_t)(lane % BPT) * 4u;
            const int myq = lane / BPT;
            for (int pg = 0; pg < p.npeers; pg += G) {
                const int ng = p.npeers - pg < G ? p.npeers - pg : G;
                // codes of a batch of peers, all loads in flight together (slots past the
                // group read later peers or the table's copies of the last one, and are
                // not accumulated).  Split: a piece's 4 codes per load, merged so that
                // codes 0-3 are piece 0's and 4-7 piece 1's.
                u32x2 w[kDrPeerBatch][U];
                auto load_batch = [&](int q0) {
#pragma unroll
                    for (int b = 0; b < kDrPeerBatch; ++b) {
                        const auto ct = buffer_rsrc(p.peer[pg + q0 + b].codes + cbase, TILE * BITS / 8);
#pragma unroll
                        for (int u = 0; u < U; ++u) {
                            if constexpr (SPLIT) {
                                const u32x2 c0 = load_codes_at<BITS, 4>(ct, (uint32_t)pos[u][0] * BITS / 8);
                                const u32x2 c1 = load_codes_at<BITS, 4>(ct, (uint32_t)pos[u][1] * BITS / 8);
                                if constexpr (BITS == 8) w[b][u] = u32x2{c0.x, c1.x};
                                else w[b][u] = u32x2{c0.x | (c1.x << (4 * BITS)), 0u};
                            } else {
                                w[b][u] = load_codes_at<BITS, 8>(ct, (uint32_t)pos[u][0] * BITS / 8);
                            }
                        }
                    }
                };
                load_batch(0);  // issued before the scales, so both latencies overlap
                float stp = p.fixed_step;
                if constexpr (!FIXED) {
                    constexpr int QMAX = (1 << (BITS - 1)) - 1;
                    // every lane loads its block's absmax of each peer of a batch and keeps
                    // the one of its own peer
                    float am = 0.0f;
                    for (int q0 = 0; q0 < ng; q0 += kDrPeerBatch) {
                        float a[kDrPeerBatch];
#pragma unroll
                        for (int b = 0; b < kDrPeerBatch; ++b)
                            a[b] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                buffer_rsrc(p.peer[pg + q0 + b].absmax + blk0, BPT * 4), aoff, 0, 0));
#pragma unroll
                        for (int b = 0; b < kDrPeerBatch; ++b) am = (myq == q0 + b) ? a[b] : am;
                    }
                    stp = am / (float)QMAX;  // 0 for an all-zero block
                }
                // Every lane now holds one peer's step of one block (the fixed step is the
                // same in all).  The fma forms of the decoder need |step| < 2^100 (their
                // -2^(b-1)*step and step*2^24 must not overflow): a tile with a larger,
                // infinite or NaN step is redone from the start by the element-wise path
                // below, which forms q * step.
                if constexpr (BITS != 2) {
                    if (__builtin_amdgcn_ballot_w64(!(fabsf(stp) < 0x1p100f)) != 0) {
                        whole = false;
                        break;
                    }
                }
                // the decoder's scales (4 bits: also step * 2^20, for upper nibbles) and its
                // offset -2^(b-1)*step, all exact, once per scale
                const float scl = (BITS != 2 && kDecodeF16) ? stp * kF16SubScale : stp;
                constexpr bool S16 = BITS == 4 && kDecodeF16;
                const float scl16 = S16 ? stp * (kF16SubScale / 16.0f) : scl;
                const float offp = -(float)(1 << (BITS - 1)) * stp;
                for (int q0 = 0; q0 < ng; q0 += kDrPeerBatch) {
                    if (q0 > 0) load_batch(q0);
                    // byte address (ds_bpermute) of the lane holding peer q0's scale of a
                    // piece's block in sub-tile u; peer q0 + b is b*BPT lanes further, an
                    // immediate offset
                    int src[U][2];
#pragma unroll
                    for (int u = 0; u < U; ++u)
#pragma unroll
                        for (int pc = 0; pc < 2; ++pc) src[u][pc] = (q0 * BPT + pos[u][pc] / B) * 4;
                    // accumulate in peer order
#pragma unroll
                    for (int b = 0; b < kDrPeerBatch; ++b) {
                        if (q0 + b < ng) {
#pragma unroll
                            for (int u = 0; u < U; ++u) {
                                float sa = scl, oa = offp, sb = scl, ob = offp, sa16 = scl16, sb16 = scl16;
                                if constexpr (!FIXED) {
                                    auto fetch = [](int addr, float x) {
                                        return __builtin_bit_cast(
                                            float, __builtin_amdgcn_ds_bpermute(addr, __builtin_bit_cast(int, x)));
                                    };
                                    const int a0 = src[u][0] + b * BPT * 4;
                                    sa = fetch(a0, scl);
                                    if constexpr (BITS != 2) oa = fetch(a0, offp);
                                    if constexpr (S16) sa16 = fetch(a0, scl16);
                                    sb = sa;
                                    ob = oa;
                                    sb16 = sa16;
                                    if constexpr (TWO) {
                                        const int a1 = src[u][1] + b * BPT * 4;
                                        sb = fetch(a1, scl);
                                        if constexpr (BITS != 2) ob = fetch(a1, offp);
                                        if constexpr (S16) sb16 = fetch(a1, scl16);
                                    }
                                }
                                accumulate8<BITS>(acc[u], w[b][u], sa, oa, sb, ob, sa16, sb16);
                            }
                        }
                    }
                }
            }
            if (!whole) {
                // redone element-wise below
            } else if constexpr (ADAM) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
#pragma unroll
                    for (int j = 0; j < kDrVec; ++j) adam1(p, acc[u][j] * p.out_scale, th[u][j], mo[u][j], ve[u][j]);
#pragma unroll
                    for (int pc = 0; pc < 2; ++pc) {
                        const int64_t i0 = tb + pos[u][pc];
                        store4f(p.theta, i0, th[u] + 4 * pc);
                        store4f(p.m, i0, mo[u] + 4 * pc);
                        store4f(p.v, i0, ve[u] + 4 * pc);
                        if (p.theta_bf16) {
                            const u32x2 s = {bf16x2_rne(th[u][4 * pc], th[u][4 * pc + 1]),
                                             bf16x2_rne(th[u][4 * pc + 2], th[u][4 * pc + 3])};
                            __builtin_nontemporal_store(s, (u32x2*)(p.theta_bf16 + i0));
                        }
                    }
                }
            } else {
#pragma unroll
                for (int u = 0; u < U; ++u) store_out8<MODE>(p.out, tb + pos[u][0], tb + pos[u][1], acc[u], p.out_scale);
            }
        }
        if (!whole) {
            // the ragged tail, or a tile with a step of at least 2^100 or not finite:
            // element-wise, reading only the bytes that exist, d = q * step.  Its element
            // offsets derive from a lane index the compiler cannot see through, so they are
            // formed here rather than hoisted out of the tile loop (where they would stay
            // live, or be spilled, on every tile).
            int lane_e = lane;
            asm volatile("" : "+v"(lane_e));
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int j = 0; j < kDrVec; ++j) acc[u][j] = 0.0f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int pc = 0; pc < 2; ++pc) {
                    const int64_t i0 = tb + (u * SUB + LY::piece(lane_e, pc));
                    const int64_t left = p.n - i0;
                    const int nvalid = left <= 0 ? 0 : (left >= 4 ? 4 : (int)left);
                    if (nvalid == 0) continue;
                    float* ac = acc[u] + 4 * pc;
                    for (int pi = 0; pi < p.npeers; ++pi) {
                        const DrPeerDev pe = p.peer[pi];
                        const float step = peer_step<BITS, B, FIXED>(pe, i0, p.fixed_step);
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            if (j < nvalid) {
                                const int64_t i = i0 + j;
                                const uint32_t byte = pe.codes[(i * BITS) / 8];
                                const int q = __builtin_amdgcn_sbfe(byte, (int)((i * BITS) % 8), BITS);
                                ac[j] = ac[j] + (float)q * step;
                            }
                        }
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if (j < nvalid) {
                            const int64_t i = i0 + j;
                            const float g = ac[j] * p.out_scale;
                            if constexpr (ADAM) {
                                float th1 = p.theta[i], m1 = p.m[i], v1 = p.v[i];
                                adam1(p, g, th1, m1, v1);
                                p.theta[i] = th1;
                                p.m[i] = m1;
                                p.v[i] = v1;
                                if (p.theta_bf16) p.theta_bf16[i] = bf16_rne(th1);
                            } else if constexpr (MODE == kDrOutBf16) {
                                ((uint16_t*)p.out)[i] = bf16_rne(g);
                            } else {
                                ((float*)p.out)[i] = g;
                            }
                        }
                    }
                }
            }
        }
    }
}

template <int BITS, bool FIXED, int MODE>
const void* pick_block(int block) {
    if constexpr (FIXED) {
        return (const void*)&dr_kernel<BITS, 64, true, MODE>;
    } else {
        switch (block) {
            case 64: return (const void*)&dr_kernel<BITS, 64, false, MODE>;
            case 128: return (const void*)&dr_kernel<BITS, 128, false, MODE>;
            case 256: return (const void*)&dr_kernel<BITS, 256, false, MODE>;
            case 512: return (const void*)&dr_kernel<BITS, 512, false, MODE>;
        }
        return nullptr;
    }
}

template <bool FIXED, int MODE>
const void* pick_bits(int bits, int block) {
    switch (bits) {
        case 2: return pick_block<2, FIXED, MODE>(block);
        case 4: return pick_block<4, FIXED, MODE>(block);
        case 8: return pick_block<8, FIXED, MODE>(block);
    }
    return nullptr;
}

template <int MODE>
const void* pick_fixed(bool fixed, int bits, int block) {
    return fixed ? pick_bits<true, MODE>(bits, block) : pick_bits<false, MODE>(bits, block);
}

}  // namespace

hipError_t launch_dr(const DrParams& p, int bits, int block, bool fixed, int mode, hipStream_t stream) {
    const void* k = nullptr;
    switch (mode) {
        case kDrOutF32: k = pick_fixed<kDrOutF32>(fixed, bits, block); break;
        case kDrOutBf16: k = pick_fixed<kDrOutBf16>(fixed, bits, block); break;
        case kDrOutAdam: k = pick_fixed<kDrOutAdam>(fixed, bits, block); break;
    }
    if (!k) return hipErrorInvalidValue;
    // one wave per tile; launches of at most kMaxGrid workgroups
    const int threads = dr_threads(mode);
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
