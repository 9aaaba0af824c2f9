// Device helpers for the gfx950 kernels: vector types, bf16 conversion, wavefront
// reductions and ballots.  Every kernel of the library includes this file.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace loco {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---- bf16 ---------------------------------------------------------------------

// bf16 -> f32 is exact: the pattern becomes the high half of the f32 pattern.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// f32 pair -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
    __bf16 a = (__bf16)lo;
    __bf16 b = (__bf16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ uint16_t bf16_rne(float x) {
    __bf16 a = (__bf16)x;
    return __builtin_bit_cast(uint16_t, a);
}

// v_cvt_f32_ubyteN: byte N of x as a float, in one instruction (the compiler otherwise
// extracts the byte with a separate bit-field op first).
template <int N>
__device__ __forceinline__ float ubyte_to_f32(uint32_t x) {
    float r;
    if constexpr (N == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(r) : "v"(x));
    else if constexpr (N == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(r) : "v"(x));
    else if constexpr (N == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(r) : "v"(x));
    else asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(r) : "v"(x));
    return r;
}

// ---- block scales ----------------------------------------------------------------

// The quantiser's reciprocal inv = fl(1/step) (correctly rounded by build flag), or 0 where
// it is not finite: step = 0 (an all-zero block) or step below ~2^-128, where 1/step
// overflows fp32.  Such a block cannot be scaled into the code range; with inv = 0 every
// code is 0 and error feedback keeps the block's values whole.
__device__ __forceinline__ float finite_recip(float step) {
    const float r = 1.0f / step;
    return r < __builtin_huge_valf() ? r : 0.0f;
}

// ---- code packing -----------------------------------------------------------------

// Eight BITS-bit two's-complement codes q[j] (integer-valued floats in [-2^(BITS-1),
// 2^(BITS-1) - 1]) packed in element order: code j in bits [BITS*j, BITS*j + BITS) of the
// 8*BITS-bit result (lo: bits 0-31, hi: bits 32-63).  Each byte is formed as an exact float
// sum of the biased codes q + 2^(BITS-1) (in [0, 2^BITS)), put in its byte by
// v_cvt_pk_u8_f32, and one xor per word turns every biased field back into the code
// (within a BITS-bit field, q + 2^(BITS-1) == q ^ 2^(BITS-1) mod 2^BITS).
template <int BITS>
__device__ __forceinline__ void pack_codes8(const float (&q)[8], uint32_t& lo, uint32_t& hi) {
    lo = 0u;
    hi = 0u;
    if constexpr (BITS == 8) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            lo = __builtin_amdgcn_cvt_pk_u8_f32(q[j] + 128.0f, j, lo);
            hi = __builtin_amdgcn_cvt_pk_u8_f32(q[4 + j] + 128.0f, j, hi);
        }
        lo ^= 0x80808080u;
        hi ^= 0x80808080u;
    } else if constexpr (BITS == 4) {
        // byte b holds codes 2b (low nibble) and 2b+1: (q0 + 8) + 16 (q1 + 8)
#pragma unroll
        for (int b = 0; b < 4; ++b)
            lo = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(q[2 * b + 1], 16.0f, q[2 * b] + 136.0f), b, lo);
        lo ^= 0x88888888u;
    } else {
        static_assert(BITS == 2, "2, 4 or 8 bits");
        // byte b holds codes 4b..4b+3: sum of (q_i + 2) 4^i
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            float v = q[4 * b] + 170.0f;
            v = __builtin_fmaf(q[4 * b + 1], 4.0f, v);
            v = __builtin_fmaf(q[4 * b + 2], 16.0f, v);
            v = __builtin_fmaf(q[4 * b + 3], 64.0f, v);
            lo = __builtin_amdgcn_cvt_pk_u8_f32(v, b, lo);
        }
        lo ^= 0xAAAAu;
    }
}

// Low bytes of four words, in order: b0's low byte in bits 0-7 ... b3's in bits 24-31.
__device__ __forceinline__ uint32_t low_bytes4(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) {
    // v_perm_b32: selector byte values 0-3 pick bytes of the second operand, 4-7 of the
    // first, 0x0c gives zero
    const uint32_t t01 = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);
    const uint32_t t23 = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);
    return __builtin_amdgcn_perm(t23, t01, 0x05040100u);
}

// ---- buffer resources ------------------------------------------------------------

// A raw buffer resource over `bytes` bytes at p.  Loads through it take the base from
// SGPRs and a 32-bit lane offset (no per-lane 64-bit address arithmetic), and an offset
// past `bytes` reads 0 without touching memory.  Word 3 is gfx9's raw-buffer format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
constexpr int kLoadNt = 2;  // cache-policy bit of a non-temporal (streaming) load on gfx950

// ---- wavefront primitives -------------------------------------------------------

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Number of set bits of m in the lanes below this one.
__device__ __forceinline__ int mbcnt(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}

// Max of v over aligned groups of LANES consecutive lanes (LANES a power of two up
// to 64); every lane of the group gets the result.  All 64 lanes must be active.
// Unsigned compare: applied to the bit patterns of non-negative floats it is the
// float max, exactly.
template <int LANES>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
    if constexpr (LANES >= 2) v = max(v, dpp<0xB1>(v));    // quad_perm [1,0,3,2]
    if constexpr (LANES >= 4) v = max(v, dpp<0x4E>(v));    // quad_perm [2,3,0,1]
    if constexpr (LANES >= 8) v = max(v, dpp<0x141>(v));   // row_half_mirror
    if constexpr (LANES >= 16) v = max(v, dpp<0x140>(v));  // row_mirror
    if constexpr (LANES >= 32) {
        auto s = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        v = max((uint32_t)s[0], (uint32_t)s[1]);
    }
    if constexpr (LANES >= 64) {
        auto s = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        v = max((uint32_t)s[0], (uint32_t)s[1]);
    }
    return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) { return group_max_u32<64>(v); }

// Position of the r-th (1-based) set bit of m (r >= 1).  If m holds fewer than r set
// bits the result is still a lane number (0..63), never out of range.
__device__ __forceinline__ int nth_set_bit(uint64_t m, int r) {
    for (int t = 1; t < r; ++t) m &= m - 1;
    return m ? __builtin_ctzll(m) : 63;
}

// Logical workgroup number of physical workgroup b out of g: groups of RUN consecutive
// logical numbers share one XCD (dispatch is round-robin over NX XCDs).  Workgroups of an
// incomplete last group keep their own number.
template <int NX, int RUN>
__device__ __forceinline__ int64_t xcd_remap(int64_t b, int64_t g) {
    if constexpr (RUN <= 1) {
        return b;
    } else {
        constexpr int64_t SPAN = (int64_t)NX * RUN;
        if (b >= g - g % SPAN) return b;
        const int64_t x = b % NX, r = b / NX;
        return (r / RUN) * SPAN + x * RUN + (r % RUN);
    }
}

// Wave-uniform value as an SGPR.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

}  // namespace loco
