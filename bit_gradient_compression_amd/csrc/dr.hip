// Dequantize and average the peers' low-bit payloads of one partition.
//
// LoCo ("LoCo: Low-Bit Communication Adaptor for Large-scale Model Training"),
// Sec. 3.3, Eqn. (8): each node gathers the N low-bit partitions it owns (all2all) and
// averages their decompressed values in high precision:
//   acc = sum over p = 0..N-1 (in that order) of q_p * step_p;  out = acc * out_scale
//
// Mapping: lane l of a wavefront owns 32 consecutive outputs, so each peer's codes for
// the lane are one 16-byte load at 4 bits (8 bytes at 2 bits, 32 at 8 bits) and the
// 32 outputs sit in one scale block (blocks are >= 64 elements).  The fp32
// accumulator never leaves registers; only the reduced shard is written.  The grid is
// persistent and grid-strides over wave tiles of 2048 elements.

#include "loco_device.hpp"
#include "loco_internal.hpp"

namespace loco {
namespace {

template <int BITS>
__device__ __forceinline__ int field(const uint32_t (&w)[kDrVec * BITS / 32], int j) {
    constexpr int PER = 32 / BITS;  // codes per 32-bit word
    return __builtin_amdgcn_sbfe(w[j / PER], (j % PER) * BITS, BITS);
}

template <int BITS>
__device__ __forceinline__ void load_codes(const uint8_t* c, int64_t i0, uint32_t (&w)[kDrVec * BITS / 32]) {
    const uint8_t* p = c + (i0 * BITS) / 8;
    if constexpr (BITS == 2) {
        u32x2 v = __builtin_nontemporal_load((const u32x2*)p);
        w[0] = v.x; w[1] = v.y;
    } else if constexpr (BITS == 4) {
        u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else {
        u32x4 a = __builtin_nontemporal_load((const u32x4*)p);
        u32x4 b = __builtin_nontemporal_load((const u32x4*)p + 1);
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    }
}

template <int BITS, int B, bool FIXED>
__device__ __forceinline__ float peer_step(const DrPeerDev& pe, int64_t i0, float fixed_step) {
    constexpr int QMAX = (1 << (BITS - 1)) - 1;
    if constexpr (FIXED) return fixed_step;
    else return pe.absmax[i0 / B] / (float)QMAX;  // 0 for an all-zero block
}

template <int BITS, int B, bool FIXED, bool OBF>
__global__ __launch_bounds__(kDrThreads) void dr_kernel(DrParams p) {
    constexpr int NW = kDrVec * BITS / 32;
    const int lane = lane_id();
    const int64_t wave0 = (int64_t)blockIdx.x * (kDrThreads / kWave) + uniform(threadIdx.x / kWave);
    const int64_t nwaves = (int64_t)gridDim.x * (kDrThreads / kWave);
    for (int64_t t = wave0; t < p.ntiles; t += nwaves) {
        const int64_t i0 = t * kDrTile + lane * kDrVec;
        float acc[kDrVec];
#pragma unroll
        for (int j = 0; j < kDrVec; ++j) acc[j] = 0.0f;

        if ((t + 1) * kDrTile <= p.n) {
            // whole wave tile in range
#pragma unroll 2
            for (int pi = 0; pi < p.npeers; ++pi) {
                const DrPeerDev pe = p.peer[pi];
                uint32_t w[NW];
                load_codes<BITS>(pe.codes, i0, w);
                const float step = peer_step<BITS, B, FIXED>(pe, i0, p.fixed_step);
#pragma unroll
                for (int j = 0; j < kDrVec; ++j) acc[j] = acc[j] + (float)field<BITS>(w, j) * step;
            }
            if constexpr (OBF) {
                uint16_t* o = (uint16_t*)p.out + i0;
#pragma unroll
                for (int v = 0; v < kDrVec / 8; ++v) {
                    u32x4 s;
                    s.x = bf16x2_rne(acc[8 * v + 0] * p.out_scale, acc[8 * v + 1] * p.out_scale);
                    s.y = bf16x2_rne(acc[8 * v + 2] * p.out_scale, acc[8 * v + 3] * p.out_scale);
                    s.z = bf16x2_rne(acc[8 * v + 4] * p.out_scale, acc[8 * v + 5] * p.out_scale);
                    s.w = bf16x2_rne(acc[8 * v + 6] * p.out_scale, acc[8 * v + 7] * p.out_scale);
                    __builtin_nontemporal_store(s, (u32x4*)(o + 8 * v));
                }
            } else {
                float* o = (float*)p.out + i0;
#pragma unroll
                for (int v = 0; v < kDrVec / 4; ++v) {
                    f32x4 s = {acc[4 * v] * p.out_scale, acc[4 * v + 1] * p.out_scale,
                               acc[4 * v + 2] * p.out_scale, acc[4 * v + 3] * p.out_scale};
                    __builtin_nontemporal_store(s, (f32x4*)(o + 4 * v));
                }
            }
        } else {
            // ragged tail: element-wise, reading only the bytes that exist
            const int64_t left = p.n - i0;
            const int nvalid = left <= 0 ? 0 : (left >= kDrVec ? kDrVec : (int)left);
            if (nvalid == 0) continue;
            for (int pi = 0; pi < p.npeers; ++pi) {
                const DrPeerDev pe = p.peer[pi];
                const float step = peer_step<BITS, B, FIXED>(pe, i0, p.fixed_step);
#pragma unroll
                for (int j = 0; j < kDrVec; ++j) {
                    if (j < nvalid) {
                        const int64_t i = i0 + j;
                        const uint32_t byte = pe.codes[(i * BITS) / 8];
                        const int q = __builtin_amdgcn_sbfe(byte, (int)((i * BITS) % 8), BITS);
                        acc[j] = acc[j] + (float)q * step;
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < kDrVec; ++j) {
                if (j < nvalid) {
                    const float v = acc[j] * p.out_scale;
                    if constexpr (OBF) ((uint16_t*)p.out)[i0 + j] = bf16_rne(v);
                    else ((float*)p.out)[i0 + j] = v;
                }
            }
        }
    }
}

template <int BITS, bool FIXED, bool OBF>
const void* pick_block(int block) {
    if constexpr (FIXED) {
        return (const void*)&dr_kernel<BITS, 64, true, OBF>;
    } else {
        switch (block) {
            case 64: return (const void*)&dr_kernel<BITS, 64, false, OBF>;
            case 128: return (const void*)&dr_kernel<BITS, 128, false, OBF>;
            case 256: return (const void*)&dr_kernel<BITS, 256, false, OBF>;
            case 512: return (const void*)&dr_kernel<BITS, 512, false, OBF>;
        }
        return nullptr;
    }
}

template <bool FIXED, bool OBF>
const void* pick_bits(int bits, int block) {
    switch (bits) {
        case 2: return pick_block<2, FIXED, OBF>(block);
        case 4: return pick_block<4, FIXED, OBF>(block);
        case 8: return pick_block<8, FIXED, OBF>(block);
    }
    return nullptr;
}

}  // namespace

hipError_t launch_dr(const DrParams& p, int bits, int block, bool fixed, bool out_bf16,
                     int max_blocks, hipStream_t stream) {
    const void* k = nullptr;
    if (fixed) k = out_bf16 ? pick_bits<true, true>(bits, block) : pick_bits<true, false>(bits, block);
    else k = out_bf16 ? pick_bits<false, true>(bits, block) : pick_bits<false, false>(bits, block);
    if (!k) return hipErrorInvalidValue;
    const int64_t waves_per_block = kDrThreads / kWave;
    int64_t blocks = (p.ntiles + waves_per_block - 1) / waves_per_block;
    if (blocks > max_blocks) blocks = max_blocks;
    if (blocks < 1) blocks = 1;
    void* args[] = {(void*)&p};
    return hipLaunchKernel(k, dim3((unsigned)blocks), dim3(kDrThreads), args, 0, stream);
}

}  // namespace loco
