// SparseLoCo's sparse aggregation: the peers' Top-k payloads of one shard, dequantized
// and summed into a dense output.
//
// "Communication Efficient LLM Pre-training with SparseLoCo" (summary and abstract) names
// a sparse aggregation of the nodes' sparse updates.  It is computed as LoCo's
// high-precision average ("LoCo: Low-Bit Communication Adaptor for Large-scale Model
// Training", Sec. 3.3, Eqn. (8)) over sparse vectors: for peers p = 0..N-1 in order and
// every used slot j of chunk c,
//   acc[c*C + idx_p[c][j]] += q_p[c][j] * step_p[c],   step = absmax / qmax
// and out = acc * out_scale; elements that no peer names are 0.
//
// Mapping: one workgroup of NT threads per chunk, the grid covering all chunks.  The
// chunk's fp32 accumulator lives in LDS (C floats, 16 KB at C = 4096) and is zeroed first.
// Thread t owns slots t, t+NT, ... of every peer.  The first slot of a batch of peers is
// loaded into registers in one go (all loads in flight together); then the peers are
// applied one at a time with a barrier between them, so every element adds its
// contributions in peer order.  Within one peer the slots name distinct elements, so
// their read-add-writes never collide.  The dense chunk is then written once, each
// thread storing whole runs of up to 8 outputs.

#include "loco_device.hpp"
#include "loco_internal.hpp"

namespace loco {
namespace {

// VEC consecutive outputs starting at element i0 of `out` (VEC in {1, 2, 4, 8}).
template <int VEC, bool OBF>
__device__ __forceinline__ void store_vec(void* out, int64_t i0, const float (&v)[VEC]) {
    if constexpr (OBF) {
        uint16_t* o = (uint16_t*)out + i0;
        if constexpr (VEC == 8) {
            u32x4 w = {bf16x2_rne(v[0], v[1]), bf16x2_rne(v[2], v[3]), bf16x2_rne(v[4], v[5]),
                       bf16x2_rne(v[6], v[7])};
            __builtin_nontemporal_store(w, (u32x4*)o);
        } else if constexpr (VEC == 4) {
            u32x2 w = {bf16x2_rne(v[0], v[1]), bf16x2_rne(v[2], v[3])};
            __builtin_nontemporal_store(w, (u32x2*)o);
        } else if constexpr (VEC == 2) {
            __builtin_nontemporal_store(bf16x2_rne(v[0], v[1]), (uint32_t*)o);
        } else {
            __builtin_nontemporal_store(bf16_rne(v[0]), o);
        }
    } else {
        float* o = (float*)out + i0;
        if constexpr (VEC >= 4) {
#pragma unroll
            for (int q = 0; q < VEC / 4; ++q) {
                f32x4 w = {v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
                __builtin_nontemporal_store(w, (f32x4*)o + q);
            }
        } else if constexpr (VEC == 2) {
            typedef float f32x2 __attribute__((ext_vector_type(2)));
            f32x2 w = {v[0], v[1]};
            __builtin_nontemporal_store(w, (f32x2*)o);
        } else {
            __builtin_nontemporal_store(v[0], o);
        }
    }
}

// acc[ix] += q * step for one slot whose code is bits [shift, shift+BITS) of `word`.
template <int BITS>
__device__ __forceinline__ void apply_slot(float* acc, uint32_t ix, uint32_t word, int shift, float step,
                                           int len) {
    if ((int)ix < len) {  // unused slots (0xFFFF) and indices past a short chunk are skipped
        const int q = __builtin_amdgcn_sbfe(word, shift, BITS);
        acc[ix] = acc[ix] + (float)q * step;
    }
}

template <int C, int BITS, bool OBF, int NT>
__global__ __launch_bounds__(NT) void sa_kernel(SaParams p, int64_t c0) {
    static_assert(C % NT == 0, "a chunk is a whole number of thread rows");
    constexpr int QMAX = (1 << (BITS - 1)) - 1;
    constexpr int VEC = C / NT >= 8 ? 8 : C / NT;
    constexpr int GROUPS = C / (NT * VEC);
    __shared__ __attribute__((aligned(16))) float acc[C];
    const int t = threadIdx.x;
    const int lane = lane_id();
    const int k = p.k;
    // one chunk per workgroup; the launch covers chunks [c0, c0 + gridDim.x)
    const int64_t c = c0 + xcd_remap<kXcds, kSaXcdRun>(blockIdx.x, gridDim.x);
    if (c >= p.nchunks) return;
    const int64_t base = c * C;
    const int len = (int)(p.n - base < C ? p.n - base : C);
    const int shift0 = (t * BITS) % 8;
    const int ts = t < k ? t : k - 1;  // threads past k re-read slot k-1 and drop it

    // Slot t of a batch of peers, loaded without branches so that every pointer and
    // load is issued back to back: per peer a uniform chunk pointer, and one lane offset
    // shared by all peers.  The batch's scales are uniform loads; lane b keeps peer b's
    // and divides it (one division per lane), and readlane returns the steps.
    uint32_t ix[kSaPeerBatch], cw[kSaPeerBatch];
    float am_mine = 0.0f;
    auto load_batch = [&](int p0) {
        SaPeerDev pe[kSaPeerBatch];
#pragma unroll
        for (int b = 0; b < kSaPeerBatch; ++b) pe[b] = p.peer[p0 + b < p.npeers ? p0 + b : p.npeers - 1];
        const uint32_t io = (uint32_t)ts, co = (uint32_t)(ts * BITS) / 8u;
        float am[kSaPeerBatch];
#pragma unroll
        for (int b = 0; b < kSaPeerBatch; ++b) {
            am[b] = pe[b].absmax[c];
            ix[b] = (pe[b].idx + c * k)[io];
            cw[b] = (pe[b].codes + c * p.cbytes)[co];
        }
#pragma unroll
        for (int b = 0; b < kSaPeerBatch; ++b) {
            am_mine = (lane == b) ? am[b] : am_mine;
            ix[b] = t < k ? ix[b] : 0xFFFFu;
        }
    };
    load_batch(0);  // before the LDS clear, so the clear overlaps the loads
#pragma unroll
    for (int i = t * 4; i < C; i += NT * 4) *(f32x4*)&acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    __syncthreads();

    for (int p0 = 0; p0 < p.npeers; p0 += kSaPeerBatch) {
        if (p0 > 0) load_batch(p0);
        const float step_mine = am_mine / (float)QMAX;  // 0 for an all-zero chunk
#pragma unroll
        for (int b = 0; b < kSaPeerBatch; ++b) {
            if (p0 + b < p.npeers) {  // uniform: the barrier below is reached by all threads
                const float step =
                    __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, step_mine), b));
                apply_slot<BITS>(acc, ix[b], cw[b], shift0, step, len);
                if (k > NT) {  // slots past the first row, loaded where used
                    const SaPeerDev pe = p.peer[p0 + b];
                    for (int j = t + NT; j < k; j += NT)
                        apply_slot<BITS>(acc, pe.idx[c * k + j], pe.codes[c * p.cbytes + (j * BITS) / 8],
                                         (j * BITS) % 8, step, len);
                }
                __syncthreads();
            }
        }
    }

    const float scale = p.out_scale;
    if (len == C) {
#pragma unroll
        for (int g = 0; g < GROUPS; ++g) {
            const int i0 = g * NT * VEC + t * VEC;
            float v[VEC];
#pragma unroll
            for (int j = 0; j < VEC; ++j) v[j] = acc[i0 + j] * scale;
            store_vec<VEC, OBF>(p.out, base + i0, v);
        }
    } else {
        for (int i = t; i < len; i += NT) {
            float v[1] = {acc[i] * scale};
            store_vec<1, OBF>(p.out, base + i, v);
        }
    }
}

// Threads per chunk: measured on MI355X for 8 peers of 2^28 in chunks of 4096, fp32 output
// runs best with 256 threads per chunk, bf16 output with 128 (0.12 against 0.19 ms).
template <int C, int BITS>
const void* pick_out(bool out_bf16) {
    return out_bf16 ? (const void*)&sa_kernel<C, BITS, true, kSaThreadsBf16>
                    : (const void*)&sa_kernel<C, BITS, false, kSaThreadsF32>;
}

template <int C>
const void* pick_bits(int bits, bool out_bf16) {
    switch (bits) {
        case 2: return pick_out<C, 2>(out_bf16);
        case 4: return pick_out<C, 4>(out_bf16);
        case 8: return pick_out<C, 8>(out_bf16);
    }
    return nullptr;
}

}  // namespace

hipError_t launch_sa(const SaParams& p, int chunk, int bits, bool out_bf16, hipStream_t stream) {
    const void* k = nullptr;
    switch (chunk) {
        case 256: k = pick_bits<256>(bits, out_bf16); break;
        case 512: k = pick_bits<512>(bits, out_bf16); break;
        case 1024: k = pick_bits<1024>(bits, out_bf16); break;
        case 2048: k = pick_bits<2048>(bits, out_bf16); break;
        case 4096: k = pick_bits<4096>(bits, out_bf16); break;
    }
    if (!k) return hipErrorInvalidValue;
    const int threads = out_bf16 ? kSaThreadsBf16 : kSaThreadsF32;
    // one workgroup per chunk, in launches of at most kMaxGrid workgroups
    for (int64_t c0 = 0; c0 < p.nchunks; c0 += kMaxGrid) {
        const int64_t blocks = p.nchunks - c0 < kMaxGrid ? p.nchunks - c0 : kMaxGrid;
        void* args[] = {(void*)&p, (void*)&c0};
        const hipError_t err = hipLaunchKernel(k, dim3((unsigned)blocks), dim3(threads), args, 0, stream);
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace loco
