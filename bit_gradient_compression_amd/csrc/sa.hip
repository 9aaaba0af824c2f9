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
// Mapping: one workgroup of NT threads per chunk at a time; a persistent grid of a few
// workgroups per compute unit walks the chunks, loading each chunk's payload while it
// processes the previous one.  The chunk's fp32 accumulator lives in LDS (C floats, 16 KB
// at C = 4096) and is zeroed first.
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

template <int C, int BITS, bool OBF, int NT, bool PERSIST>
__global__ __launch_bounds__(NT) void sa_kernel(SaParams p, int64_t c0, int64_t c1) {
    static_assert(C % NT == 0, "a chunk is a whole number of thread rows");
    constexpr int QMAX = (1 << (BITS - 1)) - 1;
    // outputs per thread per store: 16 bytes (4 fp32 or 8 bf16), so each store instruction
    // of a wave writes one contiguous 1 KB row
    constexpr int VMAX = OBF ? 8 : LOCO_SA_VEC_F32;
    constexpr int VEC = C / NT >= VMAX ? VMAX : C / NT;
    constexpr int GROUPS = C / (NT * VEC);
    __shared__ __attribute__((aligned(16))) float acc[C];
    const int t = threadIdx.x;
    const int lane = lane_id();
    const int k = p.k;
    const int shift0 = (t * BITS) % 8;
    const int ts = t < k ? t : k - 1;  // threads past k re-read slot k-1 and drop it

    // Slot t of a batch of peers for chunk c, loaded without branches so that every pointer
    // and load is issued back to back: per peer a uniform chunk pointer, and one lane offset
    // shared by all peers.  The batch's scales are uniform loads; lane b keeps peer b's and
    // divides it later (one division per lane), and readlane returns the steps.
    auto load_batch = [&](int64_t c, int p0, uint32_t (&ix)[kSaPeerBatch], uint32_t (&cw)[kSaPeerBatch],
                          float& am_mine) {
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
        am_mine = 0.0f;
#pragma unroll
        for (int b = 0; b < kSaPeerBatch; ++b) {
            am_mine = (lane == b) ? am[b] : am_mine;
            ix[b] = t < k ? ix[b] : 0xFFFFu;
        }
    };

    // workgroup w takes chunks c0 + w, c0 + w + gridDim.x, ... below c1; with a persistent
    // grid the next chunk's first batch is loaded while this one is processed
    int64_t c = c0 + xcd_remap<kXcds, kSaXcdRun>(blockIdx.x, gridDim.x);
    if (c >= c1) return;
    uint32_t ix[kSaPeerBatch], cw[kSaPeerBatch];
    float am_mine;
    load_batch(c, 0, ix, cw, am_mine);
    for (;;) {
        const int64_t cn = c + gridDim.x;
        const bool more = cn < c1;  // uniform
        uint32_t nix[kSaPeerBatch], ncw[kSaPeerBatch];
        float nam = 0.0f;
        if constexpr (PERSIST) {
            if (more && p.npeers <= kSaPeerBatch) load_batch(cn, 0, nix, ncw, nam);
        }
        const int64_t base = c * C;
        const int len = (int)(p.n - base < C ? p.n - base : C);
#pragma unroll
        for (int i = t * 4; i < C; i += NT * 4) *(f32x4*)&acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        __syncthreads();

        for (int p0 = 0; p0 < p.npeers; p0 += kSaPeerBatch) {
            if (p0 > 0) load_batch(c, p0, ix, cw, am_mine);
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
        if (!more) break;
        __syncthreads();  // the next chunk clears acc
        c = cn;
        if (PERSIST && p.npeers <= kSaPeerBatch) {
#pragma unroll
            for (int b = 0; b < kSaPeerBatch; ++b) {
                ix[b] = nix[b];
                cw[b] = ncw[b];
            }
            am_mine = nam;
        } else {
            load_batch(c, 0, ix, cw, am_mine);
        }
    }
}

// Launch shape per output type, measured on MI355X for 8 peers of 2^28 in chunks of 4096
// with the payloads out of the Infinity Cache: 128 threads per chunk and a persistent
// grid of 6 (fp32) or 8 (bf16) workgroups per compute unit: fp32 0.257 ms against 0.36 ms
// with one 256-thread workgroup per chunk; bf16 0.171 against 0.213 ms.
template <int C, int BITS>
const void* pick_out(bool out_bf16) {
    return out_bf16 ? (const void*)&sa_kernel<C, BITS, true, kSaThreadsBf16, (kSaWgPerCuBf16 > 0)>
                    : (const void*)&sa_kernel<C, BITS, false, kSaThreadsF32, (kSaWgPerCuF32 > 0)>;
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
    const int per_cu = out_bf16 ? kSaWgPerCuBf16 : kSaWgPerCuF32;
    int64_t grid = kMaxGrid;
    if (per_cu > 0) {
        int cus = 0;
        const hipError_t err = compute_units(cus);
        if (err != hipSuccess) return err;
        grid = (int64_t)cus * per_cu;
    }
    // chunks [c0, c1) per launch: one chunk per workgroup, or all of them for a persistent grid
    const int64_t span = per_cu > 0 ? p.nchunks : kMaxGrid;
    for (int64_t c0 = 0; c0 < p.nchunks; c0 += span) {
        int64_t c1 = p.nchunks - c0 < span ? p.nchunks : c0 + span;
        const int64_t blocks = c1 - c0 < grid ? c1 - c0 : grid;
        void* args[] = {(void*)&p, (void*)&c0, (void*)&c1};
        const hipError_t err = hipLaunchKernel(k, dim3((unsigned)blocks), dim3(threads), args, 0, stream);
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace loco
