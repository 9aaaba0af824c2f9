// SparseLoCo-style step: per-chunk Top-k by |h|, low-bit codes of the kept values,
// error feedback ("Communication Efficient LLM Pre-training with SparseLoCo": Top-k
// sparsification, 2-bit quantisation, error feedback).
//
// One wavefront (one 64-thread workgroup) owns one chunk of C = 64*VPT elements held
// in registers, element j*64 + lane in slot j, so every global access is a 256-byte
// coalesced row and ballot order within a slot is index order.
//
// Exact selection of the k-th largest key T = bits(|h|) (ties to the lower index):
//  1. each lane keeps its two largest keys; the k-th largest of those 128 keys, L, is
//     a lower bound of T (k of the chunk's keys are >= L);
//  2. the chunk's keys >= L (about k + a few) are compacted, in index order, into LDS;
//  3. T is found among them bit by bit (31 ballot/popcount rounds over a few slots),
//     with the count of keys > T and the index of the last tie that is kept.
// If k > 128 or more than kTkCap keys are >= L (adversarial layouts), step 3 runs over
// all registers instead.  Either way the result is the same exact set.
// The kept elements are then compacted in index order (ballot + mbcnt), their codes
// staged in LDS and packed, and the new error is written for every element.

#include "loco_device.hpp"
#include "loco_internal.hpp"

namespace loco {
namespace {

__device__ __forceinline__ uint32_t key_of(float h) { return __float_as_uint(h) & 0x7FFFFFFFu; }

template <int VPT, int BITS>
__device__ __forceinline__ void tk_chunk(const TkParams& p, int64_t chunk, uint32_t* s_key,
                                         uint16_t* s_idx, uint8_t* s_code) {
    static_assert(VPT <= 64, "one sign bit per slot in a 64-bit mask");
    constexpr int C = 64 * VPT;
    constexpr int QMAX = (1 << (BITS - 1)) - 1;
    constexpr int NSLOT = kTkCap / 64;
    const int lane = threadIdx.x;
    const int64_t base = chunk * C;
    const int64_t rem = p.n - base;
    const int len = rem < C ? (int)rem : C;
    const int keff = p.k < len ? p.k : len;
    const bool full = (len == C);

    // h = g + decay * e, kept as its key bits(|h|) plus one sign bit per slot.  Elements
    // past the end of a short chunk get key 0: every threshold tried below is >= 1, and
    // among equal keys the lower index wins, so they are never selected ahead of a real
    // element (keff <= len).
    uint32_t kv[VPT];
    uint64_t sgn = 0;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int64_t i = base + j * 64 + lane;
        float h = 0.0f;
        if (full) h = __builtin_nontemporal_load(p.g + i) + p.decay * p.e[i];
        else if (j * 64 + lane < len) h = p.g[i] + p.decay * p.e[i];
        const uint32_t u = __float_as_uint(h);
        kv[j] = u & 0x7FFFFFFFu;
        sgn |= (uint64_t)(u >> 31) << j;
    }

    // per-lane two largest keys, chunk max
    uint32_t m1 = 0, m2 = 0;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const uint32_t lo = min(m1, kv[j]);
        m1 = max(m1, kv[j]);
        m2 = max(m2, lo);
    }
    const uint32_t M = (uint32_t)uniform((int)wave_max_u32(m1));

    uint32_t T = 0;
    int need = 0, ilast = -1;
    bool done = false;

    if (keff <= 128) {
        // 1. lower bound L from the per-lane top-2 keys
        uint32_t L = 0;
        for (int bit = 30; bit >= 0; --bit) {
            const uint32_t cand = L | (1u << bit);
            const int c = __popcll(ballot(m1 >= cand)) + __popcll(ballot(m2 >= cand));
            if (c >= keff) L = cand;
        }
        // 2. compact the keys >= L in index order
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const bool c = kv[j] >= L;
            const uint64_t b = ballot(c);
            if (c) {
                const int pos = cnt + mbcnt(b);
                if (pos < kTkCap) {
                    s_key[pos] = kv[j];
                    s_idx[pos] = (uint16_t)(j * 64 + lane);
                }
            }
            cnt += __popcll(b);
        }
        if (cnt <= kTkCap) {
            __syncthreads();
            const int nslots = (cnt + 63) / 64;
            uint32_t cv[NSLOT];
#pragma unroll
            for (int s = 0; s < NSLOT; ++s) {
                const int pos = s * 64 + lane;
                cv[s] = pos < cnt ? s_key[pos] : 0u;
            }
            // 3. T = keff-th largest candidate (padding 0 never reaches a threshold >= 1)
            for (int bit = 30; bit >= 0; --bit) {
                const uint32_t cand = T | (1u << bit);
                int c = 0;
#pragma unroll
                for (int s = 0; s < NSLOT; ++s)
                    if (s < nslots) c += __popcll(ballot(cv[s] >= cand));
                if (c >= keff) T = cand;
            }
            int gt = 0;
#pragma unroll
            for (int s = 0; s < NSLOT; ++s)
                if (s < nslots) gt += __popcll(ballot(cv[s] > T));
            need = keff - gt;
            int seen = 0;
#pragma unroll
            for (int s = 0; s < NSLOT; ++s) {
                if (s < nslots && ilast < 0) {
                    const uint64_t b = ballot(s * 64 + lane < cnt && cv[s] == T);
                    const int pc = __popcll(b);
                    if (seen + pc >= need) ilast = uniform((int)s_idx[s * 64 + nth_set_bit(b, need - seen)]);
                    seen += pc;
                }
            }
            done = true;
        }
    }

    if (!done) {
        // exact search over every key of the chunk
        for (int bit = 30; bit >= 0; --bit) {
            const uint32_t cand = T | (1u << bit);
            int c = 0;
#pragma unroll
            for (int j = 0; j < VPT; ++j) c += __popcll(ballot(kv[j] >= cand));
            if (c >= keff) T = cand;
        }
        int gt = 0;
#pragma unroll
        for (int j = 0; j < VPT; ++j) gt += __popcll(ballot(kv[j] > T));
        need = keff - gt;
        int seen = 0;
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            if (ilast < 0) {
                const uint64_t b = ballot(kv[j] == T);
                const int pc = __popcll(b);
                if (seen + pc >= need) ilast = j * 64 + nth_set_bit(b, need - seen);
                seen += pc;
            }
        }
    }

    // quantise the kept values with the chunk's absmax; error feedback for all
    const float absmax = __uint_as_float(M);
    const float step = absmax / (float)QMAX;
    const float inv = (M != 0u) ? 1.0f / step : 0.0f;
    uint16_t* idx_out = p.idx + chunk * p.k;
    int cum = 0;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int i = j * 64 + lane;
        const float h = __uint_as_float(kv[j] | ((uint32_t)(sgn >> j) & 1u) << 31);
        // keys above T are real elements; ties are kept up to index ilast (< len)
        const bool sel = kv[j] > T || (kv[j] == T && i <= ilast);
        const float rq = __builtin_amdgcn_fmed3f(__builtin_rintf(h * inv), (float)(-QMAX - 1), (float)QMAX);
        const int q = (int)rq;
        const float d = (float)q * step;
        const float en = sel ? h - d : h;
        if (full || i < len) p.e[base + i] = en;
        const uint64_t b = ballot(sel);
        if (sel) {
            // pos < keff when the selection is right; the guard keeps a wrong selection
            // from writing outside this chunk's slots
            const int pos = cum + mbcnt(b);
            if (pos < keff) {
                idx_out[pos] = (uint16_t)i;
                s_code[pos] = (uint8_t)((uint32_t)q & ((1u << BITS) - 1u));
            }
        }
        cum += __popcll(b);
    }
    __syncthreads();
    for (int pos = keff + lane; pos < p.k; pos += 64) idx_out[pos] = 0xFFFF;
    constexpr int PER = 8 / BITS;
    const int nbytes = (p.k * BITS + 7) / 8;
    uint8_t* codes_out = p.codes + chunk * nbytes;
    for (int b = lane; b < nbytes; b += 64) {
        uint32_t v = 0;
#pragma unroll
        for (int t = 0; t < PER; ++t) {
            const int pos = b * PER + t;
            if (pos < keff) v |= (uint32_t)s_code[pos] << (BITS * t);
        }
        codes_out[b] = (uint8_t)v;
    }
    if (lane == 0) p.absmax[chunk] = absmax;
}

// Grid-strides over chunks; the barrier at the end of each chunk lets the next one
// reuse the LDS staging arrays.
template <int VPT, int BITS>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(LOCO_TK_WAVES_PER_EU)))
void tk_kernel(TkParams p, int64_t nchunks) {
    __shared__ uint32_t s_key[kTkCap];
    __shared__ uint16_t s_idx[kTkCap];
    __shared__ uint8_t s_code[64 * VPT];
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        tk_chunk<VPT, BITS>(p, c, s_key, s_idx, s_code);
        __syncthreads();
    }
}

template <int BITS>
const void* pick_chunk(int chunk) {
    switch (chunk) {
        case 256: return (const void*)&tk_kernel<4, BITS>;
        case 512: return (const void*)&tk_kernel<8, BITS>;
        case 1024: return (const void*)&tk_kernel<16, BITS>;
        case 2048: return (const void*)&tk_kernel<32, BITS>;
        case 4096: return (const void*)&tk_kernel<64, BITS>;
    }
    return nullptr;
}

}  // namespace

hipError_t launch_tk(const TkParams& p, int chunk, int bits, hipStream_t stream) {
    const void* k = nullptr;
    switch (bits) {
        case 2: k = pick_chunk<2>(chunk); break;
        case 4: k = pick_chunk<4>(chunk); break;
        case 8: k = pick_chunk<8>(chunk); break;
    }
    if (!k) return hipErrorInvalidValue;
    int64_t chunks = (p.n + chunk - 1) / chunk;
    const int64_t grid = chunks < kTkMaxGrid ? chunks : kTkMaxGrid;
    void* args[] = {(void*)&p, (void*)&chunks};
    return hipLaunchKernel(k, dim3((unsigned)grid), dim3(64), args, 0, stream);
}

}  // namespace loco
