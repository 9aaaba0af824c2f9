// SparseLoCo-style step: per-chunk Top-k by |h|, low-bit codes of the kept values,
// error feedback ("Communication Efficient LLM Pre-training with SparseLoCo": Top-k
// sparsification, 2-bit quantisation, error feedback).
//
// One 256-thread workgroup (4 waves) owns one chunk of C = 256*VPT elements; element
// i = 256*j + 64*w + lane sits in slot j of lane `lane` of wave w, so every global access
// is a 256-byte coalesced row per wave and (slot, wave, lane) order is index order.
// Each element is held as its key bits(|h|) plus one sign bit, VPT keys per lane.
//
// Exact selection of the k kept elements (largest keys, ties to the lower index):
//  1. a lower bound L of the k-th largest key: the largest value with 12 significant key
//     bits (exponent and 4 mantissa bits) that at least k per-thread maxima reach
//     (12 ballot rounds, wave 0); k keys of the chunk are then >= L;
//  2. the keys >= L (about k + a few dozen) are compacted in index order into LDS
//     (per-wave ballot counts, a cross-wave prefix over (slot, wave) pairs, then mbcnt);
//  3. wave 0 finds the threshold T (the k-th largest candidate key) by a bit search over
//     the candidates, only over the low bits where L and the chunk's largest key differ,
//     and the last kept tie (the candidates are in index order, so the kept ties are the
//     first ones equal to T); the kept candidates' threads quantise them and write their
//     error, index and code in index order;
//  4. every other element's error is h, written by a masked store.
// If k > 256 or more than kTkCap keys are >= L, all four waves search every key instead
// (cross-wave counts through LDS) and every element is selected and compacted in place;
// the result is the same exact set.

#include "loco_device.hpp"
#include "loco_internal.hpp"

namespace loco {
namespace {

constexpr int kTkThreads = 256;
constexpr int kTkWaves = kTkThreads / kWave;
// The lower bound L keeps key bits 30..kTkBoundLowBit (exponent + 4 mantissa bits).
constexpr int kTkBoundLowBit = 19;

struct TkShared {
    uint32_t top[kTkThreads];               // per-thread maximum key
    uint32_t key[kTkCap];                   // candidate keys, index order
    uint32_t hb[kTkCap];                    // candidate h bit patterns
    uint16_t idx[kTkCap];                   // candidate chunk-local indices
    int cnt[64];                            // per (slot, wave) counts, pair p = 4*slot + wave
    uint32_t wmax[kTkWaves];
    int red[kTkWaves];
    uint32_t L, T;
    int ilast;
    uint8_t code[4096];                     // kept codes, index order (k <= C <= 4096)
};

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int t = __shfl_up(v, d, 64);
        if (lane >= d) v += t;
    }
    return v;
}

// Exclusive prefix of sh.cnt[0..NP) held by lane p for pair p; `total` is the sum.
template <int NP>
__device__ __forceinline__ int pair_prefix(const TkShared& sh, int lane, int& total) {
    const int v = lane < NP ? sh.cnt[lane] : 0;
    const int incl = wave_incl_scan(v, lane);
    total = __builtin_amdgcn_readlane(incl, 63);
    return incl - v;
}

template <int BITS>
__device__ __forceinline__ int quantise(float h, float inv) {
    constexpr int QMAX = (1 << (BITS - 1)) - 1;
    return (int)__builtin_amdgcn_fmed3f(__builtin_rintf(h * inv), (float)(-QMAX - 1), (float)QMAX);
}

__device__ __forceinline__ float h_of(uint32_t key, uint32_t sgn, int j) {
    return __uint_as_float(key | ((sgn >> j) & 1u) << 31);
}

// FULL: the chunk has all C elements (every chunk but a short last one); the loads and
// stores of a full chunk are straight-line code, so all of them are in flight at once.
template <int VPT, int BITS, bool FULL>
__device__ __forceinline__ void tk_chunk(const TkParams& p, int64_t chunk, TkShared& sh) {
    static_assert(VPT <= 16, "C <= 4096");
    constexpr int C = kTkThreads * VPT;
    constexpr int NP = kTkWaves * VPT;
    constexpr int QMAX = (1 << (BITS - 1)) - 1;
    constexpr uint32_t CMASK = (1u << BITS) - 1u;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = uniform(tid >> 6);
    const int64_t base = chunk * C;
    const int64_t rem = p.n - base;
    const int len = FULL ? C : (rem < C ? (int)rem : C);
    const int keff = p.k < len ? p.k : len;
    uint16_t* idx_out = p.idx + chunk * p.k;

    // A. h = g + decay * e as key + sign; elements past the end of a short chunk get key 0,
    //    which no threshold tried below (>= 1) admits and which loses every tie to a real
    //    element of lower index (keff <= len).
    uint32_t kv[VPT];
    uint32_t sgn = 0;
    {
        float gv[VPT], ev[VPT];
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int i = j * kTkThreads + tid;
            if (FULL) {
                gv[j] = __builtin_nontemporal_load(p.g + base + i);
                ev[j] = p.e[base + i];
            } else {
                gv[j] = i < len ? p.g[base + i] : 0.0f;
                ev[j] = i < len ? p.e[base + i] : 0.0f;
            }
        }
        // decay 1 skips the multiply: 1 * e is e exactly, so h is the same either way
        const bool unit = p.decay == 1.0f;
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const uint32_t u = __float_as_uint(unit ? gv[j] + ev[j] : gv[j] + p.decay * ev[j]);
            kv[j] = u & 0x7FFFFFFFu;
            sgn |= (u >> 31) << j;
        }
    }
    uint32_t m1 = 0;
#pragma unroll
    for (int j = 0; j < VPT; ++j) m1 = max(m1, kv[j]);
    const uint32_t wm = wave_max_u32(m1);
    if (lane == 0) sh.wmax[w] = wm;
    sh.top[tid] = m1;
    __syncthreads();
    // the chunk's absmax is its largest key, always kept (keff >= 1)
    const uint32_t M = max(max(sh.wmax[0], sh.wmax[1]), max(sh.wmax[2], sh.wmax[3]));
    const float absmax = __uint_as_float(M);
    const float step = absmax / (float)QMAX;
    const float inv = (M != 0u) ? 1.0f / step : 0.0f;

    bool fast = false;
    if (keff <= kTkThreads) {
        // B. lower bound L (wave 0)
        if (w == 0) {
            const uint32_t t0 = sh.top[lane], t1 = sh.top[lane + 64], t2 = sh.top[lane + 128],
                           t3 = sh.top[lane + 192];
            uint32_t L = 0;
            for (int bit = 30; bit >= kTkBoundLowBit; --bit) {
                const uint32_t cand = L | (1u << bit);
                const int c = __popcll(ballot(t0 >= cand)) + __popcll(ballot(t1 >= cand)) +
                              __popcll(ballot(t2 >= cand)) + __popcll(ballot(t3 >= cand));
                if (c >= keff) L = cand;
            }
            if (lane == 0) sh.L = L;
        }
        __syncthreads();

        // C. compact the keys >= L in index order
        const uint32_t L = sh.L;
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int c = __popcll(ballot(kv[j] >= L));
            if (lane == 0) sh.cnt[j * kTkWaves + w] = c;
        }
        __syncthreads();
        int total = 0;
        const int excl = pair_prefix<NP>(sh, lane, total);
        if (total <= kTkCap) {
#pragma unroll
            for (int j = 0; j < VPT; ++j) {
                // read the pair's base in uniform control flow: a lane read inside the
                // divergent branch below could be an inactive one
                const int bj = __builtin_amdgcn_readlane(excl, j * kTkWaves + w);
                const uint64_t b = ballot(kv[j] >= L);  // taken again rather than kept: SGPRs are short
                if (kv[j] >= L) {
                    const int pos = bj + mbcnt(b);
                    sh.key[pos] = kv[j];
                    sh.hb[pos] = kv[j] | ((sgn >> j) & 1u) << 31;
                    sh.idx[pos] = (uint16_t)(j * kTkThreads + tid);
                }
            }
            fast = true;
        }
        __syncthreads();

        if (fast) {
            // D. wave 0 finds T, the keff-th largest candidate key, by a bit search over the
            //    candidates (8 per lane at most), then the last kept tie: candidates are in
            //    index order, so the kept ties are the first `need` candidates equal to T.
            if (w == 0) {
                constexpr int S = kTkCap / 64;
                const int ns = (total + 63) >> 6;
                uint32_t ck[S];
#pragma unroll
                for (int s = 0; s < S; ++s) ck[s] = (s * 64 + lane < total) ? sh.key[s * 64 + lane] : 0u;
                // T lies in [L, M], so it keeps the high bits L and M share; search the rest
                uint32_t T = L;
                const uint32_t diff = L ^ M;
                if (diff != 0u) {
                    const int top = 31 - __builtin_clz(diff);
                    T = L & ~((2u << top) - 1u);
                    for (int bit = top; bit >= 0; --bit) {
                        const uint32_t cand = T | (1u << bit);
                        int c = 0;
#pragma unroll
                        for (int s = 0; s < S; ++s)
                            if (s < ns) c += __popcll(ballot(ck[s] >= cand));
                        if (c >= keff) T = cand;
                    }
                }
                int need = keff;
#pragma unroll
                for (int s = 0; s < S; ++s)
                    if (s < ns) need -= __popcll(ballot(ck[s] > T));
                int ilast = 0;
                bool found = false;
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    if (s < ns && !found) {
                        const uint64_t b = ballot(ck[s] == T);
                        const int pc = __popcll(b);
                        if (need <= pc) {
                            ilast = sh.idx[s * 64 + nth_set_bit(b, need)];
                            found = true;
                        } else {
                            need -= pc;
                        }
                    }
                }
                if (lane == 0) {
                    sh.T = T;
                    sh.ilast = ilast;
                }
            }
            __syncthreads();
            const uint32_t T = sh.T;
            const int ilast = sh.ilast;
            uint64_t selb[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int t = s * kTkThreads + tid;
                bool kept = false;
                if (t < total) {
                    const uint32_t mk = sh.key[t];
                    kept = mk > T || (mk == T && (int)sh.idx[t] <= ilast);
                }
                selb[s] = ballot(kept);
                if (lane == 0) sh.cnt[s * kTkWaves + w] = __popcll(selb[s]);
            }
            __syncthreads();
            int nkept = 0;
            const int kex = pair_prefix<2 * kTkWaves>(sh, lane, nkept);
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int bs = __builtin_amdgcn_readlane(kex, s * kTkWaves + w);  // uniform control flow
                if ((selb[s] >> lane) & 1u) {
                    const int t = s * kTkThreads + tid;
                    const int pos = bs + mbcnt(selb[s]);
                    const float h = __uint_as_float(sh.hb[t]);
                    const int i = sh.idx[t];
                    const int q = quantise<BITS>(h, inv);
                    p.e[base + i] = h - (float)q * step;
                    if (pos < keff) {
                        idx_out[pos] = (uint16_t)i;
                        sh.code[pos] = (uint8_t)((uint32_t)q & CMASK);
                    }
                }
            }
            __syncthreads();
            // E. every element that is not kept keeps its whole h as error
#pragma unroll
            for (int j = 0; j < VPT; ++j) {
                const int i = j * kTkThreads + tid;
                const bool kept = kv[j] > T || (kv[j] == T && i <= ilast);
                if (!kept && (FULL || i < len)) p.e[base + i] = h_of(kv[j], sgn, j);
            }
        }
    }

    if (!fast) {
        // D'. exhaustive: all waves search every key; counts meet in LDS
        uint32_t T = 0;
        for (int bit = 30; bit >= 0; --bit) {
            const uint32_t cand = T | (1u << bit);
            int c = 0;
#pragma unroll
            for (int j = 0; j < VPT; ++j) c += __popcll(ballot(kv[j] >= cand));
            if (lane == 0) sh.red[w] = c;
            __syncthreads();
            c = sh.red[0] + sh.red[1] + sh.red[2] + sh.red[3];
            __syncthreads();
            if (c >= keff) T = cand;
        }
        int gt = 0;
#pragma unroll
        for (int j = 0; j < VPT; ++j) gt += __popcll(ballot(kv[j] > T));
        if (lane == 0) sh.red[w] = gt;
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int c = __popcll(ballot(kv[j] == T));
            if (lane == 0) sh.cnt[j * kTkWaves + w] = c;
        }
        __syncthreads();
        const int need = keff - (sh.red[0] + sh.red[1] + sh.red[2] + sh.red[3]);
        int ties = 0;
        const int excl = pair_prefix<NP>(sh, lane, ties);
        // the first (slot, wave) pair whose running tie count reaches `need` holds the last
        // kept tie
        const int mine = lane < NP ? sh.cnt[lane] : 0;
        const uint64_t reach = ballot(lane < NP && excl + mine >= need);
        const int pstar = reach ? __builtin_ctzll(reach) : 0;
        const int before = __builtin_amdgcn_readlane(excl, pstar);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const uint64_t b = ballot(kv[j] == T);  // uniform control flow
            if (j == pstar / kTkWaves && w == pstar % kTkWaves && lane == 0)
                sh.ilast = j * kTkThreads + w * 64 + nth_set_bit(b, need - before);
        }
        __syncthreads();
        const int ilast = sh.ilast;

        // E'. count the kept elements per (slot, wave), then write every element's error
        //     and compact the kept ones (their ballots are taken again, in uniform flow)
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const bool kept = kv[j] > T || (kv[j] == T && j * kTkThreads + tid <= ilast);
            const int c = __popcll(ballot(kept));
            if (lane == 0) sh.cnt[j * kTkWaves + w] = c;
        }
        __syncthreads();
        int nkept = 0;
        const int kex = pair_prefix<NP>(sh, lane, nkept);
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int i = j * kTkThreads + tid;
            const bool kept = kv[j] > T || (kv[j] == T && i <= ilast);
            const uint64_t b = ballot(kept);
            const int bj = __builtin_amdgcn_readlane(kex, j * kTkWaves + w);  // uniform control flow
            const float h = h_of(kv[j], sgn, j);
            if (kept) {
                // pos < keff when the selection is right; the guard keeps a wrong selection
                // from writing outside this chunk's slots
                const int pos = bj + mbcnt(b);
                const int q = quantise<BITS>(h, inv);
                p.e[base + i] = h - (float)q * step;
                if (pos < keff) {
                    idx_out[pos] = (uint16_t)i;
                    sh.code[pos] = (uint8_t)((uint32_t)q & CMASK);
                }
            } else if (FULL || i < len) {
                p.e[base + i] = h;
            }
        }
    }
    __syncthreads();

    // F. unused slots, packed codes, scale
    for (int pos = keff + tid; pos < p.k; pos += kTkThreads) idx_out[pos] = 0xFFFF;
    constexpr int PER = 8 / BITS;
    const int nbytes = (p.k * BITS + 7) / 8;
    uint8_t* codes_out = p.codes + chunk * nbytes;
    for (int b = tid; b < nbytes; b += kTkThreads) {
        uint32_t v = 0;
#pragma unroll
        for (int t = 0; t < PER; ++t) {
            const int pos = b * PER + t;
            if (pos < keff) v |= (uint32_t)sh.code[pos] << (BITS * t);
        }
        codes_out[b] = (uint8_t)v;
    }
    if (tid == 0) p.absmax[chunk] = absmax;
}

// Grid-strides over chunks [c0, c1); the barrier at the end of each chunk lets the next
// one reuse the LDS staging.  Full chunks and the short last chunk are separate kernels,
// so the full-chunk code carries no bounds masks (registers are allocated per kernel).
template <int VPT, int BITS, bool FULL>
__global__ __launch_bounds__(kTkThreads) __attribute__((amdgpu_waves_per_eu(LOCO_TK_WAVES_PER_EU)))
void tk_kernel(TkParams p, int64_t c0, int64_t c1) {
    __shared__ TkShared sh;
    for (int64_t c = c0 + blockIdx.x; c < c1; c += gridDim.x) {
        tk_chunk<VPT, BITS, FULL>(p, c, sh);
        __syncthreads();
    }
}

template <int BITS, bool FULL>
const void* pick_chunk(int chunk) {
    switch (chunk) {
        case 256: return (const void*)&tk_kernel<1, BITS, FULL>;
        case 512: return (const void*)&tk_kernel<2, BITS, FULL>;
        case 1024: return (const void*)&tk_kernel<4, BITS, FULL>;
        case 2048: return (const void*)&tk_kernel<8, BITS, FULL>;
        case 4096: return (const void*)&tk_kernel<16, BITS, FULL>;
    }
    return nullptr;
}

template <bool FULL>
const void* pick(int chunk, int bits) {
    switch (bits) {
        case 2: return pick_chunk<2, FULL>(chunk);
        case 4: return pick_chunk<4, FULL>(chunk);
        case 8: return pick_chunk<8, FULL>(chunk);
    }
    return nullptr;
}

}  // namespace

hipError_t launch_tk(const TkParams& p, int chunk, int bits, hipStream_t stream) {
    const void* kfull = pick<true>(chunk, bits);
    const void* ktail = pick<false>(chunk, bits);
    if (!kfull || !ktail) return hipErrorInvalidValue;
    int64_t nfull = p.n / chunk;
    int64_t nall = (p.n + chunk - 1) / chunk;
    if (nfull > 0) {
        int64_t c0 = 0;
        const int64_t grid = nfull < kTkMaxGrid ? nfull : kTkMaxGrid;
        void* args[] = {(void*)&p, (void*)&c0, (void*)&nfull};
        const hipError_t st = hipLaunchKernel(kfull, dim3((unsigned)grid), dim3(kTkThreads), args, 0, stream);
        if (st != hipSuccess) return st;
    }
    if (nall > nfull) {
        void* args[] = {(void*)&p, (void*)&nfull, (void*)&nall};
        return hipLaunchKernel(ktail, dim3(1), dim3(kTkThreads), args, 0, stream);
    }
    return hipSuccess;
}

}  // namespace loco
