// SparseLoCo-style step: per-chunk Top-k by |h|, low-bit codes of the kept values,
// error feedback ("Communication Efficient LLM Pre-training with SparseLoCo": Top-k
// sparsification, 2-bit quantisation, error feedback).
//
// One 256-thread workgroup (4 waves) owns one chunk of C = 256*VPT elements; element
// i = 256*j + 64*w + lane sits in slot j of lane `lane` of wave w, so every global access
// is a 256-byte coalesced row per wave and (slot, wave, lane) order is index order.
// Each element is held as its key bits(|h|) plus one sign bit, VPT keys per lane.
//
// Exact selection of the k-th largest key T (ties to the lower index):
//  1. a lower bound L of T: the largest value with 12 significant key bits (exponent and
//     4 mantissa bits) that at least k per-thread maxima reach (12 ballot rounds, wave 0);
//     k keys of the chunk are then >= L;
//  2. the keys >= L (about k + a few dozen) are compacted in index order into LDS
//     (per-wave ballot counts, a cross-wave prefix over (slot, wave) pairs, then mbcnt);
//  3. every thread ranks its candidate against all candidates (16-byte broadcast LDS
//     reads); the candidate of rank k-1 gives T and the index of the last tie kept.
// If k > 256 or more than kTkCap keys are >= L, all four waves search every key instead
// (cross-wave counts through LDS); the result is the same exact set.
// The kept elements are then compacted in index order the same way, their codes staged
// in LDS and packed, and the new error is written for every element.

#include "loco_device.hpp"
#include "loco_internal.hpp"

namespace loco {
namespace {

constexpr int kTkThreads = 256;
constexpr int kTkWaves = kTkThreads / kWave;
// The lower bound L keeps key bits 30..kTkBoundLowBit (exponent + 4 mantissa bits).
constexpr int kTkBoundLowBit = 19;

struct TkShared {
    uint32_t top[kTkThreads];   // per-thread maximum key
    alignas(16) uint32_t key[kTkCap + 4];  // candidate keys, index order, zero-padded to a 16-byte row
    uint16_t idx[kTkCap];       // their chunk-local indices
    int cnt[64];                // per (slot, wave) counts, pair p = 4*slot + wave
    uint32_t wmax[kTkWaves];
    int red[kTkWaves];
    uint32_t L, T;
    int ilast;
    uint8_t code[4096];         // kept codes, index order (k <= C <= 4096)
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

// Exclusive prefix of sh.cnt over the 4*VPT (slot, wave) pairs, lane p holding pair p;
// `total` is the sum over all pairs.
template <int VPT>
__device__ __forceinline__ int pair_prefix(const TkShared& sh, int lane, int& total) {
    constexpr int NP = kTkWaves * VPT;
    const int v = lane < NP ? sh.cnt[lane] : 0;
    const int incl = wave_incl_scan(v, lane);
    total = __builtin_amdgcn_readlane(incl, 63);
    return incl - v;
}

// FULL: the chunk has all C elements (every chunk but a short last one); the loads and
// stores of a full chunk are straight-line code, so all of them are in flight at once.
template <int VPT, int BITS, bool FULL>
__device__ __forceinline__ void tk_chunk(const TkParams& p, int64_t chunk, TkShared& sh) {
    static_assert(VPT <= 16, "C <= 4096");
    constexpr int C = kTkThreads * VPT;
    constexpr int NP = kTkWaves * VPT;
    constexpr int QMAX = (1 << (BITS - 1)) - 1;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = uniform(tid >> 6);
    const int64_t base = chunk * C;
    const int64_t rem = p.n - base;
    const int len = FULL ? C : (rem < C ? (int)rem : C);
    const int keff = p.k < len ? p.k : len;

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
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const uint32_t u = __float_as_uint(gv[j] + p.decay * ev[j]);
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
    const uint32_t M = max(max(sh.wmax[0], sh.wmax[1]), max(sh.wmax[2], sh.wmax[3]));

    // B. lower bound L: the keff-th largest per-thread maximum (wave 0)
    const bool try_fast = keff <= kTkThreads;
    bool fast = false;
    if (try_fast) {
        if (w == 0) {
            const uint32_t t0 = sh.top[lane], t1 = sh.top[lane + 64], t2 = sh.top[lane + 128],
                           t3 = sh.top[lane + 192];
            // only a bound is needed: search the exponent and the top 4 mantissa bits
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
        uint64_t cb[VPT];
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            cb[j] = ballot(kv[j] >= L);
            if (lane == 0) sh.cnt[j * kTkWaves + w] = __popcll(cb[j]);
        }
        __syncthreads();
        int total = 0;
        const int excl = pair_prefix<VPT>(sh, lane, total);
        if (total <= kTkCap) {
#pragma unroll
            for (int j = 0; j < VPT; ++j) {
                // read the pair's base in uniform control flow: a lane read inside the
                // divergent branch below could be an inactive one
                const int bj = __builtin_amdgcn_readlane(excl, j * kTkWaves + w);
                if (kv[j] >= L) {
                    const int pos = bj + mbcnt(cb[j]);
                    sh.key[pos] = kv[j];
                    sh.idx[pos] = (uint16_t)(j * kTkThreads + tid);
                }
            }
            if (tid < 4 && total + tid < kTkCap + 4) sh.key[total + tid] = 0u;
            fast = true;
        }
        __syncthreads();

        // D (fast). Every thread ranks its own candidate(s) against all candidates in the
        // order (key descending, index ascending): rank = #{keys above} + #{equal keys at
        // lower positions}.  Ranks are a permutation of 0..total-1, so the candidate of
        // rank keff-1 is the last kept element: its key is T and, T being its key, its
        // index is the last kept tie.
        if (fast) {
            const int nrow = (total + 3) >> 2;
            for (int t = tid; t < total; t += kTkThreads) {
                const uint32_t mk = sh.key[t];
                int rank = 0;
                for (int r = 0; r < nrow; ++r) {
                    const u32x4 kr = *(const u32x4*)&sh.key[4 * r];
                    const int c = 4 * r;
                    rank += (kr.x > mk) + (kr.y > mk) + (kr.z > mk) + (kr.w > mk);
                    rank += (kr.x == mk && c < t) + (kr.y == mk && c + 1 < t) + (kr.z == mk && c + 2 < t) +
                            (kr.w == mk && c + 3 < t);
                }
                if (rank == keff - 1) {
                    sh.T = mk;
                    sh.ilast = sh.idx[t];
                }
            }
            __syncthreads();
        }
    }

    if (!fast) {
        // D (exhaustive). All waves search every key; counts meet in LDS.
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
        uint64_t tb[VPT];
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            tb[j] = ballot(kv[j] == T);
            if (lane == 0) sh.cnt[j * kTkWaves + w] = __popcll(tb[j]);
        }
        __syncthreads();
        const int need = keff - (sh.red[0] + sh.red[1] + sh.red[2] + sh.red[3]);
        int total = 0;
        const int excl = pair_prefix<VPT>(sh, lane, total);
        // the first (slot, wave) pair whose running tie count reaches `need` holds the last
        // kept tie
        const int mine = lane < NP ? sh.cnt[lane] : 0;
        const uint64_t reach = ballot(lane < NP && excl + mine >= need);
        const int pstar = reach ? __builtin_ctzll(reach) : 0;
        const int before = __builtin_amdgcn_readlane(excl, pstar);
        if (w == pstar % kTkWaves && lane == 0) {
#pragma unroll
            for (int j = 0; j < VPT; ++j) {
                if (j == pstar / kTkWaves) sh.ilast = j * kTkThreads + w * 64 + nth_set_bit(tb[j], need - before);
            }
        }
        if (tid == 0) sh.T = T;
        __syncthreads();
    }

    // E. quantise the kept values with the chunk's absmax; error feedback for all
    const uint32_t T = sh.T;
    const int ilast = sh.ilast;
    const float absmax = __uint_as_float(M);
    const float step = absmax / (float)QMAX;
    const float inv = (M != 0u) ? 1.0f / step : 0.0f;
    uint64_t sb[VPT];
    int qv[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int i = j * kTkThreads + tid;
        const float h = __uint_as_float(kv[j] | ((sgn >> j) & 1u) << 31);
        // keys above T are real elements; ties are kept up to index ilast (< len)
        const bool sel = kv[j] > T || (kv[j] == T && i <= ilast);
        const float rq = __builtin_amdgcn_fmed3f(__builtin_rintf(h * inv), (float)(-QMAX - 1), (float)QMAX);
        const int q = (int)rq;
        const float d = (float)q * step;
        const float en = sel ? h - d : h;
        if (FULL || i < len) p.e[base + i] = en;
        sb[j] = ballot(sel);
        qv[j] = q;
        if (lane == 0) sh.cnt[j * kTkWaves + w] = __popcll(sb[j]);
    }
    __syncthreads();
    int total = 0;
    const int excl = pair_prefix<VPT>(sh, lane, total);
    uint16_t* idx_out = p.idx + chunk * p.k;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int bj = __builtin_amdgcn_readlane(excl, j * kTkWaves + w);  // uniform control flow
        if ((sb[j] >> lane) & 1u) {
            // pos < keff when the selection is right; the guard keeps a wrong selection from
            // writing outside this chunk's slots
            const int pos = bj + mbcnt(sb[j]);
            if (pos < keff) {
                idx_out[pos] = (uint16_t)(j * kTkThreads + tid);
                sh.code[pos] = (uint8_t)((uint32_t)qv[j] & ((1u << BITS) - 1u));
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

// Grid-strides over chunks; the barrier at the end of each chunk lets the next one reuse
// the LDS staging.
template <int VPT, int BITS>
__global__ __launch_bounds__(kTkThreads) void tk_kernel(TkParams p, int64_t nchunks) {
    __shared__ TkShared sh;
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        if ((c + 1) * (kTkThreads * VPT) <= p.n) tk_chunk<VPT, BITS, true>(p, c, sh);
        else tk_chunk<VPT, BITS, false>(p, c, sh);
        __syncthreads();
    }
}

template <int BITS>
const void* pick_chunk(int chunk) {
    switch (chunk) {
        case 256: return (const void*)&tk_kernel<1, BITS>;
        case 512: return (const void*)&tk_kernel<2, BITS>;
        case 1024: return (const void*)&tk_kernel<4, BITS>;
        case 2048: return (const void*)&tk_kernel<8, BITS>;
        case 4096: return (const void*)&tk_kernel<16, BITS>;
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
    return hipLaunchKernel(k, dim3((unsigned)grid), dim3(kTkThreads), args, 0, stream);
}

}  // namespace loco
