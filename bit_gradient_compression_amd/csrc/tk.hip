// SparseLoCo-style step: per-chunk Top-k by |h|, low-bit codes of the kept values,
// error feedback ("Communication Efficient LLM Pre-training with SparseLoCo": Top-k
// sparsification, 2-bit quantisation, error feedback).
//
// One 256-thread workgroup (4 waves) owns one chunk of C = 256*VPT elements.  Thread t
// holds Q = VPT/R groups of R consecutive elements (R = min(4, VPT)): element
// i = q*256*R + t*R + r, so each load and store instruction of a wave covers one
// contiguous row of 64*R elements, and index order is (q, t, r) order.  h = g + decay*e
// is also kept in LDS, where the kept elements receive their new error before the whole
// chunk's error is copied out.
//
// Exact selection of the k kept elements (largest |h|, compared as the bit pattern
// ("key"); ties to the lower index):
//  1. a lower bound L of the k-th largest key: the largest value with 12 significant key
//     bits (exponent and 4 mantissa bits) that at least k per-thread maxima reach
//     (12 ballot rounds, wave 0); k keys of the chunk are then >= L;
//  2. the keys >= L (about k + a few dozen) are compacted in index order into LDS (a
//     workgroup prefix over the per-(q, thread) counts);
//  3. wave 0 finds the threshold T (the k-th largest candidate key) by a bit search over
//     the candidates, only over the low bits where L and the chunk's largest key differ,
//     and the last kept tie (the candidates are in index order, so the kept ties are the
//     first ones equal to T); the kept candidates' threads quantise them, write their new
//     error into the LDS copy of h, and their index and code in index order;
//  4. the LDS copy (h, or the new error where kept) is the chunk's new error.
// If k > 256 or more than kTkCap keys are >= L, all four waves search every key instead
// (cross-wave counts through LDS), and the kept elements are compacted over the whole
// chunk; the result is the same exact set.

#include "loco_device.hpp"
#include "loco_internal.hpp"

namespace loco {
namespace {

// The error is loaded and stored non-temporally (read once and written once per step;
// every access instruction of a wave covers one contiguous 1 KB row).  On 2^28 back to
// back / flushed: 0.556 / 0.542 ms, against 0.583 / 0.556 with plain error loads and
// 0.60 / 0.55 with plain loads and stores.
#ifndef LOCO_TK_NT_ERR
#define LOCO_TK_NT_ERR 1
#endif
#ifndef LOCO_TK_NT_ERR_LOAD
#define LOCO_TK_NT_ERR_LOAD 1
#endif
constexpr int kTkThreads = 256;
constexpr int kTkWaves = kTkThreads / kWave;
// The lower bound L keeps key bits 30..kTkBoundLowBit (exponent + 4 mantissa bits).
constexpr int kTkBoundLowBit = 19;

template <int C>
struct TkShared {
    uint32_t h[C];                  // h bits; kept elements get their new error
    uint32_t top[kTkThreads];       // per-thread maximum key
    uint32_t key[kTkCap];           // candidate keys, index order
    uint16_t idx[kTkCap];           // candidate chunk-local indices
    uint8_t code[C];                // kept codes, index order (k <= C)
    int wsum[2][kTkWaves][2];       // per-wave totals of the packed prefix scans (two buffers)
    int cnt[2 * kTkWaves];          // kept candidates per (candidate slot, wave)
    int red[kTkWaves];
    uint32_t wmax[kTkWaves];
    uint32_t L, T;
    int ilast;
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

// Exclusive prefix over the workgroup's threads (thread order) of per-thread counts of up
// to 4 groups, each below 2^16 in total: groups 0 and 1 are packed into one int (bits
// 0-15, 16-31), groups 2 and 3 into another, and each packed int is scanned once.
// Returns each group's exclusive prefix in pre[q] and its total over all threads in
// tot[q].  `buf` picks one of two LDS buffers, so two calls separated by a barrier do not
// collide.  Contains one barrier.
template <int Q, class SH>
__device__ __forceinline__ void block_scan(const int (&cnt)[4], int lane, int w, SH& sh, int buf,
                                           int (&pre)[4], int (&tot)[4]) {
    const int a = cnt[0] | (Q > 1 ? cnt[1] << 16 : 0);
    const int b = (Q > 2 ? cnt[2] : 0) | (Q > 3 ? cnt[3] << 16 : 0);
    const int ia = wave_incl_scan(a, lane);
    const int ib = Q > 2 ? wave_incl_scan(b, lane) : 0;
    if (lane == 63) {
        sh.wsum[buf][w][0] = ia;
        sh.wsum[buf][w][1] = ib;
    }
    __syncthreads();
    int ba = 0, bb = 0, ta = 0, tb = 0;
#pragma unroll
    for (int x = 0; x < kTkWaves; ++x) {
        const int sa = sh.wsum[buf][x][0], sb = sh.wsum[buf][x][1];
        ta += sa;
        tb += sb;
        if (x < w) {
            ba += sa;
            bb += sb;
        }
    }
    const int ea = ba + ia - a, eb = bb + ib - b;  // exclusive, still packed
    pre[0] = ea & 0xFFFF;
    pre[1] = (ea >> 16) & 0xFFFF;
    pre[2] = eb & 0xFFFF;
    pre[3] = (eb >> 16) & 0xFFFF;
    tot[0] = ta & 0xFFFF;
    tot[1] = (ta >> 16) & 0xFFFF;
    tot[2] = tb & 0xFFFF;
    tot[3] = (tb >> 16) & 0xFFFF;
}

template <int BITS>
__device__ __forceinline__ int quantise(float h, float inv) {
    constexpr int QMAX = (1 << (BITS - 1)) - 1;
    return (int)__builtin_amdgcn_fmed3f(__builtin_rintf(h * inv), (float)(-QMAX - 1), (float)QMAX);
}

// R consecutive floats at p (R in {1, 2, 4}; p aligned to 4*R bytes).
template <int R, bool NT>
__device__ __forceinline__ void loadr(const float* p, float* x) {
    if constexpr (R == 4) {
        const f32x4 v = NT ? __builtin_nontemporal_load((const f32x4*)p) : *(const f32x4*)p;
        x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
    } else if constexpr (R == 2) {
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        const f32x2 v = NT ? __builtin_nontemporal_load((const f32x2*)p) : *(const f32x2*)p;
        x[0] = v.x; x[1] = v.y;
    } else {
        x[0] = NT ? __builtin_nontemporal_load(p) : *p;
    }
}

// Elements per thread VPT = Q groups of R consecutive elements; ROW elements per group row.
template <int VPT>
struct TkShape {
    static_assert(VPT <= 16, "C <= 4096");
    static constexpr int C = kTkThreads * VPT;
    static constexpr int R = VPT < 4 ? VPT : 4;
    static constexpr int Q = VPT / R;
    static constexpr int ROW = kTkThreads * R;
};

// g and e of one chunk into registers.  FULL: the chunk has all C elements (every chunk
// but a short last one), loaded as whole vectors with no bounds masks.
template <int VPT, bool FULL>
__device__ __forceinline__ void tk_load(const TkParams& p, int64_t chunk, float (&gv)[TkShape<VPT>::Q][TkShape<VPT>::R],
                                        float (&ev)[TkShape<VPT>::Q][TkShape<VPT>::R]) {
    using S = TkShape<VPT>;
    const int tid = threadIdx.x;
    const int64_t base = chunk * S::C;
    const int64_t rem = p.n - base;
    const int len = FULL ? S::C : (rem < S::C ? (int)rem : S::C);
    const float* gb = p.g + base;
    const float* eb = p.e + base;
#pragma unroll
    for (int q = 0; q < S::Q; ++q) {
        const int i0 = q * S::ROW + tid * S::R;
        if (FULL) {
            loadr<S::R, true>(gb + i0, gv[q]);
            loadr<S::R, LOCO_TK_NT_ERR_LOAD != 0>(eb + i0, ev[q]);
        } else {
#pragma unroll
            for (int r = 0; r < S::R; ++r) {
                gv[q][r] = i0 + r < len ? gb[i0 + r] : 0.0f;
                ev[q][r] = i0 + r < len ? eb[i0 + r] : 0.0f;
            }
        }
    }
}

// One chunk, from its loaded g and e.
template <int VPT, int BITS, bool FULL>
__device__ __forceinline__ void tk_chunk(const TkParams& p, int64_t chunk, TkShared<kTkThreads * VPT>& sh,
                                         const float (&gv)[TkShape<VPT>::Q][TkShape<VPT>::R],
                                         const float (&ev)[TkShape<VPT>::Q][TkShape<VPT>::R]) {
    constexpr int C = TkShape<VPT>::C;
    constexpr int R = TkShape<VPT>::R;
    constexpr int Q = TkShape<VPT>::Q;
    constexpr int ROW = TkShape<VPT>::ROW;  // elements per group row
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

    // A. h = g + decay * e; its key goes to registers, h itself to LDS.  Elements past the
    //    end of a short chunk get key 0, which no threshold tried below (>= 1) admits and
    //    which loses every tie to a real element of lower index (keff <= len).
    uint32_t kv[Q][R];
    {
        // decay 1 skips the multiply: 1 * e is e exactly, so h is the same either way
        const bool unit = p.decay == 1.0f;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            uint32_t hb[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                hb[r] = __float_as_uint(unit ? gv[q][r] + ev[q][r] : gv[q][r] + p.decay * ev[q][r]);
                kv[q][r] = hb[r] & 0x7FFFFFFFu;
            }
            uint32_t* hs = &sh.h[q * ROW + tid * R];
            if constexpr (R == 4) *(u32x4*)hs = u32x4{hb[0], hb[1], hb[2], hb[3]};
            else if constexpr (R == 2) *(u32x2*)hs = u32x2{hb[0], hb[1]};
            else hs[0] = hb[0];
        }
    }
    uint32_t m1 = 0;
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
        for (int r = 0; r < R; ++r) m1 = max(m1, kv[q][r]);
    const uint32_t wm = wave_max_u32(m1);
    if (lane == 0) sh.wmax[w] = wm;
    sh.top[tid] = m1;
    __syncthreads();
    // the chunk's absmax is its largest key, always kept (keff >= 1)
    const uint32_t M = max(max(sh.wmax[0], sh.wmax[1]), max(sh.wmax[2], sh.wmax[3]));
    const float absmax = __uint_as_float(M);
    const float step = absmax / (float)QMAX;
    const float inv = finite_recip(step);  // 0 for a zero chunk or one too small to scale

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
        int cnt[4] = {0, 0, 0, 0};
#pragma unroll
        for (int q = 0; q < Q; ++q)
#pragma unroll
            for (int r = 0; r < R; ++r) cnt[q] += kv[q][r] >= L ? 1 : 0;
        int pre[4], tot[4];
        block_scan<Q>(cnt, lane, w, sh, 0, pre, tot);
        int total = 0;
#pragma unroll
        for (int q = 0; q < Q; ++q) total += tot[q];
        if (total <= kTkCap) {
            int gbase = 0;
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                int pos = gbase + pre[q];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if (kv[q][r] >= L) {
                        sh.key[pos] = kv[q][r];
                        sh.idx[pos] = (uint16_t)(q * ROW + tid * R + r);
                        ++pos;
                    }
                }
                gbase += tot[q];
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
            // the kept candidates, in index order: quantise, new error into the LDS copy,
            // index and code
            const int v = lane < 2 * kTkWaves ? sh.cnt[lane] : 0;
            const int kex = wave_incl_scan(v, lane) - v;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int bs = __builtin_amdgcn_readlane(kex, s * kTkWaves + w);  // uniform control flow
                if ((selb[s] >> lane) & 1u) {
                    const int t = s * kTkThreads + tid;
                    const int pos = bs + mbcnt(selb[s]);
                    const int i = sh.idx[t];
                    const float h = __uint_as_float(sh.h[i]);
                    const int q = quantise<BITS>(h, inv);
                    sh.h[i] = __float_as_uint(h - (float)q * step);
                    if (pos < keff) {
                        idx_out[pos] = (uint16_t)i;
                        sh.code[pos] = (uint8_t)((uint32_t)q & CMASK);
                    }
                }
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
            for (int q = 0; q < Q; ++q)
#pragma unroll
                for (int r = 0; r < R; ++r) c += __popcll(ballot(kv[q][r] >= cand));
            if (lane == 0) sh.red[w] = c;
            __syncthreads();
            c = sh.red[0] + sh.red[1] + sh.red[2] + sh.red[3];
            __syncthreads();
            if (c >= keff) T = cand;
        }
        // ties: the kept ones are the first `need` keys equal to T in index order
        int gt = 0;
#pragma unroll
        for (int q = 0; q < Q; ++q)
#pragma unroll
            for (int r = 0; r < R; ++r) gt += __popcll(ballot(kv[q][r] > T));
        if (lane == 0) sh.red[w] = gt;
        int teq[4] = {0, 0, 0, 0};
#pragma unroll
        for (int q = 0; q < Q; ++q)
#pragma unroll
            for (int r = 0; r < R; ++r) teq[q] += kv[q][r] == T ? 1 : 0;
        int tpre[4], ttot[4];
        block_scan<Q>(teq, lane, w, sh, 1, tpre, ttot);  // its barrier also publishes sh.red
        const int need = keff - (sh.red[0] + sh.red[1] + sh.red[2] + sh.red[3]);
        // the thread whose tie range holds the need-th tie records its index
        {
            int gbase = 0;
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                int seen = gbase + tpre[q];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if (kv[q][r] == T) {
                        ++seen;
                        if (seen == need) sh.ilast = q * ROW + tid * R + r;
                    }
                }
                gbase += ttot[q];
            }
        }
        __syncthreads();
        const int ilast = sh.ilast;

        // E'. compact the kept elements over the whole chunk: new error into the LDS copy,
        //     index and code in index order
        int kc[4] = {0, 0, 0, 0};
#pragma unroll
        for (int q = 0; q < Q; ++q)
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int i = q * ROW + tid * R + r;
                kc[q] += (kv[q][r] > T || (kv[q][r] == T && i <= ilast)) ? 1 : 0;
            }
        int kpre[4], ktot[4];
        block_scan<Q>(kc, lane, w, sh, 0, kpre, ktot);
        int gbase = 0;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            int pos = gbase + kpre[q];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int i = q * ROW + tid * R + r;
                if (kv[q][r] > T || (kv[q][r] == T && i <= ilast)) {
                    const float h = __uint_as_float(sh.h[i]);
                    const int qc = quantise<BITS>(h, inv);
                    sh.h[i] = __float_as_uint(h - (float)qc * step);
                    // pos < keff when the selection is right; the guard keeps a wrong
                    // selection from writing outside this chunk's slots
                    if (pos < keff) {
                        idx_out[pos] = (uint16_t)i;
                        sh.code[pos] = (uint8_t)((uint32_t)qc & CMASK);
                    }
                    ++pos;
                }
            }
            gbase += ktot[q];
        }
    }
    __syncthreads();

    // E. the chunk's new error: h, or the kept elements' residual, copied out of LDS
    {
        float* eb = p.e + base;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int i0 = q * ROW + tid * R;
            const uint32_t* hs = &sh.h[i0];
            if (FULL) {
                if constexpr (R == 4) {
                    if constexpr (LOCO_TK_NT_ERR) __builtin_nontemporal_store(*(const u32x4*)hs, (u32x4*)(eb + i0));
                    else *(u32x4*)(eb + i0) = *(const u32x4*)hs;
                }
                else if constexpr (R == 2) *(u32x2*)(eb + i0) = *(const u32x2*)hs;
                else *(uint32_t*)(eb + i0) = hs[0];
            } else {
#pragma unroll
                for (int r = 0; r < R; ++r)
                    if (i0 + r < len) eb[i0 + r] = __uint_as_float(hs[r]);
            }
        }
    }

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

// Workgroup b takes chunk c0 + b of [c0, c1).  One chunk per workgroup and no loop, so no
// lane address is kept live (or spilled) across chunks.  Full chunks and the short last
// chunk are separate kernels, so the full-chunk code carries no bounds masks (registers
// are allocated per kernel).  (Measured on MI355X: one workgroup per chunk beats a
// persistent grid that loads the next chunk while processing the current one, 0.61
// against 0.66-0.68 ms on 2^28.)
template <int VPT, int BITS, bool FULL>
__global__ __launch_bounds__(kTkThreads) __attribute__((amdgpu_waves_per_eu(LOCO_TK_WAVES_PER_EU)))
void tk_kernel(TkParams p, int64_t c0, int64_t c1) {
    __shared__ TkShared<kTkThreads * VPT> sh;
    const int64_t c = c0 + blockIdx.x;
    if (c >= c1) return;
    float gv[TkShape<VPT>::Q][TkShape<VPT>::R], ev[TkShape<VPT>::Q][TkShape<VPT>::R];
    tk_load<VPT, FULL>(p, c, gv, ev);
    tk_chunk<VPT, BITS, FULL>(p, c, sh, gv, ev);
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
    // whole chunks, at most kTkMaxGrid per launch
    for (int64_t c0 = 0; c0 < nfull; c0 += kTkMaxGrid) {
        int64_t c1 = nfull - c0 < kTkMaxGrid ? nfull : c0 + kTkMaxGrid;
        void* args[] = {(void*)&p, (void*)&c0, (void*)&c1};
        const hipError_t st = hipLaunchKernel(kfull, dim3((unsigned)(c1 - c0)), dim3(kTkThreads), args, 0, stream);
        if (st != hipSuccess) return st;
    }
    if (nall > nfull) {
        void* args[] = {(void*)&p, (void*)&nfull, (void*)&nall};
        return hipLaunchKernel(ktail, dim3(1), dim3(kTkThreads), args, 0, stream);
    }
    return hipSuccess;
}

}  // namespace loco
