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
// Mapping: one workgroup of NT threads per chunk at a time.  The chunk's fp32 accumulator
// lives in LDS (C floats, 16 KB at C = 4096) and is zeroed first.  Thread t owns slots t,
// t+NT, ... of every peer.  The first slot of a batch of peers is loaded into registers in
// one go (all loads in flight together); then the peers are applied one at a time with a
// barrier between them, so every element adds its contributions in peer order.  Within
// one peer the slots name distinct elements, so their read-add-writes never collide.  The
// dense chunk is then written once, each thread storing whole runs of up to 8 outputs.
// Two kernels: a streaming one (k <= NT, at most kSaPeerBatch peers), a persistent grid
// of a few workgroups per compute unit that loads each chunk's payload while it processes
// the previous chunk, and first reads the payloads of many chunks in a read-only pass so
// that its output writes meet no DRAM reads (taken for bf16 output); and a general one,
// one workgroup per chunk, preceded by a pre-read kernel over the payloads of the chunks
// it covers, for the same reason (taken for fp32 output, and whenever the streaming one
// does not apply).

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

// The steps of one chunk, shared by both kernels below.  Thread t owns slot t of every
// peer (and t + NT, ... in the general kernel when k > NT).
template <int C, int BITS, bool OBF, int NT>
struct SaChunk {
    static constexpr int QMAX = (1 << (BITS - 1)) - 1;
    // outputs per thread per store: 16 bytes (4 fp32 or 8 bf16), so each store instruction
    // of a wave writes one contiguous 1 KB row
    static constexpr int VMAX = OBF ? 8 : LOCO_SA_VEC_F32;
    static constexpr int VEC = C / NT >= VMAX ? VMAX : C / NT;
    static constexpr int GROUPS = C / (NT * VEC);
    static_assert(C % NT == 0, "a chunk is a whole number of thread rows");

    // Slot t of a batch of kSaPeerBatch peers for one chunk.
    struct Batch {
        uint32_t ix[kSaPeerBatch], cw[kSaPeerBatch];
        float am[kSaPeerBatch];
    };

    const SaParams& p;
    float* acc;
    int t, lane, k, shift0;
    uint32_t io, co;  // this thread's slot and code-byte offsets inside a chunk's payload

    __device__ SaChunk(const SaParams& p_, float* acc_) : p(p_), acc(acc_) {
        t = threadIdx.x;
        lane = lane_id();
        k = p.k;
        shift0 = (t * BITS) % 8;
        const int ts = t < k ? t : k - 1;  // threads past k re-read slot k-1 and drop it
        io = (uint32_t)ts;
        co = (uint32_t)(ts * BITS) / 8u;
    }

    // Loads without branches, so every load is issued back to back: per peer a uniform
    // chunk pointer, and one lane offset shared by all peers.  The loads only fill
    // registers: nothing reads them until the batch is applied.
    __device__ __forceinline__ void load(int64_t c, int p0, Batch& B) const {
#pragma unroll
        for (int b = 0; b < kSaPeerBatch; ++b) {
            const SaPeerDev pe = p.peer[p0 + b < p.npeers ? p0 + b : p.npeers - 1];
            B.am[b] = pe.absmax[c];
            B.ix[b] = (pe.idx + c * k)[io];
            B.cw[b] = (pe.codes + c * p.cbytes)[co];
        }
    }

    __device__ __forceinline__ void clear() const {
        constexpr int V4 = C / 4;  // 16-byte words per chunk
#pragma unroll
        for (int j = 0; j < (V4 + NT - 1) / NT; ++j) {
            const int i = j * NT + t;
            if (V4 % NT == 0 || i < V4) *(f32x4*)&acc[i * 4] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    }

    // Adds the batch of peers p0.. to the accumulator, one peer at a time with a barrier
    // after each.  Lane b keeps peer b's scale and divides it (one division per lane);
    // readlane hands each step to every lane.  An all-zero chunk has step 0.  WIDE: slots
    // past the first row (k > NT), loaded where used.
    template <bool WIDE>
    __device__ __forceinline__ void apply(int64_t c, int p0, const Batch& B, int len) const {
        float am_mine = 0.0f;
#pragma unroll
        for (int b = 0; b < kSaPeerBatch; ++b) am_mine = (lane == b) ? B.am[b] : am_mine;
        const float step_mine = am_mine / (float)QMAX;
#pragma unroll
        for (int b = 0; b < kSaPeerBatch; ++b) {
            if (p0 + b < p.npeers) {  // uniform: the barrier below is reached by all threads
                const float step =
                    __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, step_mine), b));
                apply_slot<BITS>(acc, t < k ? B.ix[b] : 0xFFFFu, B.cw[b], shift0, step, len);
                if constexpr (WIDE) {
                    const SaPeerDev pe = p.peer[p0 + b];
                    for (int j = t + NT; j < k; j += NT)
                        apply_slot<BITS>(acc, pe.idx[c * k + j], pe.codes[c * p.cbytes + (j * BITS) / 8],
                                         (j * BITS) % 8, step, len);
                }
                __syncthreads();
            }
        }
    }

    // out[base + i] = acc[i] * out_scale for the chunk's len elements
    __device__ __forceinline__ void store(int64_t base, int len) const {
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

    // One chunk, any k, any number of peers, possibly short: every batch is loaded where
    // it is applied.
    __device__ void whole(int64_t c) const {
        const int64_t base = c * C;
        const int len = (int)(p.n - base < C ? p.n - base : C);
        clear();
        __syncthreads();
        for (int p0 = 0; p0 < p.npeers; p0 += kSaPeerBatch) {
            Batch B;
            load(c, p0, B);
            apply<true>(c, p0, B, len);
        }
        store(base, len);
    }
};

// Makes the compiler treat the batch's registers as redefined here: it waits for their
// loads at this point, and later uses need no wait.
template <class Batch>
__device__ __forceinline__ void settle(Batch& B) {
#pragma unroll
    for (int b = 0; b < kSaPeerBatch; ++b) asm volatile("" : "+v"(B.ix[b]), "+v"(B.cw[b]), "+v"(B.am[b]));
}

// Reads 16 bytes per lane at g into the caches and drops them: global_load_lds sends the
// data to LDS at `lds` (+ 16 * lane), an area nothing reads, so no register waits for it.
// It is issued from asm because the compiler orders every load to LDS after the previous
// one (each waits for vmcnt(0)); the caller waits for all of them with an explicit
// s_waitcnt vmcnt(0) before any other memory operation, which also keeps the compiler's
// own counts exact.  M0 holds the LDS address (one wait state before the load reads it)
// and is restored.
__device__ __forceinline__ void read_to_lds16(const void* g, uint32_t lds) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds), "v"(g)
        : "memory");
}

// The whole 16-byte vectors of bytes [lo, hi) of one payload array of `total` bytes
// (16-byte aligned), read into the caches by the NT threads of this workgroup.
template <int NT>
__device__ __forceinline__ void read_pass_range(const void* base, int64_t lo, int64_t hi, int64_t total,
                                                uint32_t lds) {
    const int64_t v1 = min((hi + 15) / 16, total / 16);
    const u32x4* v = (const u32x4*)base;
    for (int64_t i = lo / 16 + threadIdx.x; i < v1; i += NT) read_to_lds16(v + i, lds);
}

// s_waitcnt vmcnt(0), the other counters left as they are (expcnt 7, lgkmcnt 15)
constexpr int kWaitVmcnt0 = 0x0f70;

// The whole 16-byte vectors of bytes [lo, hi) of one payload array of `total` bytes,
// read into the caches by the threads of the grid (thread `first` of `stride`).
__device__ __forceinline__ void read_range_grid(const void* base, int64_t lo, int64_t hi, int64_t total,
                                                int64_t first, int64_t stride, uint32_t lds) {
    const int64_t v1 = min((hi + 15) / 16, total / 16);
    const u32x4* v = (const u32x4*)base;
    for (int64_t i = lo / 16 + first; i < v1; i += stride) read_to_lds16(v + i, lds);
}

// Pre-read for the general kernel: reads every peer's payload of chunks [c0, c1) into the
// caches, so that the aggregation launched next on the stream finds it there and its
// output writes meet no DRAM reads.
template <int NT>
__global__ __launch_bounds__(NT) void sa_preread_kernel(SaParams p, int64_t c0, int64_t c1) {
    __shared__ __attribute__((aligned(16))) uint32_t land[64 * 4];  // one wave's 16-byte loads
    const uint32_t lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)land;
    const int64_t kb = 2 * (int64_t)p.k, cb = p.cbytes;
    const int64_t first = (int64_t)blockIdx.x * NT + threadIdx.x, stride = (int64_t)gridDim.x * NT;
    for (int q = 0; q < p.npeers; ++q) {
        const SaPeerDev pe = p.peer[q];
        read_range_grid(pe.idx, c0 * kb, c1 * kb, p.nchunks * kb, first, stride, lds);
        read_range_grid(pe.codes, c0 * cb, c1 * cb, p.nchunks * cb, first, stride, lds);
        read_range_grid(pe.absmax, c0 * 4, c1 * 4, p.nchunks * 4, first, stride, lds);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
}
constexpr int kSaPrereadThreads = 256;

// General kernel: one workgroup per chunk of [c0, c1), any k and number of peers.
template <int C, int BITS, bool OBF, int NT>
__global__ __launch_bounds__(NT) void sa_kernel(SaParams p, int64_t c0, int64_t c1) {
    __shared__ __attribute__((aligned(16))) float acc[C];
    const SaChunk<C, BITS, OBF, NT> ch(p, acc);
    for (int64_t c = c0 + xcd_remap<kXcds, kSaXcdRun>(blockIdx.x, gridDim.x); c < c1; c += gridDim.x) {
        ch.whole(c);
        __syncthreads();  // the next chunk clears acc
    }
}

// Streaming kernel for k <= NT and at most kSaPeerBatch peers: a persistent grid walks
// the whole chunks, workgroup w taking w, w + gridDim.x, ...  Each step issues the loads
// of the workgroup's next chunk before it processes the current one, so they are in
// flight while it does.  Every step runs the same instructions (the loads are issued
// unconditionally, for the current chunk again on the last step; whole chunks only, so
// the stores are straight-line), and the next batch is settled at the end of a step,
// after the stores: the wait for it then leaves those stores in flight.  A short last
// chunk is done by the last workgroup afterwards.
//
// Read passes: at the start of every p.pass_chunks chunks (whole passes of the grid, so
// all workgroups start one together), the grid first reads the payloads of those chunks,
// each workgroup an equal slice, and waits for them.  The output writes that follow then
// find the payloads in the Infinity Cache instead of mixing DRAM reads into the write
// stream (8 peers of 2^28 into fp32 cache-cold: 0.252 ms without, 0.205 ms after a
// separate read of the payloads).  The pass sizes are set by launch_sa.
template <int C, int BITS, bool OBF, int NT>
__global__ __launch_bounds__(NT) void sa_stream_kernel(SaParams p) {
    __shared__ __attribute__((aligned(16))) float acc[C];
    __shared__ __attribute__((aligned(16))) uint32_t land[64 * 4];  // one wave's 16-byte loads
    using Ch = SaChunk<C, BITS, OBF, NT>;
    const Ch ch(p, acc);
    const int64_t nfull = p.n / C;
    // XCD x (dispatch is round-robin over the XCDs) takes the x-th block of gridDim.x / 8
    // consecutive chunks of every pass, the same on each pass, so chunks whose payloads
    // share cache lines meet in one L2: the L2s fetch the payloads once (runs of 64 that
    // change XCD from pass to pass fetched 1.5x, runs of 1 2.5x)
    const int64_t g = gridDim.x, b = blockIdx.x;
    int64_t c = g % kXcds == 0 ? (b % kXcds) * (g / kXcds) + b / kXcds : b;
    if (c < nfull) {
        using Batch = typename Ch::Batch;
        const int64_t G = gridDim.x;
        const int64_t c0 = c, kb = 2 * (int64_t)p.k, cb = p.cbytes;
        int64_t pass = 0;  // first chunk of the next read pass
        Batch cur, nxt;
        ch.load(c, 0, cur);
        settle(cur);
        for (;;) {
            if (p.pass_chunks > 0 && c - c0 == pass) {  // uniform: c - c0 is this grid pass's first chunk
                // chunks [pass, end) in equal runs, one per workgroup
                const int64_t end = min(pass + p.pass_chunks, nfull), per = (end - pass + G - 1) / G;
                const int64_t ra = min(pass + b * per, end), rb = min(ra + per, end);
                const uint32_t lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)land;
#pragma unroll
                for (int q = 0; q < kSaPeerBatch; ++q) {
                    if (q < p.npeers) {
                        read_pass_range<NT>(p.peer[q].idx, ra * kb, rb * kb, p.nchunks * kb, lds);
                        read_pass_range<NT>(p.peer[q].codes, ra * cb, rb * cb, p.nchunks * cb, lds);
                        read_pass_range<NT>(p.peer[q].absmax, ra * 4, rb * 4, p.nchunks * 4, lds);
                    }
                }
                // all of it in before this workgroup writes again; an explicit wait also
                // leaves no load to LDS pending for the compiler to wait on in later steps
                __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
                pass += p.pass_chunks;
            }
            const int64_t cn = c + G;
            const bool more = cn < nfull;  // uniform
            ch.load(more ? cn : c, 0, nxt);
            ch.clear();
            __syncthreads();
            ch.template apply<false>(c, 0, cur, C);
            ch.store(c * C, C);
            if (!more) break;
            __syncthreads();  // the next chunk clears acc
            c = cn;
            cur = nxt;
            settle(cur);
        }
    }
    if (nfull < p.nchunks && blockIdx.x == gridDim.x - 1) {
        __syncthreads();
        ch.whole(nfull);
    }
}

// Launch shape per output type, measured on MI355X for 8 peers of 2^28 in chunks of 4096
// (cache-cold / back to back): 128 threads per chunk.  The streaming kernel with its read
// passes, fp32 out: 3 workgroups per compute unit 0.211 / 0.206 ms, against 0.331 / 0.330
// with 1, 0.258 / 0.245 with 2, 0.241 / 0.229 with 4 and 0.241 / 0.221 with 6; the
// general kernel after one pre-read beats it (0.193 / 0.195), and is what fp32 output
// takes.  bf16 out: the streaming kernel with 8, 0.127 / 0.116 ms.  The output is ~92% of
// the bytes; a persistent grid with few waves in flight leaves the payload loads' latency
// exposed, one workgroup per chunk hides it once the payloads are in the caches.
template <int C, int BITS>
void pick_out(bool out_bf16, bool stream, const void*& k) {
    // (the streaming kernel is built for an output type only where its setting takes it)
    if (stream && out_bf16) {
        if constexpr (kSaWgPerCuBf16 > 0) k = (const void*)&sa_stream_kernel<C, BITS, true, kSaThreadsBf16>;
    } else if (stream) {
        if constexpr (kSaWgPerCuF32 > 0) k = (const void*)&sa_stream_kernel<C, BITS, false, kSaThreadsF32>;
    } else {
        k = out_bf16 ? (const void*)&sa_kernel<C, BITS, true, kSaThreadsBf16>
                     : (const void*)&sa_kernel<C, BITS, false, kSaThreadsF32>;
    }
}

template <int C>
void pick_bits(int bits, bool out_bf16, bool stream, const void*& k) {
    switch (bits) {
        case 2: pick_out<C, 2>(out_bf16, stream, k); break;
        case 4: pick_out<C, 4>(out_bf16, stream, k); break;
        case 8: pick_out<C, 8>(out_bf16, stream, k); break;
    }
}

}  // namespace

hipError_t launch_sa(const SaParams& p, int chunk, int bits, bool out_bf16, hipStream_t stream) {
    const int threads = out_bf16 ? kSaThreadsBf16 : kSaThreadsF32;
    const int per_cu = out_bf16 ? kSaWgPerCuBf16 : kSaWgPerCuF32;
    const bool streaming = per_cu > 0 && p.k <= threads && p.npeers <= kSaPeerBatch;
    const void* k = nullptr;
    switch (chunk) {
        case 256: pick_bits<256>(bits, out_bf16, streaming, k); break;
        case 512: pick_bits<512>(bits, out_bf16, streaming, k); break;
        case 1024: pick_bits<1024>(bits, out_bf16, streaming, k); break;
        case 2048: pick_bits<2048>(bits, out_bf16, streaming, k); break;
        case 4096: pick_bits<4096>(bits, out_bf16, streaming, k); break;
    }
    if (!k) return hipErrorInvalidValue;
    if (streaming) {
        int cus = 0;
        const hipError_t err = compute_units(cus);
        if (err != hipSuccess) return err;
        // at least one workgroup, at most one per whole chunk (a short last chunk alone
        // takes one workgroup)
        const int64_t nfull = p.n / chunk;
        const int64_t grid = (int64_t)cus * per_cu;
        const int64_t blocks = nfull < 1 ? 1 : (nfull < grid ? nfull : grid);
        // chunks per read pass: whole grid passes whose payloads fit the budget (at least one)
        SaParams q = p;
        const int64_t per_chunk = (int64_t)p.npeers * (2 * (int64_t)p.k + p.cbytes + 4);
        const long long budget = out_bf16 ? kSaPassBytesBf16 : kSaPassBytesF32;
        const int64_t passes = budget / per_chunk / blocks;
        q.pass_chunks = budget <= 0 ? 0 : (passes < 1 ? 1 : passes) * blocks;
        void* args[] = {(void*)&q};
        return hipLaunchKernel(k, dim3((unsigned)blocks), dim3(threads), args, 0, stream);
    }
    // one workgroup per chunk, chunks [c0, c1) per launch; with a pre-read budget, each
    // launch covers chunks whose payloads fit it and is preceded by their pre-read
    const long long pre = out_bf16 ? kSaPrereadBytesBf16 : kSaPrereadBytesF32;
    const int64_t per_chunk = (int64_t)p.npeers * (2 * (int64_t)p.k + p.cbytes + 4);
    int64_t span = pre > 0 ? (int64_t)(pre / per_chunk) : kMaxGrid;
    span = span < 1 ? 1 : (span > kMaxGrid ? kMaxGrid : span);
    int cus = 0;
    if (pre > 0) {
        const hipError_t err = compute_units(cus);
        if (err != hipSuccess) return err;
    }
    for (int64_t c0 = 0; c0 < p.nchunks; c0 += span) {
        int64_t c1 = p.nchunks - c0 < span ? p.nchunks : c0 + span;
        void* args[] = {(void*)&p, (void*)&c0, (void*)&c1};
        if (pre > 0) {
            const int64_t vecs = (c1 - c0) * per_chunk / 16 + 3 * (int64_t)p.npeers;
            int64_t pb = (vecs + kSaPrereadThreads - 1) / kSaPrereadThreads;
            if (pb > (int64_t)cus * 8) pb = (int64_t)cus * 8;
            if (pb < 1) pb = 1;
            const hipError_t err = hipLaunchKernel((const void*)&sa_preread_kernel<kSaPrereadThreads>,
                                                   dim3((unsigned)pb), dim3(kSaPrereadThreads), args, 0, stream);
            if (err != hipSuccess) return err;
        }
        const hipError_t err = hipLaunchKernel(k, dim3((unsigned)(c1 - c0)), dim3(threads), args, 0, stream);
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace loco
