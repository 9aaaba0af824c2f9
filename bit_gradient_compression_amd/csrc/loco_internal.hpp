// Host-side interface between the C ABI (abi.hip) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace loco {

// ---- compensate-quantize -----------------------------------------------------------

// Launch shape of the streaming kernels.  The grid is not persistent: each wave takes one
// tile and exits, so the waves in flight sweep memory in address order.  Past kMaxGrid
// workgroups the launcher launches again, from the next tile.
#ifndef LOCO_CQ_UNROLL
#define LOCO_CQ_UNROLL 1
#endif
// An 8-bit error moves 4.5 bytes per element and spends ~25 VALU instructions on it, so
// its waves take 2 sub-tiles (50 VGPRs, 8 waves per SIMD) and XCD runs of 64: measured
// when chosen, 0.674 ms on the 7B shard against 0.70 with 4 sub-tiles (5 waves) and 0.78
// with 1.
#ifndef LOCO_CQ_UNROLL_I8
#define LOCO_CQ_UNROLL_I8 2
#endif
#ifndef LOCO_CQ_XCD_RUN_I8
#define LOCO_CQ_XCD_RUN_I8 64
#endif
// A bf16 error (6.5 B per element) keeps 1 sub-tile per wave (32 VGPRs) and XCD runs of
// 32: the MoE experts' 1,409,286,144 elements take 1.46-1.47 ms, against 1.48-1.53 with 2
// or 4 sub-tiles (runs of 32 or 64) and 1.50-1.52 with runs of 16.
#ifndef LOCO_CQ_UNROLL_BF16
#define LOCO_CQ_UNROLL_BF16 1
#endif
#ifndef LOCO_CQ_XCD_RUN_BF16
#define LOCO_CQ_XCD_RUN_BF16 32
#endif
// Workgroup size and XCD run per error kind, with runs of 128 waves in each case.  An fp32
// error takes one-wave workgroups in runs of 128, an 8-bit error two-wave workgroups in
// runs of 64, a bf16 error four-wave workgroups in runs of 32.  Measured on MI355X (back
// to back / flushed, ms): 7B shard 1.389 / 1.387 against 1.403-1.412 / 1.403 with 4-wave
// workgroups; LLaMA layer 0.329 / 0.327 against 0.335 / 0.335; 8-bit error 0.612 / 0.614
// against 0.629 / 0.620.  The MoE experts (bf16 error) are slower with smaller workgroups
// (1.46-1.56 against 1.43-1.44).  Other mixes (64-thread workgroups in runs of 64 or 256;
// 128-thread ones in runs of 64 for the fp32 error; one-wave ones for the 8-bit error)
// fall between these and the old default.
#ifndef LOCO_CQ_THREADS
#define LOCO_CQ_THREADS 64
#endif
#ifndef LOCO_DR_UNROLL
#define LOCO_DR_UNROLL 2
#endif
#ifndef LOCO_DR_THREADS
#define LOCO_DR_THREADS 256
#endif
// Top-k: at least 6 waves per SIMD.  Since each workgroup takes one chunk and nothing is
// carried from chunk to chunk, the kernel needs 60 VGPRs and spills nothing.
#ifndef LOCO_TK_WAVES_PER_EU
#define LOCO_TK_WAVES_PER_EU 6
#endif
#ifndef LOCO_CQ_XCD_RUN
#define LOCO_CQ_XCD_RUN 128
#endif
#ifndef LOCO_SA_XCD_RUN
#define LOCO_SA_XCD_RUN 64
#endif
#ifndef LOCO_DR_XCD_RUN
#define LOCO_DR_XCD_RUN 16
#endif
constexpr int64_t kMaxGrid = (int64_t)1 << 22;
// Workgroups are dispatched round-robin over the chip's 8 XCDs (each with its own L2).
// The streaming kernels renumber their workgroups so that runs of consecutive logical
// workgroups execute on one XCD (1: identity).  Measured on MI355X for compensate-
// quantize: runs of ~128 waves per XCD moved the fused kernel from ~68% to ~71.5% of peak
// HBM bandwidth; short runs (16-32 waves) are slower than the identity.
constexpr int kXcds = 8;
constexpr int kCqXcdRun = LOCO_CQ_XCD_RUN;
constexpr int kCqXcdRunI8 = LOCO_CQ_XCD_RUN_I8;
constexpr int kCqXcdRunBf16 = LOCO_CQ_XCD_RUN_BF16;
constexpr int cq_xcd_run(int err_kind) {
    return err_kind == 2 ? kCqXcdRunI8 : err_kind == 1 ? kCqXcdRunBf16 : kCqXcdRun;
}
constexpr int kDrXcdRun = LOCO_DR_XCD_RUN;
constexpr int kSaXcdRun = LOCO_SA_XCD_RUN;

// Segments per launch; a call with more segments is split into several launches.
constexpr int kCqMaxSeg = 32;
// Elements per lane per sub-tile, and sub-tiles per wave tile.
constexpr int kCqVec = 8;
constexpr int kCqUnroll = LOCO_CQ_UNROLL;
// An int8 error moves 4.5 B per element instead of 10.5, so its waves take more sub-tiles
// to keep as many bytes in flight.
constexpr int kCqUnrollI8 = LOCO_CQ_UNROLL_I8;
constexpr int kCqUnrollBf16 = LOCO_CQ_UNROLL_BF16;
constexpr int cq_unroll(int err_kind) {
    return err_kind == 2 ? kCqUnrollI8 : err_kind == 1 ? kCqUnrollBf16 : kCqUnroll;
}
constexpr int cq_tile_elems(int err_kind) { return 64 * kCqVec * cq_unroll(err_kind); }  // per wave tile
constexpr int kCqThreads = LOCO_CQ_THREADS;
// Workgroup size per error kind (threads; a multiple of 64).
#ifndef LOCO_CQ_THREADS_I8
#define LOCO_CQ_THREADS_I8 128
#endif
#ifndef LOCO_CQ_THREADS_BF16
#define LOCO_CQ_THREADS_BF16 256
#endif
constexpr int kCqThreadsI8 = LOCO_CQ_THREADS_I8;
constexpr int kCqThreadsBf16 = LOCO_CQ_THREADS_BF16;
constexpr int cq_threads(int err_kind) {
    return err_kind == 2 ? kCqThreadsI8 : err_kind == 1 ? kCqThreadsBf16 : kCqThreads;
}

struct CqSegDev {
    const void* g;
    void* e;
    uint8_t* codes;
    float* absmax;
    int64_t n;
    int64_t tile0;  // first wave tile of this segment in the launch's tile space
};

struct CqParams {
    CqSegDev seg[kCqMaxSeg];
    int nseg;
    int64_t ntiles;
    float beta, omega;            // e' = beta*e + omega*r, omega = fl(1 - beta)
    float fixed_inv, fixed_step;  // fixed-scale mode: inv = s, step = fl(1/s)
    float err_scale, err_step;    // 8-bit error: e8 = clamp(rint(e*s_e)), e = e8*fl(1/s_e)
    int reset;                    // nonzero: store e' = 0 this step
};

// Element kinds: grad_kind 0 fp32 / 1 bf16; err_kind 0 fp32 / 1 bf16 / 2 int8 codes.
hipError_t launch_cq(const CqParams& p, int grad_kind, int err_kind, int bits, int block,
                     bool fixed, hipStream_t stream);

// ---- dequant-reduce ---------------------------------------------------------------

constexpr int kDrMaxPeers = 128;
constexpr int kDrVec = 8;                          // consecutive outputs per lane per sub-tile
constexpr int kDrUnroll = LOCO_DR_UNROLL;          // sub-tiles per wave tile
constexpr int kDrThreads = LOCO_DR_THREADS;
// The fused Adam step: one-wave workgroups in XCD runs of 64 (0.527-0.529 / 0.526-0.528 ms
// back to back / flushed on 8 peers x 105,250,000, against 0.531-0.533 / 0.536-0.538
// with the shard's 4-wave workgroups in runs of 16; the bf16 shard is within noise of its
// default with either).
#ifndef LOCO_DRA_THREADS
#define LOCO_DRA_THREADS 64
#endif
#ifndef LOCO_DRA_XCD_RUN
#define LOCO_DRA_XCD_RUN 64
#endif

// Output modes: the reduced shard as fp32 or bf16, or the fused Adam-family step.
enum : int { kDrOutF32 = 0, kDrOutBf16 = 1, kDrOutAdam = 2 };
constexpr int dr_threads(int mode) { return mode == kDrOutAdam ? LOCO_DRA_THREADS : kDrThreads; }
constexpr int dr_xcd_run(int mode) { return mode == kDrOutAdam ? LOCO_DRA_XCD_RUN : LOCO_DR_XCD_RUN; }
// The fused step holds theta, m and v of each sub-tile in registers as well, so its waves
// take one sub-tile.
#ifndef LOCO_DRA_UNROLL
#define LOCO_DRA_UNROLL 1
#endif
constexpr int kDrUnrollAdam = LOCO_DRA_UNROLL;
constexpr int dr_unroll(int mode) { return mode == kDrOutAdam ? kDrUnrollAdam : kDrUnroll; }
constexpr int dr_tile_elems(int mode) { return 64 * kDrVec * dr_unroll(mode); }  // per wave tile
constexpr int kDrPeerBatch = 8;                    // peers whose codes are loaded together

struct DrPeerDev {
    const uint8_t* codes;
    const float* absmax;
};

struct DrParams {
    // Entries npeers .. npeers + kDrPeerBatch - 1 repeat the last peer, so a batch of
    // loads past the last peer reads valid memory and needs no bounds branch.
    DrPeerDev peer[kDrMaxPeers + kDrPeerBatch];
    int npeers;
    int64_t n;
    int64_t ntiles;
    float fixed_step;
    float out_scale;
    void* out;
    // fused Adam-family step (mode kDrOutAdam)
    float* theta;
    float* m;
    float* v;
    uint16_t* theta_bf16;  // may be null
    float lr, beta1, omb1, beta2, omb2, delta;  // omb = fl(1 - beta)
};

hipError_t launch_dr(const DrParams& p, int bits, int block, bool fixed, int mode, hipStream_t stream);

// ---- chunked Top-k ----------------------------------------------------------------

// Candidate list capacity of the fast selection path.
constexpr int kTkCap = 512;

// Workgroups of one Top-k launch (one 256-thread workgroup per chunk).
constexpr int64_t kTkMaxGrid = 1 << 20;

struct TkParams {
    const float* g;
    float* e;
    int64_t n;
    int k;
    float decay;
    uint16_t* idx;
    uint8_t* codes;
    float* absmax;
};

hipError_t launch_tk(const TkParams& p, int chunk, int bits, hipStream_t stream);

// Compute units of the current device, queried once per device and kept (so launches that
// size a persistent grid make no device query while a caller captures a graph).
// Thread-safe: concurrent first calls store the same value.
inline hipError_t compute_units(int& cus) {
    static std::atomic<int> cached[64];
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    const bool cacheable = dev >= 0 && dev < 64;
    if (cacheable) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            cus = c;
            return hipSuccess;
        }
    }
    err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
    if (cus <= 0) return hipErrorInvalidValue;
    if (cacheable) cached[dev].store(cus, std::memory_order_relaxed);
    return hipSuccess;
}

// ---- sparse aggregation ------------------------------------------------------------

#ifndef LOCO_SA_WG_PER_CU_F32
#define LOCO_SA_WG_PER_CU_F32 0
#endif
#ifndef LOCO_SA_WG_PER_CU_BF16
#define LOCO_SA_WG_PER_CU_BF16 8
#endif
#ifndef LOCO_SA_VEC_F32
#define LOCO_SA_VEC_F32 4
#endif
#ifndef LOCO_SA_THREADS_F32
#define LOCO_SA_THREADS_F32 128
#endif
#ifndef LOCO_SA_THREADS_BF16
#define LOCO_SA_THREADS_BF16 128
#endif
constexpr int kSaThreadsF32 = LOCO_SA_THREADS_F32;    // threads per chunk, fp32 output
constexpr int kSaThreadsBf16 = LOCO_SA_THREADS_BF16;  // threads per chunk, bf16 output
constexpr int kSaPeerBatch = 8;  // peers whose first slot is loaded together
// Workgroups per compute unit of the persistent grid, per output type: each workgroup
// takes every gridDim.x-th chunk and loads the next chunk's payload while it processes
// the current one (0: the general kernel, one workgroup per chunk, after a pre-read).
// Measured on 8 peers of 2^28 in chunks of 4096 (back to back / cache-flushed, ms): fp32
// out 0.195 / 0.193 with the general kernel and one pre-read, against 0.203 / 0.213 with
// 3 persistent workgroups per compute unit and 0.178 / 0.240 for the general kernel
// without the pre-read; bf16 out 0.116 / 0.127 with 8 persistent workgroups, against
// 0.127 / 0.130 with the general kernel and a pre-read.
constexpr int kSaWgPerCuF32 = LOCO_SA_WG_PER_CU_F32;
constexpr int kSaWgPerCuBf16 = LOCO_SA_WG_PER_CU_BF16;
#ifndef LOCO_SA_PASS_BYTES_F32
#define LOCO_SA_PASS_BYTES_F32 (64LL << 20)
#endif
#ifndef LOCO_SA_PASS_BYTES_BF16
#define LOCO_SA_PASS_BYTES_BF16 (128LL << 20)
#endif
// The streaming kernel reads the peers' payloads in read-only passes before it writes the
// output they cover, at most this many payload bytes per pass, per output type (0: no
// read pass).  A pass leaves them in the 256 MB Infinity Cache, so the output writes that
// follow meet no DRAM reads.  Measured on 8 peers of 2^28 (94.5 MiB of payloads), the
// slower of cache-cold and back-to-back, ms: fp32 out 0.263 without, 0.219 in one pass,
// 0.210 in two of <= 64 MiB, 0.220 in <= 32 MiB passes; bf16 out 0.171 without, 0.131
// in one pass, 0.154 in two.
constexpr long long kSaPassBytesF32 = LOCO_SA_PASS_BYTES_F32;
constexpr long long kSaPassBytesBf16 = LOCO_SA_PASS_BYTES_BF16;
// The general kernel (one workgroup per chunk): payload bytes per launch, each launch
// preceded by a pre-read of its chunks' payloads into the caches (0: one launch, no
// pre-read).  fp32 out, 8 peers of 2^28 (99 MB of payloads), back to back / flushed, ms:
// one pre-read of all of it 0.195 / 0.193; launches of <= 64 MB 0.197 / 0.200, <= 32 MB
// 0.201 / 0.207.
#ifndef LOCO_SA_PREREAD_BYTES_F32
#define LOCO_SA_PREREAD_BYTES_F32 (128LL << 20)
#endif
#ifndef LOCO_SA_PREREAD_BYTES_BF16
#define LOCO_SA_PREREAD_BYTES_BF16 0
#endif
constexpr long long kSaPrereadBytesF32 = LOCO_SA_PREREAD_BYTES_F32;
constexpr long long kSaPrereadBytesBf16 = LOCO_SA_PREREAD_BYTES_BF16;

struct SaPeerDev {
    const uint16_t* idx;
    const uint8_t* codes;
    const float* absmax;
};

struct SaParams {
    SaPeerDev peer[kDrMaxPeers];
    int npeers;
    int k;
    int cbytes;  // code bytes per chunk, ceil(k*bits/8)
    int64_t n;
    int64_t nchunks;
    float out_scale;
    void* out;
    int64_t pass_chunks;  // chunks whose payloads one read pass covers (a multiple of the
                          // grid; 0: no read pass); set by launch_sa
};

hipError_t launch_sa(const SaParams& p, int chunk, int bits, bool out_bf16, hipStream_t stream);

}  // namespace loco
