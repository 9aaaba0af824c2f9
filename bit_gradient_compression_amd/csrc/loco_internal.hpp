// Host-side interface between the C ABI (abi.hip) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace loco {

// ---- compensate-quantize -----------------------------------------------------------

// Segments per launch; a call with more segments is split into several launches.
constexpr int kCqMaxSeg = 32;
// Elements per lane per sub-tile, and sub-tiles per wave tile.
constexpr int kCqVec = 8;
constexpr int kCqUnroll = 2;
constexpr int kCqTile = 64 * kCqVec * kCqUnroll;  // elements per wave tile
constexpr int kCqThreads = 256;

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
};

hipError_t launch_cq(const CqParams& p, bool grad_bf16, bool err_bf16, int bits, int block,
                     bool fixed, int max_blocks, hipStream_t stream);

// ---- dequant-reduce ---------------------------------------------------------------

constexpr int kDrMaxPeers = 128;
constexpr int kDrVec = 32;                 // elements per lane
constexpr int kDrTile = 64 * kDrVec;       // elements per wave tile
constexpr int kDrThreads = 256;

struct DrPeerDev {
    const uint8_t* codes;
    const float* absmax;
};

struct DrParams {
    DrPeerDev peer[kDrMaxPeers];
    int npeers;
    int64_t n;
    int64_t ntiles;
    float fixed_step;
    float out_scale;
    void* out;
};

hipError_t launch_dr(const DrParams& p, int bits, int block, bool fixed, bool out_bf16,
                     int max_blocks, hipStream_t stream);

// ---- chunked Top-k ----------------------------------------------------------------

// Candidate list capacity of the fast selection path.
constexpr int kTkCap = 512;
// Workgroups of one Top-k launch (one 64-lane workgroup per chunk at a time).
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

// Compute units of the current device (cached per device).
int device_cus();

}  // namespace loco
