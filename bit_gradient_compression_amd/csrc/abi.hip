// C ABI of the library: argument validation on the host, then one launch per call on
// the caller's stream.  Validation runs before any HIP call, so an error status means
// nothing was launched and nothing was written.

#include <math.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "loco.h"
#include "loco_internal.hpp"

#define LOCO_API extern "C" __attribute__((visibility("default")))

namespace loco {

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool bits_ok(int bits) { return bits == 2 || bits == 4 || bits == 8; }
bool block_ok(int block) { return block == 64 || block == 128 || block == 256 || block == 512; }
bool dtype_ok(int d) { return d == LOCO_F32 || d == LOCO_BF16; }
int dtype_size(int d) { return d == LOCO_I8 ? 1 : (d == LOCO_BF16 ? 2 : 4); }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};
Range range_of(const void* p, int64_t bytes) { return {(uintptr_t)p, (uintptr_t)p + (uintptr_t)bytes}; }
bool overlap(Range a, Range b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

// True if some written range overlaps any other range (written or read); read-only
// ranges may overlap each other.  Empty ranges never overlap.  Sorted by start, a range
// overlaps an earlier one exactly when it starts before the largest end seen so far.
struct Span {
    Range r;
    bool written;
};
bool any_write_overlap(std::vector<Span>& v) {
    std::sort(v.begin(), v.end(), [](const Span& a, const Span& b) { return a.r.lo < b.r.lo; });
    uintptr_t end_any = 0, end_written = 0;
    for (const Span& s : v) {
        if (s.r.lo >= s.r.hi) continue;
        if (s.r.lo < (s.written ? end_any : end_written)) return true;
        end_any = std::max(end_any, s.r.hi);
        if (s.written) end_written = std::max(end_written, s.r.hi);
    }
    return false;
}

int64_t code_bytes(int64_t n, int bits) { return (n * bits + 7) / 8; }
int64_t nblocks(int64_t n, int block) { return (n + block - 1) / block; }

// Sizes beyond this are refused: far above any device memory, and safe from overflow in
// the byte arithmetic above.
constexpr int64_t kMaxElems = (int64_t)1 << 52;

}  // namespace
}  // namespace loco

using namespace loco;

LOCO_API int loco_version(void) { return 10100; }

LOCO_API const char* loco_status_string(int status) {
    switch (status) {
        case LOCO_OK: return "LOCO_OK";
        case LOCO_ERR_INVALID: return "LOCO_ERR_INVALID: invalid argument";
        case LOCO_ERR_ALIGN: return "LOCO_ERR_ALIGN: device pointer not 16-byte aligned";
        case LOCO_ERR_UNSUPPORTED: return "LOCO_ERR_UNSUPPORTED: valid but not built";
        case LOCO_ERR_HIP: return "LOCO_ERR_HIP: kernel launch failed";
    }
    return "unknown status";
}

namespace {

// Shared body of both compensate-quantize entry points.
int compensate_quantize(const loco_cq_segment_t* segs, int nseg, int grad_dtype, int err_dtype,
                        const loco_cq_options_t& o, hipStream_t st) {
    if (nseg < 0 || (nseg > 0 && !segs)) return LOCO_ERR_INVALID;
    if (!dtype_ok(grad_dtype)) return LOCO_ERR_INVALID;
    if (!dtype_ok(err_dtype) && err_dtype != LOCO_I8) return LOCO_ERR_INVALID;
    const int bits = o.bits, block = o.block;
    if (bits < 1 || bits > 8) return LOCO_ERR_INVALID;
    if (!bits_ok(bits)) return LOCO_ERR_UNSUPPORTED;
    if (!isfinite(o.beta) || o.beta < 0.0f || o.beta > 1.0f) return LOCO_ERR_INVALID;
    if (!isfinite(o.fixed_scale) || o.fixed_scale < 0.0f) return LOCO_ERR_INVALID;
    float err_step = 0.0f;
    if (err_dtype == LOCO_I8) {
        // s_e > 0 and 256/s_e finite: the decode e8*fl(1/s_e) and its biased form stay finite.
        if (!isfinite(o.err_scale) || !(o.err_scale > 0.0f)) return LOCO_ERR_INVALID;
        err_step = 1.0f / o.err_scale;
        if (!isfinite(256.0f * err_step)) return LOCO_ERR_INVALID;
    }
    const bool fixed = o.fixed_scale > 0.0f;
    if (!fixed) {
        if (block <= 0) return LOCO_ERR_INVALID;
        if (!block_ok(block)) return LOCO_ERR_UNSUPPORTED;
    }
    const int gs = dtype_size(grad_dtype), es = dtype_size(err_dtype);
    int64_t live = 0;
    for (int i = 0; i < nseg; ++i) {
        const loco_cq_segment_t& s = segs[i];
        if (s.n < 0 || s.n > kMaxElems) return LOCO_ERR_INVALID;
        if (s.n == 0) continue;
        if (!s.grad || !s.err || !s.codes || (!fixed && !s.absmax)) return LOCO_ERR_INVALID;
        if (!aligned16(s.grad) || !aligned16(s.err) || !aligned16(s.codes) || (!fixed && !aligned16(s.absmax)))
            return LOCO_ERR_ALIGN;
        Range r[4] = {range_of(s.grad, s.n * gs), range_of(s.err, s.n * es),
                      range_of(s.codes, code_bytes(s.n, bits)),
                      range_of(s.absmax, fixed ? 0 : nblocks(s.n, block) * 4)};
        for (int a = 0; a < 4; ++a)
            for (int b = a + 1; b < 4; ++b)
                if (overlap(r[a], r[b])) return LOCO_ERR_INVALID;
        ++live;
    }
    if (live == 0) return LOCO_OK;
    // across segments: no buffer the call writes (any segment's err, codes, absmax) may overlap another
    // buffer of the call; gradients are only read and may overlap each other
    std::vector<Span> spans;
    spans.reserve(4 * live);
    for (int i = 0; i < nseg; ++i) {
        const loco_cq_segment_t& s = segs[i];
        if (s.n == 0) continue;
        spans.push_back({range_of(s.grad, s.n * gs), false});
        spans.push_back({range_of(s.err, s.n * es), true});
        spans.push_back({range_of(s.codes, code_bytes(s.n, bits)), true});
        if (!fixed) spans.push_back({range_of(s.absmax, nblocks(s.n, block) * 4), true});
    }
    if (any_write_overlap(spans)) return LOCO_ERR_INVALID;

    CqParams p;
    memset(&p, 0, sizeof(p));
    p.beta = o.beta;
    p.omega = 1.0f - o.beta;
    if (fixed) {
        p.fixed_inv = o.fixed_scale;
        p.fixed_step = 1.0f / o.fixed_scale;
    }
    if (err_dtype == LOCO_I8) {
        p.err_scale = o.err_scale;
        p.err_step = err_step;
    }
    p.reset = o.reset_error != 0;
    const int64_t tile = cq_tile_elems(err_dtype);
    int i = 0;
    while (i < nseg) {
        p.nseg = 0;
        p.ntiles = 0;
        for (; i < nseg && p.nseg < kCqMaxSeg; ++i) {
            const loco_cq_segment_t& s = segs[i];
            if (s.n == 0) continue;
            CqSegDev& d = p.seg[p.nseg++];
            d.g = s.grad;
            d.e = s.err;
            d.codes = s.codes;
            d.absmax = s.absmax;
            d.n = s.n;
            d.tile0 = p.ntiles;
            p.ntiles += (s.n + tile - 1) / tile;
        }
        if (p.nseg == 0) break;
        if (launch_cq(p, grad_dtype, err_dtype, bits, block, fixed, st) != hipSuccess) return LOCO_ERR_HIP;
    }
    return LOCO_OK;
}

}  // namespace

LOCO_API int loco_compensate_quantize(const loco_cq_segment_t* segs, int nseg,
                                      loco_dtype_t grad_dtype, loco_dtype_t err_dtype,
                                      int bits, int block, float beta, float fixed_scale,
                                      void* stream) {
    if (err_dtype == LOCO_I8) return LOCO_ERR_INVALID;  // needs s_e: use the _ex entry point
    loco_cq_options_t o;
    memset(&o, 0, sizeof(o));
    o.bits = bits;
    o.block = block;
    o.beta = beta;
    o.fixed_scale = fixed_scale;
    return compensate_quantize(segs, nseg, grad_dtype, err_dtype, o, (hipStream_t)stream);
}

LOCO_API int loco_compensate_quantize_ex(const loco_cq_segment_t* segs, int nseg,
                                         loco_dtype_t grad_dtype, loco_dtype_t err_dtype,
                                         const loco_cq_options_t* opt, void* stream) {
    if (!opt) return LOCO_ERR_INVALID;
    return compensate_quantize(segs, nseg, grad_dtype, err_dtype, *opt, (hipStream_t)stream);
}

namespace {

// Checks shared by both dequant-reduce entry points; fills the payload part of p.
int dr_setup(const loco_payload_t* peers, int npeers, int64_t n, int bits, int block, float fixed_scale,
             float out_scale, DrParams& p, bool& fixed) {
    if (n < 0 || n > kMaxElems) return LOCO_ERR_INVALID;
    if (npeers < 1 || !peers) return LOCO_ERR_INVALID;
    if (npeers > kDrMaxPeers) return LOCO_ERR_UNSUPPORTED;
    if (bits < 1 || bits > 8) return LOCO_ERR_INVALID;
    if (!bits_ok(bits)) return LOCO_ERR_UNSUPPORTED;
    if (!isfinite(fixed_scale) || fixed_scale < 0.0f) return LOCO_ERR_INVALID;
    if (!isfinite(out_scale)) return LOCO_ERR_INVALID;
    fixed = fixed_scale > 0.0f;
    if (!fixed) {
        if (block <= 0) return LOCO_ERR_INVALID;
        if (!block_ok(block)) return LOCO_ERR_UNSUPPORTED;
    }
    memset(&p, 0, sizeof(p));
    for (int i = 0; i < npeers; ++i) {
        if (!peers[i].codes || (!fixed && !peers[i].absmax)) return LOCO_ERR_INVALID;
        if (!aligned16(peers[i].codes) || (!fixed && !aligned16(peers[i].absmax))) return LOCO_ERR_ALIGN;
        p.peer[i].codes = peers[i].codes;
        p.peer[i].absmax = peers[i].absmax;
    }
    for (int i = npeers; i < npeers + kDrPeerBatch; ++i) p.peer[i] = p.peer[npeers - 1];
    p.npeers = npeers;
    p.n = n;
    p.fixed_step = fixed ? 1.0f / fixed_scale : 0.0f;
    p.out_scale = out_scale;
    return LOCO_OK;
}

// An output range must not overlap any peer's payload.
bool overlaps_payloads(const loco_payload_t* peers, int npeers, int64_t n, int bits, int block, bool fixed, Range r) {
    for (int i = 0; i < npeers; ++i) {
        if (overlap(r, range_of(peers[i].codes, code_bytes(n, bits)))) return true;
        if (!fixed && overlap(r, range_of(peers[i].absmax, nblocks(n, block) * 4))) return true;
    }
    return false;
}

}  // namespace

LOCO_API int loco_dequant_reduce(const loco_payload_t* peers, int npeers, int64_t n, int bits,
                                 int block, float fixed_scale, float out_scale, void* out,
                                 loco_dtype_t out_dtype, void* stream) {
    DrParams p;
    bool fixed = false;
    const int st = dr_setup(peers, npeers, n, bits, block, fixed_scale, out_scale, p, fixed);
    if (st != LOCO_OK) return st;
    if (!dtype_ok(out_dtype)) return LOCO_ERR_INVALID;
    if (n == 0) return LOCO_OK;
    if (!out) return LOCO_ERR_INVALID;
    if (!aligned16(out)) return LOCO_ERR_ALIGN;
    if (overlaps_payloads(peers, npeers, n, bits, block, fixed, range_of(out, n * dtype_size(out_dtype))))
        return LOCO_ERR_INVALID;
    const int mode = out_dtype == LOCO_BF16 ? kDrOutBf16 : kDrOutF32;
    p.ntiles = (n + dr_tile_elems(mode) - 1) / dr_tile_elems(mode);
    p.out = out;
    if (launch_dr(p, bits, block, fixed, mode, (hipStream_t)stream) != hipSuccess) return LOCO_ERR_HIP;
    return LOCO_OK;
}

LOCO_API int loco_dequant_reduce_adam(const loco_payload_t* peers, int npeers, int64_t n, int bits, int block,
                                      float fixed_scale, float out_scale, const loco_adam_t* adam, float* param,
                                      float* m, float* v, uint16_t* param_bf16, void* stream) {
    DrParams p;
    bool fixed = false;
    const int st = dr_setup(peers, npeers, n, bits, block, fixed_scale, out_scale, p, fixed);
    if (st != LOCO_OK) return st;
    if (!adam) return LOCO_ERR_INVALID;
    const loco_adam_t& a = *adam;
    if (!isfinite(a.lr) || !isfinite(a.beta1) || !isfinite(a.beta2) || !isfinite(a.delta)) return LOCO_ERR_INVALID;
    if (a.beta1 < 0.0f || a.beta1 > 1.0f || a.beta2 < 0.0f || a.beta2 > 1.0f || !(a.delta > 0.0f))
        return LOCO_ERR_INVALID;
    if (n == 0) return LOCO_OK;
    if (!param || !m || !v) return LOCO_ERR_INVALID;
    if (!aligned16(param) || !aligned16(m) || !aligned16(v) || (param_bf16 && !aligned16(param_bf16)))
        return LOCO_ERR_ALIGN;
    Range r[4] = {range_of(param, n * 4), range_of(m, n * 4), range_of(v, n * 4),
                  range_of(param_bf16, param_bf16 ? n * 2 : 0)};
    for (int x = 0; x < 4; ++x) {
        for (int y = x + 1; y < 4; ++y)
            if (overlap(r[x], r[y])) return LOCO_ERR_INVALID;
        if (overlaps_payloads(peers, npeers, n, bits, block, fixed, r[x])) return LOCO_ERR_INVALID;
    }
    p.ntiles = (n + dr_tile_elems(kDrOutAdam) - 1) / dr_tile_elems(kDrOutAdam);
    p.theta = param;
    p.m = m;
    p.v = v;
    p.theta_bf16 = param_bf16;
    p.lr = a.lr;
    p.beta1 = a.beta1;
    p.omb1 = 1.0f - a.beta1;
    p.beta2 = a.beta2;
    p.omb2 = 1.0f - a.beta2;
    p.delta = a.delta;
    if (launch_dr(p, bits, block, fixed, kDrOutAdam, (hipStream_t)stream) != hipSuccess) return LOCO_ERR_HIP;
    return LOCO_OK;
}

LOCO_API int loco_topk_quantize(const float* grad, float* err, int64_t n, int chunk, int k, int bits,
                                float ef_decay, uint16_t* idx, uint8_t* codes, float* absmax,
                                void* stream) {
    if (n < 0 || n > kMaxElems) return LOCO_ERR_INVALID;
    if (chunk <= 0 || chunk > 65536) return LOCO_ERR_INVALID;
    if (k < 1 || k > chunk) return LOCO_ERR_INVALID;
    if (bits < 1 || bits > 8) return LOCO_ERR_INVALID;
    if (!isfinite(ef_decay) || ef_decay < 0.0f || ef_decay > 1.0f) return LOCO_ERR_INVALID;
    if (!bits_ok(bits)) return LOCO_ERR_UNSUPPORTED;
    if (chunk != 256 && chunk != 512 && chunk != 1024 && chunk != 2048 && chunk != 4096)
        return LOCO_ERR_UNSUPPORTED;
    if (n == 0) return LOCO_OK;
    if (!grad || !err || !idx || !codes || !absmax) return LOCO_ERR_INVALID;
    if (!aligned16(grad) || !aligned16(err) || !aligned16(idx) || !aligned16(codes) || !aligned16(absmax))
        return LOCO_ERR_ALIGN;
    const int64_t chunks = (n + chunk - 1) / chunk;
    Range r[5] = {range_of(grad, n * 4), range_of(err, n * 4), range_of(idx, chunks * k * 2),
                  range_of(codes, chunks * code_bytes(k, bits)), range_of(absmax, chunks * 4)};
    for (int a = 0; a < 5; ++a)
        for (int b = a + 1; b < 5; ++b)
            if (overlap(r[a], r[b])) return LOCO_ERR_INVALID;
    TkParams p;
    p.g = grad;
    p.e = err;
    p.n = n;
    p.k = k;
    p.decay = ef_decay;
    p.idx = idx;
    p.codes = codes;
    p.absmax = absmax;
    if (launch_tk(p, chunk, bits, (hipStream_t)stream) != hipSuccess) return LOCO_ERR_HIP;
    return LOCO_OK;
}

LOCO_API int loco_sparse_aggregate(const loco_sparse_payload_t* peers, int npeers, int64_t n, int chunk, int k,
                                   int bits, float out_scale, void* out, loco_dtype_t out_dtype, void* stream) {
    if (n < 0 || n > kMaxElems) return LOCO_ERR_INVALID;
    if (npeers < 1 || !peers) return LOCO_ERR_INVALID;
    if (npeers > kDrMaxPeers) return LOCO_ERR_UNSUPPORTED;
    if (chunk <= 0 || chunk > 65536) return LOCO_ERR_INVALID;
    if (k < 1 || k > chunk) return LOCO_ERR_INVALID;
    if (bits < 1 || bits > 8) return LOCO_ERR_INVALID;
    if (!bits_ok(bits)) return LOCO_ERR_UNSUPPORTED;
    if (chunk != 256 && chunk != 512 && chunk != 1024 && chunk != 2048 && chunk != 4096)
        return LOCO_ERR_UNSUPPORTED;
    if (!isfinite(out_scale)) return LOCO_ERR_INVALID;
    if (!dtype_ok(out_dtype)) return LOCO_ERR_INVALID;
    if (n == 0) return LOCO_OK;
    if (!out) return LOCO_ERR_INVALID;
    if (!aligned16(out)) return LOCO_ERR_ALIGN;
    const int64_t chunks = (n + chunk - 1) / chunk;
    const Range ro = range_of(out, n * dtype_size(out_dtype));
    for (int i = 0; i < npeers; ++i) {
        const loco_sparse_payload_t& pe = peers[i];
        if (!pe.idx || !pe.codes || !pe.absmax) return LOCO_ERR_INVALID;
        if (!aligned16(pe.idx) || !aligned16(pe.codes) || !aligned16(pe.absmax)) return LOCO_ERR_ALIGN;
        if (overlap(ro, range_of(pe.idx, chunks * k * 2)) || overlap(ro, range_of(pe.codes, chunks * code_bytes(k, bits))) ||
            overlap(ro, range_of(pe.absmax, chunks * 4)))
            return LOCO_ERR_INVALID;
    }
    SaParams p;
    memset(&p, 0, sizeof(p));
    for (int i = 0; i < npeers; ++i) {
        p.peer[i].idx = peers[i].idx;
        p.peer[i].codes = peers[i].codes;
        p.peer[i].absmax = peers[i].absmax;
    }
    p.npeers = npeers;
    p.k = k;
    p.cbytes = (int)code_bytes(k, bits);
    p.n = n;
    p.nchunks = chunks;
    p.out_scale = out_scale;
    p.out = out;
    if (launch_sa(p, chunk, bits, out_dtype == LOCO_BF16, (hipStream_t)stream) != hipSuccess) return LOCO_ERR_HIP;
    return LOCO_OK;
}
