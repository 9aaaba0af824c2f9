/*
 * loco.h - C ABI of the MI355X (gfx950) library for LoCo's per-GPU gradient path.
 *
 * Sources of the operations (page title, section and equation):
 *   "LoCo: Low-Bit Communication Adaptor for Large-scale Model Training"
 *   (arXiv 2407.04480): Sec. 3.1 Eqns. (1)-(3) compensate and compress,
 *   Sec. 3.2 Eqns. (4)-(5) the moving-average compression error,
 *   Sec. 3.3 Eqn. (8) the all2all partitions and their high-precision average,
 *   Sec. 4 Eqn. (9) the Adam-family step that consumes the average.
 *   "Communication Efficient LLM Pre-training with SparseLoCo" (summary and
 *   abstract): Top-k sparsification, 2-bit codes and error feedback, and the sparse
 *   aggregation of the nodes' sparse updates.
 *
 * The pages hand the method a flattened gradient (the FSDP communication hook) and
 * keep the error local to each node; the exchange between nodes is not part of this
 * library.  A rank calls loco_compensate_quantize on its flat gradient, split into
 * one segment per destination partition, sends each partition's payload
 * (codes + absmax) to its owner, and calls loco_dequant_reduce on the payloads it
 * receives.  loco_topk_quantize is the SparseLoCo-style mode and loco_sparse_aggregate
 * its receiving side.
 *
 * Conventions shared by every entry point
 *   - Device pointers are caller-owned device memory (e.g. PyTorch tensors) and must
 *     be 16-byte aligned; host arrays (segs, peers) are read during the call only.
 *   - The library allocates nothing and keeps no state between calls, apart from the
 *     compute-unit count of each device, read once and cached.  Every call is
 *     asynchronous on `stream` (a hipStream_t; NULL is the default stream) and runs on
 *     the calling thread's current device; buffers must stay alive until the stream has
 *     consumed them.
 *   - Arguments are validated on the host before anything is launched: a validation
 *     status (LOCO_ERR_INVALID, LOCO_ERR_ALIGN, LOCO_ERR_UNSUPPORTED) means nothing was
 *     launched and nothing was written.  LOCO_ERR_HIP means a kernel launch failed; a
 *     call that takes several launches (more than 32 segments, a short last Top-k
 *     chunk, or more chunks than one grid holds) may have enqueued the launches before
 *     it.  Device faults surface at the caller's next synchronisation, as for any HIP
 *     call.
 *   - Arithmetic: IEEE binary32, round to nearest even, no fused multiply-add, in
 *     the order stated below; bf16 stores round to nearest even.
 *   - Stateless and reentrant across host threads and streams.
 */
#ifndef LOCO_H
#define LOCO_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of gradients, errors and outputs.  LOCO_I8 is only an error type of
 * loco_compensate_quantize_ex: the paper's 8-bit error codes of a fixed scale s_e. */
typedef enum { LOCO_F32 = 0, LOCO_BF16 = 1, LOCO_I8 = 2 } loco_dtype_t;

/* Status codes: 0 ok, < 0 error (nothing launched, except as LOCO_ERR_HIP below). */
#define LOCO_OK 0
#define LOCO_ERR_INVALID (-1)     /* bad size, bits, block, k, chunk, beta, scale, dtype,
                                     peer count < 1, null pointer, or overlapping buffers */
#define LOCO_ERR_ALIGN (-2)       /* a device pointer is not 16-byte aligned */
#define LOCO_ERR_UNSUPPORTED (-3) /* valid but not built: bits not in {2,4,8}, block not
                                     in {64,128,256,512}, chunk not in
                                     {256,512,1024,2048,4096}, more than LOCO_MAX_PEERS
                                     peers */
#define LOCO_ERR_HIP (-4)         /* the HIP launch failed */

/* Largest number of peers one dequant-reduce call accepts. */
#define LOCO_MAX_PEERS 128

/*
 * One segment of a compensate-quantize call: a contiguous gradient range with its
 * own error buffer and payload.  Scale blocks restart at element 0 of every
 * segment, so each segment's payload is self-contained (one all2all partition,
 * LoCo Sec. 3.3).
 *   grad    device, n elements of grad_dtype (read)
 *   err     device, n elements of err_dtype (4, 2 or 1 bytes each), read and
 *           updated in place
 *   codes   device, ceil(n*bits/8) bytes (written); codes are two's complement,
 *           packed little end first (4 bits: element 2j in the low nibble of byte j;
 *           2 bits: element 4j+t at bits 2t of byte j); unused high bits of the last
 *           byte are 0
 *   absmax  device, ceil(n/block) floats (written): the block's max |h|; unused and
 *           may be NULL when fixed_scale > 0
 *   n       elements (>= 0; 0 is a no-op)
 * No buffer a call writes (the err, codes and absmax of any of its segments) may
 * overlap another buffer of the call; gradients are only read and may overlap each
 * other (LOCO_ERR_INVALID otherwise).
 */
typedef struct {
    const void* grad;
    void* err;
    uint8_t* codes;
    float* absmax;
    int64_t n;
} loco_cq_segment_t;

/*
 * loco_compensate_quantize - LoCo Sec. 3.1-3.2, Eqns. (1)-(5), fused in one pass.
 *
 * For every segment and every block of `block` elements (the last may be partial):
 *   h      = g + e                                  Eqn. (2), g and e widened to f32
 *   absmax = max |h| over the block
 *   step   = absmax / qmax,  inv = 1 / step         qmax = 2^(bits-1) - 1; both 0
 *                                                   when absmax == 0
 *   q      = clamp(rint(h * inv), -2^(bits-1), qmax) Eqns. (1),(3); ties to even
 *   r      = h - q * step                           Eqn. (4)
 *   e     <- beta * e + (1 - beta) * r              Eqn. (5); 1 - beta rounded to f32
 * and stores the packed q, the block absmax and the new e (bf16: round to nearest
 * even).  fixed_scale = s > 0 is Eqn. (1) as printed: inv = s and step = 1/s for
 * every element, and no absmax is written.
 *   segs        host array of nseg segments (nseg >= 0)
 *   grad_dtype  LOCO_F32 or LOCO_BF16 (all segments); err_dtype likewise
 *   bits        2, 4 or 8
 *   block       64, 128, 256 or 512 (ignored when fixed_scale > 0)
 *   beta        in [0, 1]
 *   fixed_scale 0 for per-block absmax scales, or a finite s > 0
 * g and e must be finite, and so must h = g + e; for NaN or infinite values the codes,
 * scales and error are unspecified (no fault).
 * Any number of segments is accepted (they are launched 32 at a time, in order).
 * err_dtype LOCO_I8 is refused here (LOCO_ERR_INVALID): it needs the error scale of
 * loco_compensate_quantize_ex.
 * Returns LOCO_OK or an error status.
 */
int loco_compensate_quantize(const loco_cq_segment_t* segs, int nseg,
                             loco_dtype_t grad_dtype, loco_dtype_t err_dtype,
                             int bits, int block, float beta, float fixed_scale,
                             void* stream);

/* Options of loco_compensate_quantize_ex (a host struct, read during the call). */
typedef struct {
    int bits;          /* 2, 4 or 8 */
    int block;         /* 64, 128, 256 or 512 (ignored when fixed_scale > 0) */
    float beta;        /* in [0, 1] */
    float fixed_scale; /* 0, or a finite s > 0 */
    float err_scale;   /* s_e of an 8-bit error (err_dtype LOCO_I8); ignored otherwise */
    int reset_error;   /* nonzero: this step stores e = 0 */
} loco_cq_options_t;

/*
 * loco_compensate_quantize_ex - loco_compensate_quantize plus LoCo Sec. 3.2, Eqn. (7):
 * the compensation error kept in 8 bits, and its periodic reset.
 *
 * Same segments, arithmetic and outputs as loco_compensate_quantize, with:
 *   err_dtype LOCO_I8: err holds n int8 codes e8 of the scale s_e = err_scale, which
 *     must be finite, > 0, with 256 / s_e finite.  On load e = e8 * fl(1 / s_e) (the
 *     decompressor of Eqn. (1) with the error's own scale); on store
 *     e8 <- clamp(rint(e * s_e), -128, 127), ties to even (Eqn. (7)).
 *   reset_error != 0: the codes and absmax are those of h = g + e as usual, but the
 *     stored error is 0 (Eqn. (7) resets the error every T_c steps; the caller
 *     passes reset_error on those steps).  Any err_dtype.
 * Returns LOCO_OK or an error status (LOCO_ERR_INVALID for a NULL opt).
 */
int loco_compensate_quantize_ex(const loco_cq_segment_t* segs, int nseg,
                                loco_dtype_t grad_dtype, loco_dtype_t err_dtype,
                                const loco_cq_options_t* opt, void* stream);

/* One peer's payload for a partition: what loco_compensate_quantize wrote. */
typedef struct {
    const uint8_t* codes;  /* device, ceil(n*bits/8) bytes */
    const float* absmax;   /* device, ceil(n/block) floats; may be NULL when fixed_scale > 0 */
} loco_payload_t;

/*
 * loco_dequant_reduce - LoCo Sec. 3.3, Eqn. (8): decompress and average the N peers'
 * low-bit payloads of one partition, in high precision.
 *
 * For every element i:
 *   acc = 0;  for p = 0 .. npeers-1 in order:  acc = acc + q_p[i] * step_p
 *   out[i] = acc * out_scale                      (out_scale = 1/N for the average)
 * with step_p = absmax_p[block of i] / qmax (0 for an all-zero block), or 1/s in
 * fixed-scale mode.  The accumulator lives in registers; bf16 output rounds to
 * nearest even.  Every product and sum is the IEEE fp32 result for any absmax value,
 * up to FLT_MAX and including inf and NaN (a tile whose step is 2^100 or more, or not
 * finite, takes a slower element-wise path).
 *   peers      host array of npeers payloads, 1 <= npeers <= LOCO_MAX_PEERS
 *   n          elements of the partition (>= 0; 0 is a no-op)
 *   bits       2, 4 or 8;  block  64, 128, 256 or 512 (ignored when fixed_scale > 0)
 *   fixed_scale 0, or the s the payloads were made with
 *   out_scale  finite
 *   out        device, n elements of out_dtype (written); must not overlap a payload
 *   out_dtype  LOCO_F32 or LOCO_BF16
 */
int loco_dequant_reduce(const loco_payload_t* peers, int npeers, int64_t n,
                        int bits, int block, float fixed_scale, float out_scale,
                        void* out, loco_dtype_t out_dtype, void* stream);

/* Hyper-parameters of the LoCo-Adam step (host struct, read during the call). */
typedef struct {
    float lr;     /* learning rate eta, finite */
    float beta1;  /* weight of the new gradient in m, in [0, 1] (the page's typical 0.1) */
    float beta2;  /* weight of the new squared gradient in v, in [0, 1] (typical 0.001-0.05) */
    float delta;  /* finite, > 0: added to v under the square root */
} loco_adam_t;

/*
 * loco_dequant_reduce_adam - LoCo Sec. 3.3 Eqn. (8) fused with Sec. 4 Eqn. (9): the
 * peers' payloads are averaged exactly as loco_dequant_reduce does (fp32, peer order,
 * times out_scale; never rounded to bf16), and the average g drives one Adam-family
 * step on the partition's fp32 weights and moments, in one pass:
 *   m     <- (1 - beta1) * m + beta1 * g              (1 - beta rounded to f32 first)
 *   v     <- (1 - beta2) * v + beta2 * (g * g)
 *   u      = 1 / sqrt(v + delta)                      (correctly rounded sqrt and divide)
 *   param <- param - lr * (m * u)
 * in that order of roundings, with no bias correction or weight decay (the page names
 * neither); m and v start at 0 (the caller zeroes them).  The reduced gradient is not
 * written anywhere.
 *   peers, npeers, n, bits, block, fixed_scale, out_scale: as loco_dequant_reduce
 *   adam        host pointer to the hyper-parameters
 *   param, m, v device f32[n] each, read and updated in place
 *   param_bf16  device u16[n] (written: the RNE bf16 copy of the new param), or NULL
 * None of param, m, v, param_bf16 may overlap each other or a payload.
 */
int loco_dequant_reduce_adam(const loco_payload_t* peers, int npeers, int64_t n,
                             int bits, int block, float fixed_scale, float out_scale,
                             const loco_adam_t* adam, float* param, float* m, float* v,
                             uint16_t* param_bf16, void* stream);

/*
 * loco_topk_quantize - SparseLoCo-style per-chunk Top-k with low-bit codes and error
 * feedback ("Communication Efficient LLM Pre-training with SparseLoCo").
 *
 * For every chunk c of `chunk` elements (the last may be short; it keeps
 * keff = min(k, its length)):
 *   h  = g + ef_decay * e
 *   keep the keff elements with the largest |h| (compared as the bit pattern of
 *   |h|), ties to the lower index
 *   absmax = max |h| over the kept values; step = absmax / qmax; inv = 1 / step
 *   (both 0 if absmax == 0); q = clamp(rint(h * inv), -2^(bits-1), qmax)
 *   e <- h - q * step on the kept elements, e <- h elsewhere
 *   grad     device f32[n] (read);  err  device f32[n] (read and updated in place)
 *   n        elements (>= 0; 0 is a no-op)
 *   chunk    256, 512, 1024, 2048 or 4096;  1 <= k <= chunk
 *   bits     2, 4 or 8;  ef_decay in [0, 1]
 *   idx      device u16[chunks * k]: chunk-local indices of the kept elements,
 *            ascending; unused slots 0xFFFF
 *   codes    device u8[chunks * ceil(k*bits/8)]: the kept codes in index order,
 *            packed as in loco_cq_segment_t; unused slots 0
 *   absmax   device f32[chunks]
 * where chunks = ceil(n / chunk).  No two buffers may overlap.
 */
int loco_topk_quantize(const float* grad, float* err, int64_t n, int chunk, int k,
                       int bits, float ef_decay, uint16_t* idx, uint8_t* codes,
                       float* absmax, void* stream);

/* One peer's Top-k payload of a shard: what loco_topk_quantize wrote. */
typedef struct {
    const uint16_t* idx;   /* device u16[chunks * k] */
    const uint8_t* codes;  /* device u8[chunks * ceil(k*bits/8)] */
    const float* absmax;   /* device f32[chunks] */
} loco_sparse_payload_t;

/*
 * loco_sparse_aggregate - SparseLoCo's sparse aggregation ("Communication Efficient LLM
 * Pre-training with SparseLoCo", summary and abstract) of the peers' Top-k payloads of
 * one shard into a dense output, computed as the high-precision average of LoCo
 * Sec. 3.3, Eqn. (8) over sparse vectors.
 *
 * For every element i:
 *   acc = 0;  for p = 0 .. npeers-1 in order: if peer p's chunk c = i / chunk has a
 *   used slot j with idx_p[c*k + j] == i - c*chunk:  acc = acc + q_p[c, j] * step_p[c]
 *   out[i] = acc * out_scale                      (out_scale = 1/N for the average)
 * with step_p[c] = absmax_p[c] / qmax (0 for an all-zero chunk).  A slot is used when
 * its index lies inside its chunk (the last chunk may be short); other slots, such as
 * the 0xFFFF that loco_topk_quantize writes in unused slots, are skipped.  Elements no
 * peer names are 0.  The slots of one peer's chunk must name distinct elements (as
 * loco_topk_quantize writes them); repeated ones give an unspecified sum of their
 * values but never touch memory outside the output.  The accumulator is fp32; bf16
 * output rounds to nearest even.
 *   peers      host array of npeers payloads, 1 <= npeers <= LOCO_MAX_PEERS
 *   n          elements of the shard (>= 0; 0 is a no-op)
 *   chunk      256, 512, 1024, 2048 or 4096;  1 <= k <= chunk;  bits 2, 4 or 8
 *   out_scale  finite
 *   out        device, n elements of out_dtype (written); must not overlap a payload
 *   out_dtype  LOCO_F32 or LOCO_BF16
 * where chunks = ceil(n / chunk).
 */
int loco_sparse_aggregate(const loco_sparse_payload_t* peers, int npeers, int64_t n,
                          int chunk, int k, int bits, float out_scale, void* out,
                          loco_dtype_t out_dtype, void* stream);

/* A static, human-readable name for a status code. */
const char* loco_status_string(int status);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int loco_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LOCO_H */
