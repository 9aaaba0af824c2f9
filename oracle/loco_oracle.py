"""Plain CPU oracle for LoCo's per-GPU gradient path and its SparseLoCo-style mode.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links this
module: only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may use it.  It shares no code, table or helper with the HIP kernels.

Sources (cited by page title and section; the equation bodies are missing from the
extracted text, so each step below is rebuilt from the prose around the equation):

* "LoCo: Low-Bit Communication Adaptor for Large-scale Model Training"
  (arXiv 2407.04480, HTML body):
    - Sec. 3.1, Eqn. (1): element-wise compressor, round to the nearest integer
      inside [-2^(p-1), 2^(p-1)-1]; the decompressor undoes the scale.
    - Sec. 3.1, Eqn. (2): compensation, the error is added to the gradient.
    - Sec. 3.1, Eqn. (3): the compensated gradient is compressed to 4 bits.
    - Sec. 3.2, Eqn. (4): the compression error is compensated value minus its
      decompressed low-bit version.
    - Sec. 3.2, Eqn. (5): the error is a beta-weighted moving average of the
      historical compression errors, starting from zero.
    - Sec. 3.2, Eqn. (7): the error is kept as 8-bit codes of a fixed scale s_e
      (the compressor of Eqn. (1) with 8 bits), and reset to zero every T_c steps.
    - Sec. 3.3, Eqn. (8): the synchronised gradient is the average over the N nodes
      of the decompressed low-bit gradients, computed in high precision; with FSDP
      each node averages only its own partition (all2all, then a local average).
    - Sec. 4, Eqn. (9): the Adam-family step on the synchronised gradient: moving
      averages m (weight beta1 on the new gradient, m_0 = 0) and v (weight beta2 on
      its square, v_0 = 0), the pre-conditioner 1 / sqrt(v + delta), and the update
      of the weights by the learning rate times the pre-conditioned m.
* "Communication Efficient LLM Pre-training with SparseLoCo" (summary and
  abstract): Top-k sparsification, 2-bit quantisation and error feedback, and a
  sparse aggregation of the nodes' sparse updates.

Readings where the pages are silent (each is also listed in the design notes):
* per-block absmax scale: the stored scale is the block's max |h| (exact); the
  dequantisation step is fl(absmax / qmax) and quantisation multiplies by the
  explicit reciprocal fl(1 / step).  Where that reciprocal is not finite (an
  all-zero block, or a block whose absmax is below ~qmax * 2^-128, where 1/step
  overflows fp32) inv = 0: the block is sent as zero codes and stays in the error.
* "nearest integer" ties go to even (PyTorch's default quantiser does this).
* the moving average is e' = beta * e + (1 - beta) * r with r = h - d.
* every floating-point value is one IEEE binary32 operation (round to nearest
  even, no fused multiply-add) in the order written below.
* SparseLoCo: per-chunk Top-k by |h| (compared as the bit pattern of |h|), ties to
  the lower index; the kept values get codes of the same quantiser with b = 2 and
  the chunk's absmax; error feedback h = g + decay * e, e' = h - transmitted.
* SparseLoCo's sparse aggregation: the high-precision average of LoCo Eqn. (8)
  applied to the peers' sparse payloads (each scattered into a dense zero vector),
  accumulated in peer order.
* LoCo-Adam (Eqn. (9)): m' = (1 - beta1) m + beta1 g (the v recursion is printed;
  m follows it by analogy), no bias correction and no weight decay (the page names
  neither), theta' = theta - lr * (m' * u) with u = 1 / sqrt(v' + delta).

Parity unpinned: where the pages leave the form open, only the readings above
decide it: the form of the moving average (Eqn. (5)), the 2-bit codebook, the
SparseLoCo error-feedback decay, the form of the sparse aggregation, and the m
recursion and update order of the Adam-family step (Eqn. (9)).  The tests pin
every function to closed forms, bounds and worked examples under these readings;
the pages cannot choose between the readings.

The functions are generic over the float type of their inputs: called with
float32 arrays they are the parity oracle; called with float64 arrays they are
the real-arithmetic twin used by the telescoping check.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_rne", "bf16_to_f32", "widen", "qmax_of", "finite_reciprocal",
    "compensate", "absmax_quantize", "fixed_scale_quantize", "dequantize",
    "error_update", "error_decompress", "error_compress", "pack_codes", "unpack_codes",
    "compensate_quantize",
    "cq_algorithmic_bytes", "block_steps", "dequant_reduce", "dr_algorithmic_bytes",
    "adam_step", "dequant_reduce_adam", "dra_algorithmic_bytes",
    "topk_order_select", "topk_quantize", "tk_algorithmic_bytes",
    "sparse_aggregate", "sa_algorithmic_bytes",
]


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def bf16_rne(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    Finite inputs only (NaN/Inf are outside the contract).  Adds 0x7FFF plus the
    lowest kept bit, then drops the low 16 bits.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return (u >> np.uint64(16)).astype(np.uint16)


def bf16_to_f32(u: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32, exact."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def widen(x: np.ndarray, dtype: str, ftype=np.float32) -> np.ndarray:
    """Load a stored gradient/error as the working float type.

    dtype: 'bf16' (uint16 patterns), 'f32', or 'f64' (the real-arithmetic twin).
    """
    if dtype == "bf16":
        return bf16_to_f32(x).astype(ftype)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(ftype)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64).astype(ftype)
    raise ValueError(dtype)


def qmax_of(bits: int) -> int:
    """Largest positive code, 2^(b-1) - 1 (LoCo Sec. 3.1, Eqn. (1) range)."""
    return (1 << (bits - 1)) - 1


# ---------------------------------------------------------------------------
# LoCo, Sec. 3.1 - 3.2
# ---------------------------------------------------------------------------

def compensate(g: np.ndarray, e: np.ndarray) -> np.ndarray:
    """Eqn. (2): the compensated gradient h = g + e (e already in float form)."""
    return g + e


def _blocks(h: np.ndarray, block: int):
    n = h.size
    nb = -(-n // block)
    pad = np.zeros(nb * block, dtype=h.dtype)
    pad[:n] = h
    return pad.reshape(nb, block), nb


def absmax_quantize(h: np.ndarray, bits: int, block: int):
    """Eqn. (1) with a per-block absmax scale instead of the paper's global s.

    Blocks tile h from element 0; the last block may be partial (its padding is
    zero, which cannot change a max of absolute values).  step = fl(absmax / qmax),
    inv = fl(1 / step), q = clamp(rint(fl(h * inv))).  A block whose reciprocal is
    not finite (an all-zero block, or one so small that 1/step overflows) gets
    inv = 0: its codes are 0 and its values stay whole in the error.  Returns
    (q int64[n], absmax[nb], step[nb]) in h's float type.
    """
    ft = h.dtype.type
    qmax = qmax_of(bits)
    hb, nb = _blocks(h, block)
    absmax = np.max(np.abs(hb), axis=1)
    step = absmax / ft(qmax)
    inv = finite_reciprocal(step)
    scaled = hb * inv[:, None]
    q = np.clip(np.rint(scaled), -(qmax + 1), qmax).astype(np.int64)
    return q.reshape(-1)[: h.size], absmax, step


def finite_reciprocal(step: np.ndarray) -> np.ndarray:
    """inv = fl(1 / step), or 0 where that is not finite.

    step >= 0.  The reciprocal is +inf for step = 0 (an all-zero block) and for a step
    below about 2^-128 in fp32, where 1/step exceeds the largest finite float.  Such a
    block cannot be scaled into the code range, so it is sent as zero codes (inv = 0
    makes every q = 0) and the error feedback keeps its values.
    """
    step = np.asarray(step)
    with np.errstate(divide="ignore", over="ignore"):
        inv = step.dtype.type(1) / step
    return np.where(np.isfinite(inv), inv, step.dtype.type(0)).astype(step.dtype)


def fixed_scale_quantize(h: np.ndarray, bits: int, s: float):
    """Eqn. (1) as printed: Round_b(s * h), with one global scale s > 0.

    Returns (q int64[n], step) with step = fl(1 / s) the decompressor's factor.
    """
    ft = h.dtype.type
    qmax = qmax_of(bits)
    q = np.clip(np.rint(h * ft(s)), -(qmax + 1), qmax).astype(np.int64)
    return q, ft(1) / ft(s)


def dequantize(q: np.ndarray, step_per_elem: np.ndarray) -> np.ndarray:
    """Decompressor of Eqn. (1): d = q * step."""
    return q.astype(step_per_elem.dtype) * step_per_elem


def error_update(e: np.ndarray, r: np.ndarray, beta: float) -> np.ndarray:
    """Eqn. (5), read as e' = beta * e + (1 - beta) * r, with r from Eqn. (4).

    beta = 0 gives the plain error-feedback error of Eqn. (4).  The weight on r is
    fl(1 - beta) in the working float type.
    """
    ft = e.dtype.type
    b = ft(beta)
    w = ft(1) - b
    return b * e + w * r


def pack_codes(q: np.ndarray, bits: int) -> np.ndarray:
    """Pack signed codes, two's complement, little end first.

    8 bits: one int8 per code.  4 bits: byte j holds code 2j in its low nibble and
    code 2j+1 in its high nibble.  2 bits: byte j holds code 4j+t at bits 2t.
    The unused high part of the last byte is zero.
    """
    q = np.asarray(q, dtype=np.int64)
    if bits == 8:
        return (q & 0xFF).astype(np.uint8)
    per = 8 // bits
    mask = (1 << bits) - 1
    nbytes = -(-q.size * bits // 8)
    u = np.zeros(nbytes * per, dtype=np.int64)
    u[: q.size] = q & mask
    u = u.reshape(nbytes, per)
    out = np.zeros(nbytes, dtype=np.int64)
    for t in range(per):
        out |= u[:, t] << (bits * t)
    return out.astype(np.uint8)


def unpack_codes(packed: np.ndarray, bits: int, n: int) -> np.ndarray:
    """Inverse of pack_codes, with sign extension; returns int64[n]."""
    p = np.asarray(packed, dtype=np.uint8).astype(np.int64)
    per = 8 // bits
    mask = (1 << bits) - 1
    fields = np.stack([(p >> (bits * t)) & mask for t in range(per)], axis=1).reshape(-1)[:n]
    return np.where(fields >= (1 << (bits - 1)), fields - (1 << bits), fields)


def _absmax_compressor(bits, block, fixed_scale):
    def comp(h):
        if fixed_scale > 0:
            q, step = fixed_scale_quantize(h, bits, fixed_scale)
            d = dequantize(q, np.full(h.size, step, dtype=h.dtype))
            return d, {"q": q, "absmax": None, "step": step}
        q, absmax, step = absmax_quantize(h, bits, block)
        d = dequantize(q, np.repeat(step, block)[: h.size])
        return d, {"q": q, "absmax": absmax, "step": step}
    return comp


def error_decompress(e8: np.ndarray, s_e: float, ftype=np.float32) -> np.ndarray:
    """The 8-bit error as a float (LoCo Sec. 3.1, Eqn. (2)): e8 * fl(1 / s_e), the
    decompressor of Eqn. (1) with the error's own scale."""
    return np.asarray(e8, dtype=np.int8).astype(ftype) * (ftype(1) / ftype(s_e))


def error_compress(e_tilde: np.ndarray, s_e: float) -> np.ndarray:
    """LoCo Sec. 3.2, Eqn. (7): compressor(e~; s_e, 8) = Round_8(s_e * e~), nearest
    integer (ties to even) inside [-128, 127]."""
    ft = e_tilde.dtype.type
    return np.clip(np.rint(e_tilde * ft(s_e)), -128, 127).astype(np.int8)


def compensate_quantize(g, e, *, bits, block, beta, fixed_scale=0.0,
                        grad_dtype="f32", err_dtype="f32", ftype=np.float32,
                        compressor=None, err_scale=0.0, reset=False):
    """One LoCo step on one segment (LoCo Sec. 3.1 - 3.2, Eqns. (2) - (5), (7)).

    g, e: stored gradient and error (float32 arrays, uint16 bf16 patterns when the dtype
    says 'bf16', int8 codes of the paper's 8-bit error when err_dtype is 'i8', whose
    scale s_e is `err_scale`).  `reset` is the periodic reset of Eqn. (7): this step
    stores e = 0.  Returns a dict with
      codes   packed payload bytes (ceil(n*bits/8))       [compressor output]
      absmax  float per block (None in fixed-scale mode)
      e_new   the updated error in its storage format
      d       the decompressed transmitted value (working float type)
      q       the integer codes
    `compressor` replaces the quantiser (h -> (d, info)); used by the
    identity-compressor check.
    """
    gf = widen(g, grad_dtype, ftype)
    if err_dtype == "i8":
        if not err_scale > 0:
            raise ValueError("an 8-bit error needs its scale s_e > 0")
        ef = error_decompress(e, err_scale, ftype)
    else:
        ef = widen(e, err_dtype, ftype)
    h = compensate(gf, ef)
    comp = compressor or _absmax_compressor(bits, block, fixed_scale)
    d, info = comp(h)
    r = h - d
    e_new = error_update(ef, r, beta)
    if reset:
        e_new = np.zeros_like(e_new)
    if err_dtype == "bf16":
        e_store = bf16_rne(e_new.astype(np.float32))
    elif err_dtype == "i8":
        e_store = error_compress(e_new, err_scale)
    else:
        e_store = e_new.astype(ftype)
    out = {"d": d, "e_new": e_store, "q": info.get("q"), "absmax": info.get("absmax")}
    if info.get("q") is not None:
        out["codes"] = pack_codes(info["q"], bits)
    return out


def cq_algorithmic_bytes(n, grad_bytes, err_bytes, bits, block, fixed_scale=False):
    """Bytes one compensate-quantize call must move: read g and e, write e, codes, scales."""
    scales = 0 if fixed_scale else 4 * (-(-n // block))
    return n * (grad_bytes + 2 * err_bytes) + (-(-n * bits // 8)) + scales


# ---------------------------------------------------------------------------
# LoCo, Sec. 3.3: average of the peers' decompressed partitions
# ---------------------------------------------------------------------------

def block_steps(absmax: np.ndarray, bits: int) -> np.ndarray:
    """Decoder side: step = fl(absmax / qmax), 0 for an all-zero block."""
    absmax = np.asarray(absmax)
    ft = absmax.dtype.type
    step = np.zeros_like(absmax)
    np.divide(absmax, ft(qmax_of(bits)), out=step, where=absmax != 0)
    return step


def dequant_reduce(payloads, n, *, bits, block, out_scale, out_dtype="f32",
                   fixed_scale=0.0, ftype=np.float32):
    """Eqn. (8) on one partition: acc = sum over peers p = 0..N-1 (in that order)
    of q_p * step_p, then out = acc * out_scale (out_scale = 1/N for the average).

    payloads: list of (codes uint8, absmax float32 or None).  Returns float32 or
    bf16 patterns (uint16).
    """
    acc = np.zeros(n, dtype=ftype)
    for codes, absmax in payloads:
        q = unpack_codes(codes, bits, n)
        if fixed_scale > 0:
            step_e = np.full(n, ftype(1) / ftype(fixed_scale), dtype=ftype)
        else:
            step_e = np.repeat(block_steps(np.asarray(absmax, dtype=ftype), bits), block)[:n]
        acc = acc + dequantize(q, step_e)
    out = acc * ftype(out_scale)
    if out_dtype == "bf16":
        return bf16_rne(out.astype(np.float32))
    return out


def adam_step(theta, m, v, g, *, lr, beta1, beta2, delta, ftype=np.float32):
    """LoCo Sec. 4, Eqn. (9), the Adam family with Adam's pre-conditioner, on the
    synchronised gradient g:
      m' = (1 - beta1) * m + beta1 * g
      v' = (1 - beta2) * v + beta2 * (g * g)
      u  = 1 / sqrt(v' + delta)
      theta' = theta - lr * (m' * u)
    Every operation is one IEEE rounding in the working type, in the order written
    (1 - beta rounded first, as in error_update).  Returns (theta', m', v').
    """
    ft = ftype
    theta, m, v, g = (np.asarray(x, dtype=ft) for x in (theta, m, v, g))
    b1, b2 = ft(beta1), ft(beta2)
    m_new = (ft(1) - b1) * m + b1 * g
    v_new = (ft(1) - b2) * v + b2 * (g * g)
    u = ft(1) / np.sqrt(v_new + ft(delta))
    theta_new = theta - ft(lr) * (m_new * u)
    return theta_new, m_new, v_new


def dequant_reduce_adam(payloads, n, *, bits, block, out_scale, theta, m, v, lr, beta1, beta2, delta,
                        fixed_scale=0.0, ftype=np.float32):
    """Eqn. (8) then Eqn. (9) on one partition: the peers' payloads are averaged in
    high precision (dequant_reduce, fp32, never rounded to bf16) and the result is the
    gradient of one Adam-family step.  Returns dict(theta, m, v, g, theta_bf16) with
    theta_bf16 the RNE bf16 copy of the new weights."""
    g = dequant_reduce(payloads, n, bits=bits, block=block, out_scale=out_scale, out_dtype="f32",
                       fixed_scale=fixed_scale, ftype=ftype)
    theta_new, m_new, v_new = adam_step(theta, m, v, g, lr=lr, beta1=beta1, beta2=beta2, delta=delta,
                                        ftype=ftype)
    return {"theta": theta_new, "m": m_new, "v": v_new, "g": g,
            "theta_bf16": bf16_rne(np.asarray(theta_new, np.float32))}


def dra_algorithmic_bytes(n, npeers, bits, block, param_bf16=False, fixed_scale=False):
    """Peer payloads read once; theta, m, v (fp32) read and written; optional bf16 copy."""
    return dr_algorithmic_bytes(n, npeers, bits, block, 0, fixed_scale) + 24 * n + (2 * n if param_bf16 else 0)


def dr_algorithmic_bytes(n, npeers, bits, block, out_bytes, fixed_scale=False):
    scales = 0 if fixed_scale else 4 * (-(-n // block))
    return npeers * ((-(-n * bits // 8)) + scales) + n * out_bytes


# ---------------------------------------------------------------------------
# SparseLoCo mode: per-chunk Top-k, low-bit codes, error feedback
# ---------------------------------------------------------------------------

def topk_order_select(key: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest keys, ties to the lower index, returned ascending.

    A stable sort of -key puts equal keys in index order; the first k are kept.
    """
    key = np.asarray(key)
    neg = -(key.astype(np.int64)) if key.dtype.kind in "ui" else -key
    order = np.argsort(neg, kind="stable")
    return np.sort(order[:k])


def topk_quantize(g, e, *, chunk, k, bits=2, decay=1.0, ftype=np.float32):
    """SparseLoCo-style step on a flat fp32 pseudo-gradient.

    Per chunk of `chunk` elements (the last may be short; it keeps min(k, len)):
      h = g + decay * e                 error feedback
      select the k largest |h| (bit pattern of |h|; ties to the lower index)
      absmax over the kept values; step = absmax / qmax; inv = 1 / step, or 0
      where that is not finite (absmax 0, or below ~2^-128 * qmax)
      q = clamp(rint(h * inv)) on the kept values
      e' = h - q * step on the kept values, e' = h elsewhere
    Returns dict(idx uint16[chunks*k] (unused slots 0xFFFF), codes
    uint8[chunks*ceil(k*bits/8)], absmax float32[chunks], e_new, h).
    """
    g = np.asarray(g, dtype=ftype)
    e = np.asarray(e, dtype=ftype)
    h = g + ftype(decay) * e
    n = h.size
    nchunks = -(-n // chunk)
    cbytes = -(-k * bits // 8)
    qmax = qmax_of(bits)
    idx_out = np.full((nchunks, k), 0xFFFF, dtype=np.uint16)
    codes_out = np.zeros((nchunks, cbytes), dtype=np.uint8)
    absmax_out = np.zeros(nchunks, dtype=ftype)
    e_new = h.copy()
    for c in range(nchunks):
        lo, hi = c * chunk, min(n, (c + 1) * chunk)
        hc = h[lo:hi]
        keff = min(k, hi - lo)
        key = np.abs(hc.astype(np.float32)).view(np.uint32) if ftype is np.float32 else np.abs(hc)
        sel = topk_order_select(key, keff)
        vals = hc[sel]
        absmax = np.max(np.abs(vals))
        step = absmax / ftype(qmax)
        inv = finite_reciprocal(np.array([step], dtype=ftype))[0]
        q = np.clip(np.rint(vals * inv), -(qmax + 1), qmax).astype(np.int64)
        d = q.astype(ftype) * step
        e_new[lo + sel] = vals - d
        idx_out[c, :keff] = sel.astype(np.uint16)
        codes_out[c] = pack_codes(np.concatenate([q, np.zeros(k - keff, np.int64)]), bits)
        absmax_out[c] = absmax
    return {"idx": idx_out.reshape(-1), "codes": codes_out.reshape(-1),
            "absmax": absmax_out, "e_new": e_new, "h": h}


def sparse_aggregate(payloads, n, *, chunk, k, bits, out_scale, out_dtype="f32", ftype=np.float32):
    """SparseLoCo's sparse aggregation of the peers' Top-k payloads (summary and
    abstract), read as the high-precision average of LoCo Sec. 3.3, Eqn. (8) over
    sparse vectors:
      acc = 0
      for p = 0 .. N-1 (in that order), for every chunk c and used slot j of peer p:
          acc[c*chunk + idx_p[c, j]] = acc[...] + q_p[c, j] * step_p[c]
      out = acc * out_scale
    with step_p[c] = absmax_p[c] / qmax (0 when absmax is 0).  A slot is used when
    its index lies inside its chunk (the last chunk may be short); unused slots hold
    0xFFFF.  The slots of one peer's chunk name distinct elements.

    payloads: list of (idx uint16[chunks*k], codes uint8[chunks*ceil(k*bits/8)],
    absmax float32[chunks]), as topk_quantize writes them.  Returns float32 or bf16
    patterns (uint16).
    """
    nchunks = -(-n // chunk)
    cbytes = -(-k * bits // 8)
    per = 8 // bits
    base = np.arange(nchunks, dtype=np.int64)[:, None] * chunk
    length = np.minimum(chunk, n - base)
    acc = np.zeros(n, dtype=ftype)
    for idx, codes, absmax in payloads:
        ix = np.asarray(idx, dtype=np.uint16).reshape(nchunks, k).astype(np.int64)
        rows = np.asarray(codes, dtype=np.uint8).reshape(nchunks, cbytes)
        # each chunk's codes start on a byte of their own: unpack row by row
        q = unpack_codes(rows.reshape(-1), bits, nchunks * cbytes * per).reshape(nchunks, -1)[:, :k]
        step = block_steps(np.asarray(absmax, dtype=ftype), bits)
        d = dequantize(q, np.repeat(step, k).reshape(nchunks, k))
        used = ix < length
        pos = (base + ix)[used]
        acc[pos] = acc[pos] + d[used]
    out = acc * ftype(out_scale)
    if out_dtype == "bf16":
        return bf16_rne(out.astype(np.float32))
    return out


def sa_algorithmic_bytes(n, npeers, chunk, k, bits, out_bytes):
    chunks = -(-n // chunk)
    return npeers * chunks * (2 * k + (-(-k * bits // 8)) + 4) + n * out_bytes


def tk_algorithmic_bytes(n, chunk, k, bits=2):
    chunks = -(-n // chunk)
    return n * (4 + 2 * 4) + chunks * (2 * k + (-(-k * bits // 8)) + 4)
