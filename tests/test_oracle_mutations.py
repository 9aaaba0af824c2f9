"""Plant plausible mistakes in the CPU oracle and check that some pin catches each.

This shows the pins are strong enough: a dropped term, a wrong sign, a swapped
weight, an off-by-one block, the wrong rounding or tie rule, a swapped nibble order
or a missing sign extension must each fail at least one pin.  Mistakes are planted
only in the oracle, on the CPU.
"""
import numpy as np
import pytest

import oracle
import oracle_pins

O = oracle.loco_oracle
_orig = {name: getattr(O, name) for name in dir(O) if not name.startswith("__")}


def _drop_beta_term(e, r, beta):
    ft = e.dtype.type
    return (ft(1) - ft(beta)) * r


def _swap_weights(e, r, beta):
    ft = e.dtype.type
    return (ft(1) - ft(beta)) * e + ft(beta) * r


def _compensate_minus(g, e):
    return g - e


def _floor_quantise(h, bits, block):
    q, absmax, step = _orig["absmax_quantize"](h, bits, block)
    hb, nb = _orig["_blocks"](h, block)
    inv = np.zeros(nb, h.dtype)
    np.divide(h.dtype.type(1), step, out=inv, where=step != 0)
    qmax = (1 << (bits - 1)) - 1
    qf = np.clip(np.floor(hb * inv[:, None]), -qmax - 1, qmax).astype(np.int64)
    return qf.reshape(-1)[: h.size], absmax, step


def _half_away_quantise(h, bits, block):
    q, absmax, step = _orig["absmax_quantize"](h, bits, block)
    hb, nb = _orig["_blocks"](h, block)
    inv = np.zeros(nb, h.dtype)
    np.divide(h.dtype.type(1), step, out=inv, where=step != 0)
    x = hb * inv[:, None]
    qmax = (1 << (bits - 1)) - 1
    qa = np.clip(np.sign(x) * np.floor(np.abs(x) + h.dtype.type(0.5)), -qmax - 1, qmax)
    return qa.astype(np.int64).reshape(-1)[: h.size], absmax, step


def _shifted_block(h, bits, block):
    q, absmax, step = _orig["absmax_quantize"](np.roll(h, 1), bits, block)
    return np.roll(q, -1), absmax, step


def _divide_not_reciprocal(h, bits, block):
    hb, nb = _orig["_blocks"](h, block)
    qmax = (1 << (bits - 1)) - 1
    absmax = np.max(np.abs(hb), axis=1)
    step = np.zeros(nb, h.dtype)
    np.divide(absmax, h.dtype.type(qmax), out=step, where=absmax != 0)
    x = np.zeros_like(hb)
    np.divide(hb, step[:, None], out=x, where=step[:, None] != 0)
    q = np.clip(np.rint(x), -qmax - 1, qmax).astype(np.int64)
    return q.reshape(-1)[: h.size], absmax, step


def _dequantize_no_step(q, step):
    return q.astype(step.dtype)


def _dequantize_neg(q, step):
    return -(q.astype(step.dtype) * step)


def _ties_high(key, k):
    key = np.asarray(key)
    neg = -(key.astype(np.int64)) if key.dtype.kind in "ui" else -key
    order = np.argsort(neg[::-1], kind="stable")
    return np.sort((key.size - 1 - order)[:k])


def _pack_swapped(q, bits):
    p = _orig["pack_codes"](q, bits)
    if bits == 4:
        return ((p >> 4) | (p << 4)).astype(np.uint8)
    return p


def _unpack_unsigned(packed, bits, n):
    p = np.asarray(packed, dtype=np.uint8).astype(np.int64)
    per = 8 // bits
    mask = (1 << bits) - 1
    return np.stack([(p >> (bits * t)) & mask for t in range(per)], axis=1).reshape(-1)[:n]


def _bf16_truncate(x):
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _steps_no_qmax(absmax, bits):
    return np.asarray(absmax).copy()


def _edecomp_times_scale(e8, s_e, ftype=np.float32):
    return np.asarray(e8, dtype=np.int8).astype(ftype) * ftype(s_e)


def _ecomp_floor(e_tilde, s_e):
    ft = e_tilde.dtype.type
    return np.clip(np.floor(e_tilde * ft(s_e)), -128, 127).astype(np.int8)


def _ecomp_no_clamp(e_tilde, s_e):
    ft = e_tilde.dtype.type
    return np.rint(e_tilde * ft(s_e)).astype(np.int64).astype(np.int8)


def _sa_reversed(payloads, n, **kw):
    return _orig["sparse_aggregate"](list(payloads)[::-1], n, **kw)


def _sa_no_scale(payloads, n, **kw):
    return _orig["sparse_aggregate"](payloads, n, **dict(kw, out_scale=1.0))


def _sa_index_plus_one(payloads, n, **kw):
    moved = []
    for idx, codes, absmax in payloads:
        ix = np.asarray(idx, np.uint16).copy()
        ix[ix != 0xFFFF] += 1
        moved.append((ix, codes, absmax))
    return _orig["sparse_aggregate"](moved, n, **kw)


def _sa_slot_scale(payloads, n, **kw):
    # every chunk decoded with the first chunk's scale
    out = []
    for idx, codes, absmax in payloads:
        a = np.asarray(absmax)
        out.append((idx, codes, np.resize(a[:1], a.shape) if a.size else a))
    return _orig["sparse_aggregate"](out, n, **kw)


def _adam_swapped(theta, m, v, g, *, lr, beta1, beta2, delta, ftype=np.float32):
    return _orig["adam_step"](theta, m, v, g, lr=lr, beta1=1 - beta1, beta2=beta2, delta=delta, ftype=ftype)


def _adam_delta_outside(theta, m, v, g, *, lr, beta1, beta2, delta, ftype=np.float32):
    ft = ftype
    theta, m, v, g = (np.asarray(x, dtype=ft) for x in (theta, m, v, g))
    m_new = (ft(1) - ft(beta1)) * m + ft(beta1) * g
    v_new = (ft(1) - ft(beta2)) * v + ft(beta2) * (g * g)
    return theta - ft(lr) * (m_new / (np.sqrt(v_new) + ft(delta))), m_new, v_new


def _adam_bias_corrected(theta, m, v, g, *, lr, beta1, beta2, delta, ftype=np.float32):
    ft = ftype
    theta, m, v, g = (np.asarray(x, dtype=ft) for x in (theta, m, v, g))
    m_new = (ft(1) - ft(beta1)) * m + ft(beta1) * g
    v_new = (ft(1) - ft(beta2)) * v + ft(beta2) * (g * g)
    mh, vh = m_new / ft(beta1), v_new / ft(beta2)  # first-step bias correction
    return theta - ft(lr) * (mh / np.sqrt(vh + ft(delta))), m_new, v_new


def _dra_bf16_gradient(payloads, n, **kw):
    # the averaged gradient rounded to bf16 before the step
    g = _orig["dequant_reduce"](payloads, n, bits=kw["bits"], block=kw["block"], out_scale=kw["out_scale"],
                                out_dtype="bf16", fixed_scale=kw.get("fixed_scale", 0.0))
    g = _orig["bf16_to_f32"](g)
    th, m, v = _orig["adam_step"](kw["theta"], kw["m"], kw["v"], g, lr=kw["lr"], beta1=kw["beta1"],
                                  beta2=kw["beta2"], delta=kw["delta"])
    return {"theta": th, "m": m, "v": v, "g": g, "theta_bf16": _orig["bf16_rne"](th)}


def _dra_scale_after(payloads, n, **kw):
    # the step taken on the peers' sum, out_scale applied to the update afterwards
    g = _orig["dequant_reduce"](payloads, n, bits=kw["bits"], block=kw["block"], out_scale=1.0,
                                fixed_scale=kw.get("fixed_scale", 0.0))
    th, m, v = _orig["adam_step"](kw["theta"], kw["m"], kw["v"], g, lr=kw["lr"] * kw["out_scale"],
                                  beta1=kw["beta1"], beta2=kw["beta2"], delta=kw["delta"])
    return {"theta": th, "m": m, "v": v, "g": g * np.float32(kw["out_scale"]), "theta_bf16": _orig["bf16_rne"](th)}


def _dra_copy_truncated(payloads, n, **kw):
    r = _orig["dequant_reduce_adam"](payloads, n, **kw)
    r["theta_bf16"] = _bf16_truncate(r["theta"])
    return r


def _recip_keeps_overflow(step):
    # only an all-zero block gets inv = 0; a tiny one keeps 1/step = inf
    step = np.asarray(step)
    with np.errstate(divide="ignore", over="ignore"):
        inv = step.dtype.type(1) / step
    return np.where(step != 0, inv, step.dtype.type(0)).astype(step.dtype)


def _recip_zero_subnormal(step):
    # inv = 0 for every subnormal step, even where 1/step is finite
    step = np.asarray(step)
    with np.errstate(divide="ignore", over="ignore"):
        inv = step.dtype.type(1) / step
    return np.where(step >= np.finfo(step.dtype).tiny, inv, step.dtype.type(0)).astype(step.dtype)


def _dequant_offset_form(q, step_per_elem):
    # q * step formed as (q + 8) * step - 8 * step, each product rounded
    ft = step_per_elem.dtype.type
    return (q + 8).astype(step_per_elem.dtype) * step_per_elem - ft(8) * step_per_elem


def _dr_reversed(payloads, n, **kw):
    return _orig["dequant_reduce"](list(reversed(payloads)), n, **kw)


def _tk_variant(bug):
    """topk_quantize with one planted mistake (written out here, the oracle untouched)."""
    def tk(g, e, *, chunk, k, bits=2, decay=1.0, ftype=np.float32):
        g = np.asarray(g, dtype=ftype)
        e = np.asarray(e, dtype=ftype)
        h = ftype(decay) * g + e if bug == "decay on g" else g + ftype(decay) * e
        n = h.size
        nchunks = -(-n // chunk)
        cbytes = -(-k * bits // 8)
        qmax = O.qmax_of(bits)
        idx_out = np.full((nchunks, k), 0xFFFF, dtype=np.uint16)
        codes_out = np.zeros((nchunks, cbytes), dtype=np.uint8)
        absmax_out = np.zeros(nchunks, dtype=ftype)
        e_new = h.copy()
        for c in range(nchunks):
            lo, hi = c * chunk, min(n, (c + 1) * chunk)
            hc = h[lo:hi]
            keff = min(k, hi - lo)
            src = g[lo:hi] if bug == "select by g" else hc
            key = np.abs(src.astype(np.float32)).view(np.uint32)
            sel = O.topk_order_select(key, keff)
            vals = hc[sel]
            absmax = np.max(np.abs(vals))
            step = absmax / ftype(qmax)
            inv = O.finite_reciprocal(np.array([step], dtype=ftype))[0]
            q = np.clip(np.rint(vals * inv), -(qmax + 1), qmax).astype(np.int64)
            d = q.astype(ftype) * step
            e_new[lo + sel] = vals if bug == "kept error not reduced" else vals - d
            if bug == "unselected error zeroed":
                rest = np.ones(hi - lo, bool)
                rest[sel] = False
                e_new[lo:hi][rest] = 0
            idx_out[c, :keff] = sel.astype(np.uint16)
            codes_out[c] = O.pack_codes(np.concatenate([q, np.zeros(k - keff, np.int64)]), bits)
            absmax_out[c] = absmax
        return {"idx": idx_out.reshape(-1), "codes": codes_out.reshape(-1),
                "absmax": absmax_out, "e_new": e_new, "h": h}
    return tk


def _adam_v_linear(theta, m, v, g, *, lr, beta1, beta2, delta, ftype=np.float32):
    ft = ftype
    theta, m, v, g = (np.asarray(x, dtype=ft) for x in (theta, m, v, g))
    b1, b2 = ft(beta1), ft(beta2)
    m_new = (ft(1) - b1) * m + b1 * g
    v_new = (ft(1) - b2) * v + b2 * np.abs(g)
    u = ft(1) / np.sqrt(v_new + ft(delta))
    return theta - ft(lr) * (m_new * u), m_new, v_new


MUTATIONS = {
    "error_update drops beta*e": ("error_update", _drop_beta_term),
    "error_update swaps beta and 1-beta": ("error_update", _swap_weights),
    "compensate subtracts e": ("compensate", _compensate_minus),
    "floor instead of rint": ("absmax_quantize", _floor_quantise),
    "ties away from zero": ("absmax_quantize", _half_away_quantise),
    "scale of the wrong block": ("absmax_quantize", _shifted_block),
    "divide instead of reciprocal-multiply": ("absmax_quantize", _divide_not_reciprocal),
    "decompressor drops step": ("dequantize", _dequantize_no_step),
    "decompressor sign": ("dequantize", _dequantize_neg),
    "top-k ties to the higher index": ("topk_order_select", _ties_high),
    "nibbles swapped": ("pack_codes", _pack_swapped),
    "no sign extension": ("unpack_codes", _unpack_unsigned),
    "bf16 truncation": ("bf16_rne", _bf16_truncate),
    "decoder step without /qmax": ("block_steps", _steps_no_qmax),
    "8-bit error decompressed with s_e, not 1/s_e": ("error_decompress", _edecomp_times_scale),
    "8-bit error compressed with floor": ("error_compress", _ecomp_floor),
    "8-bit error compressed without clamp": ("error_compress", _ecomp_no_clamp),
    "sparse aggregation in reversed peer order": ("sparse_aggregate", _sa_reversed),
    "sparse aggregation without out_scale": ("sparse_aggregate", _sa_no_scale),
    "sparse aggregation index off by one": ("sparse_aggregate", _sa_index_plus_one),
    "sparse aggregation with the first chunk's scale": ("sparse_aggregate", _sa_slot_scale),
    "Adam with beta1 weighting the old moment": ("adam_step", _adam_swapped),
    "Adam with delta outside the square root": ("adam_step", _adam_delta_outside),
    "Adam with bias correction": ("adam_step", _adam_bias_corrected),
    "Adam on the bf16-rounded average": ("dequant_reduce_adam", _dra_bf16_gradient),
    "out_scale applied after the Adam step": ("dequant_reduce_adam", _dra_scale_after),
    "bf16 weight copy truncated": ("dequant_reduce_adam", _dra_copy_truncated),
    "tiny block keeps an infinite reciprocal": ("finite_reciprocal", _recip_keeps_overflow),
    "reciprocal zeroed for every subnormal step": ("finite_reciprocal", _recip_zero_subnormal),
    "decompressor as a biased product minus its offset": ("dequantize", _dequant_offset_form),
    "dequant-reduce in reversed peer order": ("dequant_reduce", _dr_reversed),
    "top-k decay applied to g instead of e": ("topk_quantize", _tk_variant("decay on g")),
    "top-k selects by |g| instead of |h|": ("topk_quantize", _tk_variant("select by g")),
    "top-k keeps h as the error of the sent values": ("topk_quantize", _tk_variant("kept error not reduced")),
    "top-k zeroes the error of the unsent values": ("topk_quantize", _tk_variant("unselected error zeroed")),
    "Adam second moment of |g| instead of g^2": ("adam_step", _adam_v_linear),
}


@pytest.mark.parametrize("label", sorted(MUTATIONS))
def test_mutation_is_caught(label, monkeypatch):
    name, bad = MUTATIONS[label]
    monkeypatch.setattr(O, name, bad)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(O)
        except AssertionError:
            caught.append(pin.__name__)
        except Exception as ex:  # a crash inside a pin also counts as a failed pin
            caught.append(f"{pin.__name__}:{type(ex).__name__}")
    assert caught, f"no pin catches: {label}"
