"""Readers for the hand-worked fixtures under tests/golden/ (plain text)."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for ln in f:
            ln = ln.strip()
            if ln and not ln.startswith("#"):
                yield ln


def rounding_cases():
    for ln in _lines("round_fixed_scale.txt"):
        b, m, q = ln.split()
        yield int(b), float(m), int(q)


def pack_cases():
    for ln in _lines("pack_layout.txt"):
        b, codes, hx = [x.strip() for x in ln.split("|")]
        yield int(b), [int(c) for c in codes.split()], bytes.fromhex(hx.replace(" ", ""))


def _cases(name):
    case = None
    for ln in _lines(name):
        if ln.startswith("case"):
            case = {"name": ln.split()[1]}
        elif ln == "end":
            yield case
            case = None
        else:
            k, *v = ln.split()
            case[k] = v


def cq_cases():
    for c in _cases("cq_worked.txt"):
        ed = c.get("err_dtype", ["f32"])[0]
        et = np.int8 if ed == "i8" else np.float32
        yield {"bits": int(c["bits"][0]), "block": int(c["block"][0]), "beta": float(c["beta"][0]),
               "err_dtype": ed, "err_scale": float(c.get("err_scale", ["0"])[0]),
               "reset": bool(int(c.get("reset", ["0"])[0])),
               "g": np.array(c["g"], np.float32), "e": np.array(c["e"], np.float64).astype(et),
               "absmax": np.array(c["absmax"], np.float32),
               "codes": bytes.fromhex("".join(c["codes"])),
               "e_new": np.array(c["e_new"], np.float64).astype(et)}


def dr_case():
    d = {"peers": []}
    for ln in _lines("dr_worked.txt"):
        k, rest = ln.split(None, 1)
        if k == "peer":
            hx, am = rest.split("|")
            d["peers"].append((np.frombuffer(bytes.fromhex(hx.replace(" ", "")), np.uint8).copy(),
                               np.array(am.split(), np.float32)))
        elif k == "out":
            d["out"] = np.array(rest.split(), np.float32)
        elif k == "out_scale":
            d[k] = float(rest)
        else:
            d[k] = int(rest)
    return d


def topk_cases():
    for c in _cases("topk_worked.txt"):
        yield {"chunk": int(c["chunk"][0]), "k": int(c["k"][0]), "decay": float(c["decay"][0]),
               "g": np.array(c["g"], np.float32), "e": np.array(c["e"], np.float32),
               "idx": np.array(c["idx"], np.int64).astype(np.uint16),
               "codes": bytes.fromhex("".join(c["codes"])),
               "absmax": np.array(c["absmax"], np.float32),
               "e_new": np.array(c["e_new"], np.float32)}


def sa_case():
    d = {"peers": []}
    for ln in _lines("sa_worked.txt"):
        k, rest = ln.split(None, 1)
        if k == "peer":
            ix, hx, am = rest.split("|")
            d["peers"].append((np.array(ix.split(), np.int64).astype(np.uint16),
                               np.frombuffer(bytes.fromhex(hx.replace(" ", "")), np.uint8).copy(),
                               np.array(am.split(), np.float32)))
        elif k == "out":
            d["out"] = np.array(rest.split(), np.float32)
        elif k == "out_scale":
            d[k] = float(rest)
        else:
            d[k] = int(rest)
    return d


def adam_case():
    d = {}
    for ln in _lines("adam_worked.txt"):
        k, rest = ln.split(None, 1)
        v = rest.split()
        d[k] = float(v[0]) if len(v) == 1 and k in ("lr", "beta1", "beta2", "delta") else np.array(v, np.float32)
    return d


def dra_case():
    d = {"peers": []}
    for ln in _lines("dra_worked.txt"):
        k, rest = ln.split(None, 1)
        if k == "peer":
            hx, am = rest.split("|")
            d["peers"].append((np.frombuffer(bytes.fromhex(hx.replace(" ", "")), np.uint8).copy(),
                               np.array(am.split(), np.float32)))
        elif k in ("bits", "block", "n"):
            d[k] = int(rest)
        elif k in ("out_scale", "lr", "beta1", "beta2", "delta"):
            d[k] = float(rest)
        else:
            d[k] = np.array(rest.split(), np.float32)
    return d
