"""Readers for the hand-worked text fixtures under tests/golden/."""
import os
import struct

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def h16(hexstr: str) -> np.float16:
    return np.frombuffer(struct.pack("<H", int(hexstr, 16)), dtype=np.float16)[0]


def _values(tokens):
    out = []
    for t in tokens:
        if "x" in t:
            cnt, hx = t.split("x")
            out += [h16(hx)] * int(cnt)
        else:
            out.append(h16(t))
    return np.array(out, dtype=np.float16)


def read_pack_words(name="pack_words.txt"):
    rows = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        lhs, rhs = line.split("->")
        rows.append(([int(v) for v in lhs.split()], int(rhs.strip(), 16)))
    return rows


def read_cases(name):
    cases, cur = [], None
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        tok = line.split()
        if tok[0] == "case":
            cur = {"name": tok[1], "code": {}, "deq": {}}
            cases.append(cur)
        elif tok[0] == "values":
            cur["values"] = _values(tok[1:])
        elif tok[0] == "scale":
            cur["scale"] = h16(tok[1])
            cur["zero"] = int(tok[3])
        elif tok[0] == "code":
            cur["code"][tok[1].upper()] = int(tok[2])
        elif tok[0] == "deq":
            cur["deq"][tok[1].upper()] = tok[2]
        elif tok[0] == "group":
            cur["group"] = int(tok[1])
        elif tok[0] == "cscale":
            cur["cscale"] = h16(tok[1])
        elif tok[0] == "gscale":
            cur["gscale"] = [int(v) for v in tok[1:]]
        elif tok[0] == "q":
            cur["q"] = [int(v) for v in tok[1:]]
        elif tok[0] == "q_head":
            parts = " ".join(tok[1:]).split("|")
            cur["q_head"] = [[int(v) for v in p.split()] for p in parts]
        else:
            raise ValueError(f"unknown fixture key {tok[0]!r}")
    return cases


def read_silu_cases():
    """Cases of golden/silu_mul_quant_worked.txt: ``gate_up`` (fp16 hex), ``s_a``
    (decimal) and ``xq`` (ints)."""
    cases, cur = [], None
    for line in open(os.path.join(GOLDEN, "silu_mul_quant_worked.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *rest = line.split()
        if key == "case":
            cur = {"name": rest[0]}
            cases.append(cur)
        elif key == "gate_up":
            cur["gate_up"] = _values(rest)
        elif key == "s_a":
            cur["s_a"] = float(rest[0])
        elif key == "xq":
            cur["xq"] = [int(v) for v in rest]
    return cases


def read_variant_cases():
    """Cases of golden/w4a16_variants_worked.txt: ``rule``, ``group``, ``values`` (fp16),
    ``scales`` (fp16 per group), ``zeros`` and ``codes_head`` (per 128-k block: leading
    codes) or ``codes_at`` (k -> code)."""
    cases, cur = [], None
    for line in open(os.path.join(GOLDEN, "w4a16_variants_worked.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *rest = line.split()
        if key == "case":
            cur = {"name": rest[0]}
            cases.append(cur)
        elif key == "rule":
            cur["rule"] = rest[0]
        elif key == "group":
            cur["group"] = int(rest[0])
        elif key in ("values", "scales"):
            cur[key] = _values(rest)
        elif key == "zeros":
            cur["zeros"] = [int(v) for v in rest]
        elif key == "codes_head":
            cur["codes_head"] = [[int(v) for v in part.split()] for part in " ".join(rest).split("|")]
        elif key == "codes_at":
            cur["codes_at"] = {int(k): int(v) for k, v in (t.split("=") for t in rest)}
    return cases
