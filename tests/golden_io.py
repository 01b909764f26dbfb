"""Readers for the hand-derived fixtures under tests/golden/."""
from __future__ import annotations

import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if line:
                yield line


def lfu_traces():
    """[(name, E, slots, [(selected, loads, hits)])]."""
    out = []
    cur = None
    for line in _lines("lfu_traces.txt"):
        if line.startswith("trace"):
            _, name, e, s = line.split()
            cur = (name, int(e.split("=")[1]), int(s.split("=")[1]), [])
        elif line == "end":
            out.append(cur)
            cur = None
        else:
            lhs, rhs = line.split("->")
            sel = [int(v) for v in lhs.split(",")]
            toks = rhs.split()
            hits = int(toks[-1].split("=")[1])
            loads = [tuple(int(a) for a in t.split(":")) for t in toks[:-1]]
            cur[3].append((sel, loads, hits))
    return out


def blob_layout():
    """[(d, I, bits, bytes, stride, codes[(mat,row,col,val,off,byte)], sbs[(mat,row,g,soff,boff)],
    weights[(mat,row,col,value,off,u32)])]."""
    out = []
    cur = None
    for line in _lines("blob_layout.txt"):
        t = line.split()
        if t[0] == "shape":
            kv = dict(a.split("=") for a in t[1:])
            cur = (int(kv["d"]), int(kv["I"]), int(kv.get("bits", 4)), int(kv["bytes"]),
                   int(kv["stride"]), [], [], [])
        elif t[0] == "end":
            out.append(cur)
        elif t[0] == "code":
            cur[5].append((t[1], int(t[2]), int(t[3]), int(t[4]), int(t[6]), int(t[7], 16)))
        elif t[0] == "sb":
            cur[6].append((t[1], int(t[2]), int(t[3]), int(t[5]), int(t[6])))
        elif t[0] == "weight":
            cur[7].append((t[1], int(t[2]), int(t[3]), float(t[4]), int(t[6]), int(t[7], 16)))
    return out
