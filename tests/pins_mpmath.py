"""High-precision brute force of the MoE layer, used only to pin the oracle.

Written independently of ``oracle/``: scalar loops over the raw int4 codes in
mpmath at 50 significant digits, subset enumeration for the top-k choice.
It follows the same readings of the Swiftlet pages as the oracle (routing of
each token to k of E experts, MLX affine int4 experts, resident shared expert):
softmax renormalised over the chosen k, ties to the lower index, SwiGLU
experts, sigmoid-gated shared expert.
"""
from __future__ import annotations

import itertools

import mpmath as mp
import numpy as np

mp.mp.dps = 50


def _bf16(bits):
    return mp.mpf(float((np.uint32(bits) << np.uint32(16)).view(np.float32)))


def _w(m, o, j):
    if "weights" in m:
        return mp.mpf(float(m["weights"][o, j]))
    s = mp.mpf(float(m["scales"][o, j // 64]))
    b = mp.mpf(float(m["biases"][o, j // 64]))
    return s * int(m["codes"][o, j]) + b


def _matvec(m, v):
    out, inp = (m["weights"] if "weights" in m else m["codes"]).shape
    return [mp.fsum(_w(m, o, j) * v[j] for j in range(inp)) for o in range(out)]


def _ffn(raw, xv):
    g = _matvec(raw["gate"], xv)
    u = _matvec(raw["up"], xv)
    h = [gi / (1 + mp.exp(-gi)) * ui for gi, ui in zip(g, u)]
    return _matvec(raw["down"], h)


def brute_subset(logits, k):
    """Top-k by enumerating every k-subset: the largest logit sum wins, ties
    to the lexicographically smallest index tuple; returned in rank order."""
    E = len(logits)
    best, best_key = None, None
    for S in itertools.combinations(range(E), k):
        key = (mp.fsum(logits[e] for e in S), tuple(-e for e in S))
        if best_key is None or key > best_key:
            best, best_key = S, key
    return sorted(best, key=lambda e: (-logits[e], e))


def layer_token(xbits_row, w_router, bias, k, expert, shared):
    """(y[d], idx[k], w[k], s) for one token."""
    d = len(xbits_row)
    xv = [_bf16(b) for b in xbits_row]
    E = w_router.shape[0] - 1
    logits = []
    for e in range(E):
        l = mp.fsum(xv[j] * mp.mpf(float(w_router[e, j])) for j in range(d))
        if bias is not None:
            l += mp.mpf(float(bias[e]))
        logits.append(l)
    gsh = mp.fsum(xv[j] * mp.mpf(float(w_router[E, j])) for j in range(d))
    S = brute_subset(logits, k)
    m = max(logits[e] for e in S)
    ex = [mp.exp(logits[e] - m) for e in S]
    z = mp.fsum(ex)
    w = [v / z for v in ex]
    s = 1 / (1 + mp.exp(-gsh))
    y = [mp.mpf(0)] * d
    for wr, e in zip(w, S):
        o = _ffn(expert(e), xv)
        y = [a + wr * b for a, b in zip(y, o)]
    osh = _ffn(shared, xv)
    y = [a + s * b for a, b in zip(y, osh)]
    return y, S, w, s
