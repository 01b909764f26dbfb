"""Oracle: router, expert FFN and the whole routed-expert MoE layer, fp64.

Authority (Swiftlet pages, "How it works"): each token is routed to k of E
experts (10 of 512, 8 of 256); the router and the shared expert stay resident
while routed experts are fetched; the routed outputs and the shared expert's
are combined.  Readings where the pages are silent:

  * router: logits l = x W_r[:E]^T + b (b an optional per-expert offset);
    select the k largest logits, ties to the lower expert index, in rank order
    (logit descending, index ascending); weights = softmax over the selected
    logits, i.e. the full softmax renormalised to sum 1 over the chosen k;
  * shared-expert gate s = sigmoid(x . W_r[E]) (the extra router row),
    added on top of the routed sum and not renormalised with it;
  * expert FFN is SwiGLU: h = silu(W_gate x) * (W_up x), o = W_down h,
    silu(z) = z / (1 + exp(-z));
  * y_t = sum_r w[t,r] o_{e_r}(x_t) + s_t o_shared(x_t).

A chain of L such layers (several MoE layers per token, the next item after
one layer; the pages' models stack dozens of them) follows the pre-norm
residual form of the decoder these layers sit in, read without the
attention half and without a learned norm weight:

  u_l = bf16(x_l / sqrt(mean(x_l^2) + eps)),  x_{l+1} = bf16(fp32(x_l + MoE_l(u_l))),

the residual stream and the MoE input carried in bf16 (the layer's input
type), eps = 1e-6.

Everything is float64 on exactly decoded inputs; the only library primitives
are numpy's matmul and sort.
"""
from __future__ import annotations

from typing import Callable, Optional

import numpy as np

from .quant import dequant


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (the upper half of an fp32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def router_logits(x: np.ndarray, w_router: np.ndarray, bias: Optional[np.ndarray]):
    """(l [T,E], g [T]) in fp64.  x fp64 [T,d]; w_router [E+1, d]."""
    W = np.asarray(w_router, dtype=np.float64)
    E = W.shape[0] - 1
    l = x @ W[:E].T
    if bias is not None:
        l = l + np.asarray(bias, dtype=np.float64)[None, :]
    g = x @ W[E]
    return l, g


def select_topk(l: np.ndarray, k: int) -> np.ndarray:
    """Rank-ordered top-k per row: logit descending, expert index ascending."""
    T, E = l.shape
    idx = np.empty((T, k), dtype=np.int32)
    e = np.arange(E)
    for t in range(T):
        order = np.lexsort((e, -l[t]))      # primary -l, secondary index
        idx[t] = order[:k]
    return idx


def topk_weights(l: np.ndarray, idx: np.ndarray) -> np.ndarray:
    sel = np.take_along_axis(l, idx.astype(np.int64), axis=1)
    m = sel.max(axis=1, keepdims=True)
    ex = np.exp(sel - m)
    return ex / ex.sum(axis=1, keepdims=True)


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def route(x_bits: np.ndarray, w_router, bias, k: int):
    """Full router step.  Returns idx [T,k] int32, w [T,k], s [T], logits."""
    x = bf16_to_f64(x_bits)
    l, g = router_logits(x, w_router, bias)
    idx = select_topk(l, k)
    return idx, topk_weights(l, idx), sigmoid(g), l


def expert_ffn(raw, x: np.ndarray) -> np.ndarray:
    """SwiGLU expert on fp64 activations x [n, d] -> [n, d]."""
    Wg = dequant(raw["gate"])
    Wu = dequant(raw["up"])
    Wd = dequant(raw["down"])
    gt = x @ Wg.T
    up = x @ Wu.T
    h = gt * sigmoid(gt) * up
    return h @ Wd.T


def moe_layer(x_bits: np.ndarray, w_router, bias, k: int,
              expert: Callable[[int], dict], shared: dict,
              idx: Optional[np.ndarray] = None):
    """The whole layer.  ``expert(e)`` returns expert e's raw matrices.

    ``idx`` may force the selection (used where fp32 routing on the device
    legitimately picks another member of a certified near-tie); weights are
    then the renormalised softmax over that selection.
    Returns dict(y, idx, w, s, logits).
    """
    x = bf16_to_f64(x_bits)
    l, g = router_logits(x, w_router, bias)
    if idx is None:
        idx = select_topk(l, k)
    w = topk_weights(l, idx)
    s = sigmoid(g)
    T, d = x.shape
    y = np.zeros((T, d), dtype=np.float64)
    for e in np.unique(idx):
        rows, ranks = np.nonzero(idx == e)
        o = expert_ffn(expert(int(e)), x[rows])
        y[rows] += w[rows, ranks][:, None] * o
    y += s[:, None] * expert_ffn(shared, x)
    return {"y": y, "idx": idx, "w": w, "s": s, "logits": l}


def logit_error_bound(x_bits: np.ndarray, w_router, bias, depth: int) -> np.ndarray:
    """Per-token bound on |fp32 logit - exact logit| for a device that forms
    each logit as an fp32 sum of the d products with at most ``depth``
    additions on any path (plus one for the bias): gamma_n * sum|x_j W_ej| + u|b|,
    gamma_n = n u / (1 - n u), u = 2^-24 (standard floating-point summation
    bound).  Returns [T]."""
    x = np.abs(bf16_to_f64(x_bits))
    W = np.abs(np.asarray(w_router, dtype=np.float64))
    E = W.shape[0] - 1
    a = x @ W[:E].T
    u = 2.0 ** -24
    n = depth + 2
    gam = n * u / (1 - n * u)
    r = gam * a.max(axis=1)
    if bias is not None:
        b = np.abs(np.asarray(bias, np.float64))
        r = r + 2 * u * (a.max(axis=1) + b.max())
    return r


def logit_error_bounds(x_bits: np.ndarray, w_router, depth: int) -> np.ndarray:
    """Elementwise bound on |fp32 logit - exact logit| for every router row
    (the E routed rows and the shared-gate row E), before any bias, for a
    device that forms each logit as an fp32 sum of the d products with at most
    ``depth`` additions on any path: gamma_n * sum_j |x_j W_ej|, n = depth + 2
    (the additions, the product's rounding and one spare), gamma_n =
    n u / (1 - n u), u = 2^-24 (standard floating-point summation bound).
    Returns [T, E+1]."""
    x = np.abs(bf16_to_f64(x_bits))
    W = np.abs(np.asarray(w_router, dtype=np.float64))
    u = 2.0 ** -24
    n = depth + 2
    return (n * u / (1 - n * u)) * (x @ W.T)


# ----------------------------------------------------------------- chains
def bf16_round(v) -> np.ndarray:
    """bf16 bits of fp32 values, round to nearest, ties to even (written out
    on the fp32 bit pattern; finite inputs)."""
    u = np.ascontiguousarray(np.asarray(v, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    keep = u >> 16
    rest = u & 0xFFFF
    up = (rest > 0x8000) | ((rest == 0x8000) & ((keep & 1) == 1))
    return (keep + up).astype(np.uint16)


def rms_norm_bf16(x_bits: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """u = x / sqrt(mean(x^2) + eps) per row, exact in fp64, rounded to bf16."""
    x = bf16_to_f64(x_bits)
    u = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return bf16_round(u.astype(np.float32))


def residual_bf16(x_bits: np.ndarray, y: np.ndarray) -> np.ndarray:
    """bf16(fp32(x + y)): the residual add in fp32, rounded to bf16."""
    s = bf16_to_f64(x_bits).astype(np.float32) + np.asarray(y, dtype=np.float64).astype(np.float32)
    return bf16_round(s)


def chain_layer(x_bits: np.ndarray, layer: dict, eps: float = 1e-6, idx=None):
    """One residual MoE block.  layer: dict(w_router, bias, k, expert, shared).
    Returns (x_next_bits, u_bits, layer result dict)."""
    u = rms_norm_bf16(x_bits, eps)
    res = moe_layer(u, layer["w_router"], layer["bias"], layer["k"], layer["expert"], layer["shared"], idx=idx)
    return residual_bf16(x_bits, res["y"]), u, res
