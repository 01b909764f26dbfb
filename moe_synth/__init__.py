"""Seeded synthetic inputs for the routed-expert MoE layer.

This module is the only code shared by the CPU oracle and the HIP path.  It
draws raw inputs (bf16 activations, fp32 router weights, int4 codes with fp16
group scales/biases, a slot permutation, a Zipf-shaped logit offset) and holds
none of the layer's arithmetic: no dequantisation, no matmul, no routing, no
packing into blobs.

Shapes follow the layer the Swiftlet pages describe ("How it works": every
layer sends each token to 10 of 512 experts for the 80B model, 8 of 256 for
the 35B model; the router and the shared expert stay resident; routed experts
are 4-bit MLX affine group-quantised weights).  Value distributions are the
synthetic recipe of the workload table (x ~ N(0,1) rounded to bf16, router
weights ~ N(0, 0.02) in fp32, codes uniform on 0..15, scales ~ U[0.002, 0.02]
rounded to fp16, bias = -8 * scale).  8-bit experts (the pages' kernels also
cover MLX affine int8) draw codes uniform on 0..255, scales U[0.002, 0.02]/16
rounded to fp16 and bias = -128 * scale, so their weights span the same range
as the 4-bit ones.  f32 experts (unquantised) draw weights ~ N(0, 0.05) in
fp32, about the spread of the 4-bit weights.

Every array comes from its own counter-keyed numpy PCG64 stream
(``default_rng([seed, component, index])``) so that any expert or any decode
step can be drawn on demand, in any order, with identical results.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

GROUP = 64

# stream component ids (part of the seed key; never change them)
_C_ROUTER = 1
_C_BIAS = 2
_C_SHARED = 3
_C_EXPERT = 4
_C_SLOTS = 5
_C_X = 6
_C_BIASPERM = 7


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int            # tokens per step
    d: int            # hidden size
    E: int            # routed experts
    k: int            # experts per token
    I: int            # routed expert intermediate size
    I_shared: int     # shared expert intermediate size
    n_slots: int      # HBM slot-pool capacity (blobs)
    steps: int        # seeded steps in the workload
    alpha: float      # Zipf logit-offset scale (0 = unbiased router)
    seed: int
    permute_slots: bool = True
    bits: int = 4     # code width of routed and shared experts (4, 8; 32 = fp32 weights)

    @property
    def group(self) -> int:
        return GROUP


# The five workloads.  alpha for the Zipf-skewed runs is calibrated so that a
# 256-slot LFU+recency pool over 512 experts lands inside the 43-70 % hit-rate
# band the pages report ("How it works", expert cache paragraph): 0.15 gives
# about 62 % over 1000 seeded 80B-shape decode steps.
ZIPF_ALPHA = 0.15

CONFIGS: Dict[str, LayerConfig] = {
    "tiny": LayerConfig("tiny", T=4, d=256, E=16, k=2, I=64, I_shared=64,
                        n_slots=16, steps=8, alpha=0.0, seed=1000,
                        permute_slots=False),
    "decode35b": LayerConfig("decode35b", T=1, d=2048, E=256, k=8, I=512,
                             I_shared=512, n_slots=256, steps=1000, alpha=0.0,
                             seed=1001),
    "decode80b": LayerConfig("decode80b", T=1, d=2048, E=512, k=10, I=512,
                             I_shared=512, n_slots=256, steps=1000,
                             alpha=ZIPF_ALPHA, seed=1002),
    "batch80b": LayerConfig("batch80b", T=64, d=2048, E=512, k=10, I=512,
                            I_shared=512, n_slots=512, steps=100,
                            alpha=ZIPF_ALPHA, seed=1003),
    "prefill80b": LayerConfig("prefill80b", T=4096, d=2048, E=512, k=10, I=512,
                              I_shared=512, n_slots=512, steps=1, alpha=0.0,
                              seed=1004),
    "prefill80b_zipf": LayerConfig("prefill80b_zipf", T=4096, d=2048, E=512,
                                   k=10, I=512, I_shared=512, n_slots=512,
                                   steps=1, alpha=ZIPF_ALPHA, seed=1005),
    # the same layers with 8-bit experts
    "tiny_int8": LayerConfig("tiny_int8", T=4, d=256, E=16, k=2, I=64, I_shared=64,
                             n_slots=16, steps=8, alpha=0.0, seed=1100,
                             permute_slots=False, bits=8),
    "decode80b_int8": LayerConfig("decode80b_int8", T=1, d=2048, E=512, k=10, I=512,
                                  I_shared=512, n_slots=512, steps=1000,
                                  alpha=ZIPF_ALPHA, seed=1102, bits=8),
    "batch80b_int8": LayerConfig("batch80b_int8", T=64, d=2048, E=512, k=10, I=512,
                                 I_shared=512, n_slots=512, steps=100,
                                 alpha=ZIPF_ALPHA, seed=1103, bits=8),
    "prefill80b_int8": LayerConfig("prefill80b_int8", T=4096, d=2048, E=512, k=10,
                                   I=512, I_shared=512, n_slots=512, steps=1,
                                   alpha=0.0, seed=1104, bits=8),
    # and with unquantised fp32 experts
    "tiny_f32": LayerConfig("tiny_f32", T=4, d=256, E=16, k=2, I=64, I_shared=64,
                            n_slots=16, steps=8, alpha=0.0, seed=1200,
                            permute_slots=False, bits=32),
    "decode80b_f32": LayerConfig("decode80b_f32", T=1, d=2048, E=512, k=10, I=512,
                                 I_shared=512, n_slots=512, steps=1000,
                                 alpha=ZIPF_ALPHA, seed=1202, bits=32),
    "batch80b_f32": LayerConfig("batch80b_f32", T=64, d=2048, E=512, k=10, I=512,
                                I_shared=512, n_slots=512, steps=100,
                                alpha=ZIPF_ALPHA, seed=1203, bits=32),
}


def rng(seed: int, component: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, component, index])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def x_bits(cfg: LayerConfig, step: int = 0, T: Optional[int] = None) -> np.ndarray:
    """Activations for one step: bf16 bits, shape [T, d]."""
    T = cfg.T if T is None else T
    g = rng(cfg.seed, _C_X, step)
    return f32_to_bf16_bits(g.standard_normal((T, cfg.d), dtype=np.float32))


def router_weight(cfg: LayerConfig) -> np.ndarray:
    """fp32 [E+1, d]; rows 0..E-1 route, row E is the shared-expert gate."""
    g = rng(cfg.seed, _C_ROUTER)
    return (g.standard_normal((cfg.E + 1, cfg.d), dtype=np.float32)
            * np.float32(0.02)).astype(np.float32)


def logit_bias(cfg: LayerConfig, alpha: Optional[float] = None) -> Optional[np.ndarray]:
    """Zipf(s=1.1) popularity offset on the router logits, or None if alpha=0.

    b_e = -alpha * 1.1 * ln(r_e), with r a seeded permutation of 1..E, so the
    expert with popularity rank r gets an offset proportional to log r^-1.1.
    """
    a = cfg.alpha if alpha is None else alpha
    if a == 0.0:
        return None
    g = rng(cfg.seed, _C_BIASPERM)
    r = g.permutation(cfg.E).astype(np.float64) + 1.0
    return (-a * 1.1 * np.log(r)).astype(np.float32)


def _matrix(g: np.random.Generator, out: int, inp: int, bits: int = 4):
    if bits == 4:
        codes = g.integers(0, 16, size=(out, inp), dtype=np.uint8)
        sc = g.uniform(0.002, 0.02, size=(out, inp // GROUP)).astype(np.float16)
        bi = (np.float16(-8.0) * sc).astype(np.float16)   # exact in fp16
    elif bits == 8:
        codes = g.integers(0, 256, size=(out, inp), dtype=np.uint8)
        sc = (g.uniform(0.002, 0.02, size=(out, inp // GROUP)) / 16).astype(np.float16)
        bi = (np.float16(-128.0) * sc).astype(np.float16)  # exact in fp16
    elif bits == 32:
        return {"weights": (g.standard_normal((out, inp), dtype=np.float32) * np.float32(0.05)).astype(np.float32)}
    else:
        raise ValueError(f"bits must be 4 or 8, not {bits}")
    return {"codes": codes, "scales": sc, "biases": bi}


def expert_raw(cfg: LayerConfig, e: int, I: Optional[int] = None,
               component: int = _C_EXPERT) -> Dict[str, Dict[str, np.ndarray]]:
    """Raw int4 / int8 (cfg.bits) weights of one expert, MLX orientation
    [out][in] / [out][in/64] (fp32 [out][in] for cfg.bits == 32).

    gate, up: out = I, in = d.  down: out = d, in = I.
    """
    I = cfg.I if I is None else I
    g = rng(cfg.seed, component, e)
    return {"gate": _matrix(g, I, cfg.d, cfg.bits),
            "up": _matrix(g, I, cfg.d, cfg.bits),
            "down": _matrix(g, cfg.d, I, cfg.bits)}


def shared_raw(cfg: LayerConfig):
    return expert_raw(cfg, 0, I=cfg.I_shared, component=_C_SHARED)


def slot_permutation(cfg: LayerConfig) -> np.ndarray:
    """slot_table[e] for an all-resident pool (E slots); identity if disabled."""
    if not cfg.permute_slots:
        return np.arange(cfg.E, dtype=np.int32)
    g = rng(cfg.seed, _C_SLOTS)
    return g.permutation(cfg.E).astype(np.int32)


def scaled(cfg: LayerConfig, **kw) -> LayerConfig:
    """A copy of cfg with some fields replaced (used for small test shapes)."""
    return dataclasses.replace(cfg, **kw)
