"""Pins of the CPU oracle against facts fixed outside it (CPU only).

Each test names what it pins: a count the pages print, a closed form, an
invariant, a hand-derived fixture under tests/golden/, brute force on tiny
inputs, or an independent 50-digit evaluation.
"""
import itertools
import math

import numpy as np
import pytest

import moe_synth as ms
from oracle import bucket as obucket
from oracle import layer as olayer
from oracle import lfu as olfu
from oracle import quant as oquant
import golden_io
import pins_mpmath

TINY = ms.CONFIGS["tiny"]


def _tiny_experts(cfg):
    cache = {}

    def get(e):
        if e not in cache:
            cache[e] = ms.expert_raw(cfg, e)
        return cache[e]
    return get


# ---- P1: the fan-out the pages print (10 of 512, 8 of 256) ----------------
@pytest.mark.parametrize("name,k,E", [("decode80b", 10, 512), ("decode35b", 8, 256)])
def test_topk_counts_pages(name, k, E):
    cfg = ms.CONFIGS[name]
    assert (cfg.k, cfg.E) == (k, E)
    Wr = ms.router_weight(cfg)
    for step in range(3):
        idx, w, s, _ = olayer.route(ms.x_bits(cfg, step), Wr, ms.logit_bias(cfg), cfg.k)
        assert idx.shape == (1, k)
        assert len(set(idx[0].tolist())) == k
        assert idx.min() >= 0 and idx.max() < E


# ---- P2: selection vs subset enumeration -----------------------------------
def test_selection_bruteforce():
    g = np.random.default_rng(7)
    for trial in range(40):
        E, k = 9, 3
        l = g.standard_normal(E)
        if trial % 3 == 0:          # plant exact ties, incl. at the boundary
            l[g.integers(E)] = l[g.integers(E)]
            l[:4] = np.round(l[:4])
        got = olayer.select_topk(l[None, :], k)[0].tolist()
        ref = pins_mpmath.brute_subset([float(v) for v in l], k)
        assert got == list(ref)
        chosen = set(got)
        assert min(l[e] for e in chosen) >= max(l[e] for e in range(E) if e not in chosen)


# ---- P14: equal logits go to the lower index --------------------------------
def test_tie_rule_identical_rows():
    cfg = TINY
    Wr = ms.router_weight(cfg).copy()
    Wr[11] = Wr[4]           # experts 4 and 11 now have identical logits
    x = ms.x_bits(cfg, 0)
    l, _ = olayer.router_logits(olayer.bf16_to_f64(x), Wr, None)
    assert np.array_equal(l[:, 4], l[:, 11])
    # force both to the top
    Wr2 = Wr.copy()
    Wr2[4] *= 0
    Wr2[11] *= 0
    b = np.zeros(cfg.E, np.float32)
    b[4] = b[11] = 50.0
    idx, _, _, _ = olayer.route(x, Wr2, b, 1)
    assert (idx[:, 0] == 4).all()


# ---- P3: weights -------------------------------------------------------------
def test_weights_sum_and_ratio():
    g = np.random.default_rng(3)
    l = g.standard_normal((5, 16)) * 3
    for k in (1, 2, 5, 16):
        idx = olayer.select_topk(l, k)
        w = olayer.topk_weights(l, idx)
        assert np.allclose(w.sum(1), 1.0, atol=1e-15)
        if k == 1:
            assert (w == 1.0).all()
        sel = np.take_along_axis(l, idx.astype(np.int64), 1)
        # ratio of two weights is exp of the logit difference
        assert np.allclose(w[:, 0] / w[:, -1], np.exp(sel[:, 0] - sel[:, -1]), rtol=1e-12)
        assert (np.diff(w, axis=1) <= 1e-15).all()     # rank order = weight order


# ---- P15: shared gate --------------------------------------------------------
def test_shared_gate_closed_form():
    cfg = TINY
    Wr = ms.router_weight(cfg).copy()
    Wr[cfg.E] = 0.0
    _, _, s, _ = olayer.route(ms.x_bits(cfg, 0), Wr, None, cfg.k)
    assert (s == 0.5).all()
    # one-hot x picks a single router element: s = 1 / (1 + e^-w)
    xb = np.zeros((1, cfg.d), np.uint16)
    xb[0, 5] = 0x3F80                       # bf16 1.0
    Wr[cfg.E, 5] = np.float32(math.log(3.0))
    _, _, s, _ = olayer.route(xb, Wr, None, cfg.k)
    assert abs(s[0] - 0.75) < 1e-7          # sigmoid(ln 3) = 3/4 (w rounded to fp32)


# ---- P5: whole tiny layer vs 50-digit brute force ---------------------------
@pytest.mark.parametrize("name", ["tiny", "tiny_int8", "tiny_f32"])
def test_layer_vs_mpmath_bruteforce(name):
    cfg = ms.CONFIGS[name]
    Wr = ms.router_weight(cfg)
    xb = ms.x_bits(cfg, 0)
    ex = _tiny_experts(cfg)
    sh = ms.shared_raw(cfg)
    res = olayer.moe_layer(xb, Wr, None, cfg.k, ex, sh)
    for t in (0, 3):
        y, S, w, s = pins_mpmath.layer_token(xb[t], Wr, None, cfg.k, ex, sh)
        assert res["idx"][t].tolist() == list(S)
        assert np.allclose(res["w"][t], [float(v) for v in w], rtol=1e-13, atol=0)
        assert abs(res["s"][t] - float(s)) < 1e-15
        yr = np.array([float(v) for v in y])
        assert np.max(np.abs(res["y"][t] - yr)) <= 1e-12 * np.max(np.abs(yr))


# ---- P4: k = E reduces to the dense all-experts softmax sum -----------------
def test_k_equals_E_dense():
    cfg = ms.scaled(TINY, E=6, k=6)
    Wr = ms.router_weight(cfg)
    xb = ms.x_bits(cfg, 1)
    ex = _tiny_experts(cfg)
    sh = ms.shared_raw(cfg)
    res = olayer.moe_layer(xb, Wr, None, cfg.k, ex, sh)
    # dense formula: stacked weights, full softmax, einsum over experts
    x = olayer.bf16_to_f64(xb)
    W = Wr.astype(np.float64)
    L = np.einsum("td,ed->te", x, W[:cfg.E])
    P = np.exp(L - L.max(1, keepdims=True))
    P /= P.sum(1, keepdims=True)
    Gs = np.stack([oquant.dequant(ex(e)["gate"]) for e in range(cfg.E)])
    Us = np.stack([oquant.dequant(ex(e)["up"]) for e in range(cfg.E)])
    Ds = np.stack([oquant.dequant(ex(e)["down"]) for e in range(cfg.E)])
    G = np.einsum("eid,td->tei", Gs, x)
    U = np.einsum("eid,td->tei", Us, x)
    H = G / (1 + np.exp(-G)) * U
    O = np.einsum("edi,tei->ted", Ds, H)
    dense = np.einsum("te,ted->td", P, O)
    gs = 1 / (1 + np.exp(-(x @ W[cfg.E])))
    Gsh = x @ oquant.dequant(sh["gate"]).T
    Ush = x @ oquant.dequant(sh["up"]).T
    dense += gs[:, None] * ((Gsh / (1 + np.exp(-Gsh)) * Ush) @ oquant.dequant(sh["down"]).T)
    assert np.allclose(res["y"], dense, rtol=1e-11, atol=1e-12 * np.abs(dense).max())


# ---- closed form: identical constant experts ---------------------------------
def test_constant_experts_closed_form():
    """All codes of a matrix equal, one scale/bias per matrix: every weight is a
    constant c, so g_o = c_g Sx, u_o = c_u Sx, h = silu(g) u for every o,
    o_j = c_d * I * h, and y_j = (sum_r w_r) o + s o = (1 + s) o."""
    cfg = TINY
    d, I = cfg.d, cfg.I

    def const(out, inp, q, sc, bi):
        return {"codes": np.full((out, inp), q, np.uint8),
                "scales": np.full((out, inp // 64), sc, np.float16),
                "biases": np.full((out, inp // 64), bi, np.float16)}
    raw = {"gate": const(I, d, 11, 0.0078125, -0.0625),
           "up": const(I, d, 3, 0.015625, 0.0),
           "down": const(d, I, 9, 0.001953125, -0.015625)}
    Wr = ms.router_weight(cfg)
    xb = ms.x_bits(cfg, 2)
    res = olayer.moe_layer(xb, Wr, None, cfg.k, lambda e: raw, raw)
    x = olayer.bf16_to_f64(xb)
    Sx = x.sum(1)
    cg = 0.0078125 * 11 - 0.0625
    cu = 0.015625 * 3
    cd = 0.001953125 * 9 - 0.015625
    g = cg * Sx
    h = g / (1 + np.exp(-g)) * (cu * Sx)
    o = cd * I * h
    s = 1 / (1 + np.exp(-(x @ Wr[cfg.E].astype(np.float64))))
    ref = ((1 + s) * o)[:, None] * np.ones((1, d))
    assert np.allclose(res["y"], ref, rtol=1e-12, atol=1e-14)


# ---- P10 / P11: zero expert, power-of-two scaling ---------------------------
def test_zero_expert_and_power_of_two():
    cfg = TINY
    raw = ms.expert_raw(cfg, 3)
    z = {k: dict(v) for k, v in raw.items()}
    z["down"] = {"codes": np.full_like(raw["down"]["codes"], 8),
                 "scales": raw["down"]["scales"], "biases": raw["down"]["biases"]}
    x = olayer.bf16_to_f64(ms.x_bits(cfg, 0))
    assert (olayer.expert_ffn(z, x) == 0).all()      # bias = -8 scale -> W = 0
    dbl = {k: dict(v) for k, v in raw.items()}
    dbl["down"] = {"codes": raw["down"]["codes"],
                   "scales": (raw["down"]["scales"] * 2).astype(np.float16),
                   "biases": (raw["down"]["biases"] * 2).astype(np.float16)}
    assert np.array_equal(olayer.expert_ffn(dbl, x), 2 * olayer.expert_ffn(raw, x))


def test_dequant_exact_in_fp32():
    """s*q + b with fp16 s, b = -8 s and q in 0..15 has <= 15 significant bits:
    exactly representable in fp32 (so an fp32 device loses nothing there)."""
    raw = ms.expert_raw(ms.CONFIGS["decode80b"], 5)
    for m in raw.values():
        W = oquant.dequant(m)
        assert np.array_equal(W.astype(np.float32).astype(np.float64), W)


# ---- P7: blob layout ---------------------------------------------------------
@pytest.mark.parametrize("case", range(6))
def test_blob_layout_golden(case):
    d, I, bits, nbytes, stride, codes, sbs, weights = golden_io.blob_layout()[case]
    per16 = {4: 27, 8: 51, 32: 192}[bits]
    assert oquant.blob_bytes(d, I, bits) == nbytes == per16 * d * I // 16
    assert oquant.blob_stride(d, I, bits) == stride
    dims = oquant.mat_dims(d, I)

    def zero():
        return {m: {"codes": np.zeros(dims[m], np.uint8),
                    "scales": np.zeros((dims[m][0], dims[m][1] // 64), np.float16),
                    "biases": np.zeros((dims[m][0], dims[m][1] // 64), np.float16)}
                for m in oquant.MATS}
    for mat, row, col, val, off, byte in codes:
        raw = zero()
        raw[mat]["codes"][row, col] = val
        blob = oquant.pack_expert(raw, d, I, bits)
        assert blob.size == stride
        nz = np.nonzero(blob)[0]
        assert nz.tolist() == [off] and blob[off] == byte
    for mat, row, g, soff, boff in sbs:
        raw = zero()
        raw[mat]["scales"][row, g] = np.float16(0.5)      # 0x3800
        raw[mat]["biases"][row, g] = np.float16(-2.0)     # 0xC000
        blob = oquant.pack_expert(raw, d, I, bits)
        assert blob[soff:soff + 2].tobytes() == b"\x00\x38"
        assert blob[boff:boff + 2].tobytes() == b"\x00\xc0"
        assert np.count_nonzero(blob) == 2
    for mat, row, col, val, off, bits32 in weights:
        raw = {m: {"weights": np.zeros(dims[m], np.float32)} for m in oquant.MATS}
        raw[mat]["weights"][row, col] = val
        blob = oquant.pack_expert(raw, d, I, bits)
        assert blob.size == stride
        assert blob[off:off + 4].tobytes() == int(bits32).to_bytes(4, "little")
        assert np.count_nonzero(blob) == np.count_nonzero(blob[off:off + 4])


@pytest.mark.parametrize("bits", [4, 8, 32])
def test_pack_roundtrip(bits):
    small = {4: TINY, 8: ms.CONFIGS["tiny_int8"], 32: ms.CONFIGS["tiny_f32"]}[bits]
    big = ms.scaled(ms.CONFIGS["decode80b"], bits=bits)
    for cfg in (small, big):
        raw = ms.expert_raw(cfg, 9)
        blob = oquant.pack_expert(raw, cfg.d, cfg.I, bits)
        assert blob.size == oquant.blob_stride(cfg.d, cfg.I, bits)
        assert not blob[oquant.blob_bytes(cfg.d, cfg.I, bits):].any()
        back = oquant.unpack_expert(blob, cfg.d, cfg.I, bits)
        for m in oquant.MATS:
            for f in raw[m]:
                assert np.array_equal(back[m][f], raw[m][f])
        assert np.array_equal(oquant.pack_expert(back, cfg.d, cfg.I, bits), blob)
    # 80B shape: 27/16 and 51/16 bytes per weight, already multiples of 4096
    assert oquant.blob_bytes(2048, 512) == 1769472 == oquant.blob_stride(2048, 512)
    assert oquant.blob_bytes(2048, 512, 8) == 3342336 == oquant.blob_stride(2048, 512, 8)
    assert oquant.blob_bytes(2048, 512, 32) == 12582912 == oquant.blob_stride(2048, 512, 32)


def test_int8_codes_are_bytes():
    """Every 8-bit code is one byte of the blob, each byte of the codes
    sections holds one code (a permutation of the codes, nothing lost or
    merged), and the (scale, bias) sections are the 4-bit ones."""
    cfg = ms.CONFIGS["tiny_int8"]
    raw = ms.expert_raw(cfg, 2)
    blob = oquant.pack_expert(raw, cfg.d, cfg.I, 8)
    off = 0
    for m in oquant.MATS:
        o, i = oquant.mat_dims(cfg.d, cfg.I)[m]
        sec = blob[off:off + o * i]
        assert np.array_equal(np.sort(sec), np.sort(raw[m]["codes"].ravel()))
        off += o * i
        sb = blob[off:off + (i // 64) * o * 4].view(np.float16).reshape(i // 64, o, 2)
        assert np.array_equal(sb[:, :, 0].T, raw[m]["scales"])
        assert np.array_equal(sb[:, :, 1].T, raw[m]["biases"])
        off += (i // 64) * o * 4
    assert off == oquant.blob_bytes(cfg.d, cfg.I, 8)


def test_int8_with_4bit_codes_is_the_int4_expert():
    """An 8-bit expert whose codes all lie in 0..15 is the same function as
    the 4-bit expert with those codes, scales and biases (MLX affine
    dequantisation does not depend on the code width)."""
    raw4 = ms.expert_raw(TINY, 4)
    x = ms.bf16_bits_to_f32(ms.x_bits(TINY, 1)).astype(np.float64)
    y4 = olayer.expert_ffn(raw4, x)
    blob8 = oquant.pack_expert(raw4, TINY.d, TINY.I, 8)
    raw8 = oquant.unpack_expert(blob8, TINY.d, TINY.I, 8)
    assert np.array_equal(olayer.expert_ffn(raw8, x), y4)


def test_f32_expert_is_its_weights():
    """An f32 expert whose weights are the dequantised weights of a 4-bit
    expert is the same function as that expert (both compute
    W_d (silu(W_g x) * W_u x) on the same matrices)."""
    raw4 = ms.expert_raw(TINY, 6)
    raw32 = {m: {"weights": oquant.dequant(raw4[m]).astype(np.float32)} for m in oquant.MATS}
    for m in oquant.MATS:    # the 4-bit weights are exact in fp32 (pinned above)
        assert np.array_equal(oquant.dequant(raw32[m]), oquant.dequant(raw4[m]))
    x = ms.bf16_bits_to_f32(ms.x_bits(TINY, 2)).astype(np.float64)
    assert np.array_equal(olayer.expert_ffn(raw32, x), olayer.expert_ffn(raw4, x))


def test_int8_dequant_exact_in_fp32():
    """s*q + b with fp16 s, b = -128 s and q in 0..255 is s*(q-128): at most
    11 + 8 significant bits, exactly representable in fp32."""
    raw = ms.expert_raw(ms.CONFIGS["decode80b_int8"], 5)
    for m in raw.values():
        W = oquant.dequant(m)
        assert np.array_equal(W.astype(np.float32).astype(np.float64), W)
        assert np.array_equal(W, m["scales"].astype(np.float64).repeat(64, 1)
                              * (m["codes"].astype(np.float64) - 128))


# ---- P8: placement invariance (oracle reading blobs through a slot table) ---
def test_placement_invariance_oracle():
    cfg = TINY
    Wr = ms.router_weight(cfg)
    xb = ms.x_bits(cfg, 0)
    stride = oquant.blob_stride(cfg.d, cfg.I)
    blobs = [oquant.pack_expert(ms.expert_raw(cfg, e), cfg.d, cfg.I) for e in range(cfg.E)]
    sh = ms.shared_raw(cfg)
    ys = []
    for perm_seed in (None, 1, 2):
        table = np.arange(cfg.E) if perm_seed is None else \
            np.random.default_rng(perm_seed).permutation(cfg.E)
        pool = np.zeros(cfg.E * stride, np.uint8)
        for e in range(cfg.E):
            pool[table[e] * stride:(table[e] + 1) * stride] = blobs[e]

        def fetch(e, pool=pool, table=table):
            s = int(table[e])
            return oquant.unpack_expert(pool[s * stride:(s + 1) * stride], cfg.d, cfg.I)
        ys.append(olayer.moe_layer(xb, Wr, None, cfg.k, fetch, sh)["y"])
    assert all(np.array_equal(ys[0], y) for y in ys[1:])


# ---- P9: token independence (incremental vs whole) --------------------------
def test_token_independence():
    cfg = TINY
    Wr = ms.router_weight(cfg)
    xb = ms.x_bits(cfg, 4)
    ex = _tiny_experts(cfg)
    sh = ms.shared_raw(cfg)
    whole = olayer.moe_layer(xb, Wr, None, cfg.k, ex, sh)
    for t in range(cfg.T):
        one = olayer.moe_layer(xb[t:t + 1], Wr, None, cfg.k, ex, sh)
        assert one["idx"][0].tolist() == whole["idx"][t].tolist()
        assert np.allclose(one["y"][0], whole["y"][t], rtol=1e-13, atol=1e-15)


# ---- P12: bucketing = stable counting sort -----------------------------------
def test_bucketing_bruteforce():
    g = np.random.default_rng(11)
    for T, k, E in ((1, 10, 512), (64, 10, 512), (7, 3, 5), (33, 4, 1024)):
        idx = np.stack([g.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
        counts, offsets, pair_ids = obucket.bucket(idx, E)
        flat = idx.ravel()
        ref = sorted(range(T * k), key=lambda i: (flat[i], i))
        assert pair_ids.tolist() == ref
        assert counts.sum() == T * k and offsets[-1] == T * k and offsets[0] == 0
        for e in range(E):
            seg = pair_ids[offsets[e]:offsets[e + 1]]
            assert len(seg) == counts[e] == (flat == e).sum()
            assert (flat[seg] == e).all() and (np.diff(seg) > 0).all()


# ---- P13 (oracle side): LFU + recency vs hand-derived traces -----------------
def test_lfu_golden_traces():
    for name, E, slots, steps in golden_io.lfu_traces():
        sim = olfu.SlotPoolSim(E, slots)
        for sel, loads, hits in steps:
            h0 = sim.hits
            got = sim.plan(sel)
            assert got == loads, (name, sel)
            assert sim.hits - h0 == hits, (name, sel)


def test_lfu_pool_too_small():
    sim = olfu.SlotPoolSim(4, 1)
    with pytest.raises(ValueError):
        sim.plan([0, 1])


# ---- certified near-tie bound is a true bound ---------------------------------
def test_logit_error_bound_holds_for_fp32_sums():
    cfg = ms.CONFIGS["decode80b"]
    Wr = ms.router_weight(cfg)
    b = ms.logit_bias(cfg)
    xb = ms.x_bits(cfg, 0)
    x32 = ms.bf16_bits_to_f32(xb)
    exact, _ = olayer.router_logits(olayer.bf16_to_f64(xb), Wr, b)
    # a plain sequential fp32 sum has depth d; bound must cover it
    seq = np.zeros(cfg.E, np.float32)
    for j in range(cfg.d):
        seq = (seq + x32[0, j] * Wr[:cfg.E, j]).astype(np.float32)
    seq = (seq + b).astype(np.float32)
    r = olayer.logit_error_bound(xb, Wr, b, depth=cfg.d)
    assert np.max(np.abs(seq - exact[0])) <= r[0]


def test_elementwise_logit_bounds_hold_for_fp32_sums():
    """The elementwise bound covers every router row (the shared-gate row
    included) of two real fp32 summation orders: a sequential sum (depth d)
    and a pairwise tree (depth log2 d).  A bound with a dropped |.|, a wrong
    row or a depth unit off by a factor fails on one of them."""
    cfg = ms.CONFIGS["decode80b"]
    Wr = ms.router_weight(cfg)
    xb = ms.x_bits(cfg, 1, 3)
    x32 = ms.bf16_bits_to_f32(xb)
    exact = olayer.bf16_to_f64(xb) @ Wr.astype(np.float64).T              # [T, E+1]
    for t in range(xb.shape[0]):
        prod = (x32[t][None, :] * Wr).astype(np.float32)                  # [E+1, d], fp32 products
        seq = np.zeros(cfg.E + 1, np.float32)
        for j in range(cfg.d):
            seq = (seq + prod[:, j]).astype(np.float32)
        tree = prod.copy()
        while tree.shape[1] > 1:
            tree = (tree[:, 0::2] + tree[:, 1::2]).astype(np.float32)
        r_seq = olayer.logit_error_bounds(xb[t:t + 1], Wr, depth=cfg.d)[0]
        r_tree = olayer.logit_error_bounds(xb[t:t + 1], Wr, depth=int(np.log2(cfg.d)))[0]
        assert np.all(np.abs(seq - exact[t]) <= r_seq)
        assert np.all(np.abs(tree[:, 0] - exact[t]) <= r_tree)
        # the pairwise tree is far inside the sequential bound: the depth matters
        assert np.max(r_tree) < np.max(r_seq) / 100
    # the per-token routed-row bound is the row maximum of the elementwise one
    # (no bias)
    r_all = olayer.logit_error_bounds(xb, Wr, depth=17)
    r_tok = olayer.logit_error_bound(xb, Wr, None, depth=17)
    assert np.allclose(r_all[:, :cfg.E].max(1), r_tok, rtol=1e-12, atol=0)


# ---- chains of MoE layers: norm, residual, bf16 rounding -------------------
def test_bf16_round_hand_values_and_generator_agree():
    """Round-to-nearest-even onto bf16 at hand-checked points (ties go to the
    even mantissa), and agreement with the input generator's independent
    rounding on random values."""
    v = np.float32([1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.5, 1 + 2 ** -7 + 2 ** -9, 0.0, -0.0])
    assert olayer.bf16_round(v).tolist() == [0x3F80, 0x3F82, 0xC020, 0x3F81, 0x0000, 0x8000]
    r = np.random.default_rng(3).standard_normal(100000).astype(np.float32) * 37
    assert np.array_equal(olayer.bf16_round(r), ms.f32_to_bf16_bits(r))


def test_rms_norm_closed_forms():
    # constant row: x / sqrt(x^2 + eps) rounds to 1.0 in bf16
    x = np.full((2, 256), 0x4000, np.uint16)                    # 2.0
    assert np.all(olayer.rms_norm_bf16(x) == 0x3F80)
    # (3, -4): mean square 12.5, u = (0.84853, -1.13137) -> bf16 0.84765625, -1.1328125
    x = np.array([[0x4040, 0xC080]], np.uint16)
    assert olayer.rms_norm_bf16(x).tolist() == [[0x3F59, 0xBF91]]
    # scale invariance up to eps: a power-of-two scale leaves u unchanged
    xb = ms.x_bits(TINY, 3)
    xs = ms.f32_to_bf16_bits(ms.bf16_bits_to_f32(xb) * np.float32(8.0))
    assert np.array_equal(olayer.rms_norm_bf16(xb, 0.0), olayer.rms_norm_bf16(xs, 0.0))


def test_residual_rounding_and_zero_layer():
    one = np.array([0x3F80], np.uint16)
    assert olayer.residual_bf16(one, np.array([2.0 ** -8])).tolist() == [0x3F80]       # tie -> even
    assert olayer.residual_bf16(one, np.array([3 * 2.0 ** -8])).tolist() == [0x3F82]   # tie -> even (up)
    # a layer whose experts all have zero down matrices adds nothing
    cfg = TINY
    zero_down = lambda raw: {**raw, "down": {"codes": np.zeros_like(raw["down"]["codes"]),
                                             "scales": raw["down"]["scales"],
                                             "biases": np.zeros_like(raw["down"]["biases"])}}
    ex = _tiny_experts(cfg)
    layer = dict(w_router=ms.router_weight(cfg), bias=None, k=cfg.k,
                 expert=lambda e: zero_down(ex(e)), shared=zero_down(ms.shared_raw(cfg)))
    xb = ms.x_bits(cfg, 2)
    xn, u, res = olayer.chain_layer(xb, layer)
    assert np.array_equal(xn, xb) and not res["y"].any()
    assert np.array_equal(u, olayer.rms_norm_bf16(xb))
