"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle.

Bars: routing indices, bucket offsets and pair lists bit-exact (up to
certified near-ties of fp32 logits, where any correct choice is accepted and
the output is compared with the oracle run on the device's choice); weights
and gates within fp32 rounding; layer outputs within
max|y - y_ref| <= 2e-3 * max|y_ref| per step; runs that differ only in expert
placement bit-identical.
"""
import numpy as np
import pytest

import moe_synth as ms
from oracle import bucket as obucket
from oracle import layer as olayer
from gpu_support import (DeviceLayer, certify_routing, assert_close_y, check_device_logits,
                         predicted_near_ties)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
moe = pytest.importorskip("sparse_moe_decode_router_amd")

TINY = ms.CONFIGS["tiny"]


@pytest.fixture(scope="module")
def tiny():
    return DeviceLayer(TINY)


@pytest.fixture(scope="module")
def l35():
    return DeviceLayer(ms.CONFIGS["decode35b"])


@pytest.fixture(scope="module")
def l80():
    return DeviceLayer(ms.scaled(ms.CONFIGS["decode80b"], n_slots=512))


def _np(t):
    return t.detach().cpu().numpy()


def _check_layer_step(L, step, path=moe.MOE_PATH_AUTO, T=None):
    xb, x = L.x(step, T)
    y, idx, w, s = moe.moe_layer_forward(L.layer, x, path=path)
    torch.cuda.synchronize()
    idx_np = _np(idx)
    depth = moe.moe_router_sum_depth(xb.shape[0], L.cfg.d, L.cfg.E)
    namb, amb = certify_routing(xb, L.Wr_np, L.bias_np, L.cfg.k, idx_np, depth)
    ref = L.oracle(xb, idx=idx_np if namb else None)
    assert np.array_equal(idx_np, ref["idx"])
    assert np.allclose(_np(w), ref["w"], rtol=0, atol=2e-5)
    assert np.allclose(_np(s), ref["s"], rtol=0, atol=2e-6)
    rel = [assert_close_y(_np(y)[t:t + 1], ref["y"][t:t + 1]) for t in range(xb.shape[0])]
    return max(rel), namb, _np(y), idx_np


# ------------------------------------------------------------------ router
@pytest.mark.parametrize("name,T", [("tiny", 4), ("decode35b", 1), ("decode80b", 1), ("decode80b", 3),
                                    ("decode80b", 8), ("decode80b", 64), ("decode80b", 300),
                                    ("decode80b", 4096), ("prefill80b", 4096)])
def test_router_parity(name, T):
    """Both routers (per-row GEMVs up to 8 tokens, the matrix cores beyond):
    every device logit within the fp32 rounding bound of its summation depth,
    the selection the exact top k of the device's own logits on every token,
    and the selection equal to the exact one wherever the bound separates the
    exact logits (certified); usage counters equal the selections."""
    _router_parity(ms.CONFIGS[name], name, T)


@pytest.mark.parametrize("T,d,E,k", [(129, 192, 7, 2), (40, 64, 33, 4), (300, 320, 65, 8), (257, 640, 100, 6)])
def test_router_mfma_ragged_shapes(T, d, E, k):
    """The matrix-core router where its tiles are ragged: an odd number of
    64-wide stages per split (3, 1, 5, and 5 with two splits), a last token
    tile of 1 or 44 rows, router rows far short of a 64-row tile (E + 1 = 8)
    or just past one (66), and tile grids that are not a multiple of 8."""
    cfg = ms.scaled(ms.CONFIGS["decode80b"], d=d, E=E, k=k)
    _router_parity(cfg, f"d{d}_E{E}", T)


def _router_parity(cfg, name, T):
    Wr = ms.router_weight(cfg)
    bias = ms.logit_bias(cfg)
    Wd = torch.from_numpy(Wr).cuda()
    bd = None if bias is None else torch.from_numpy(bias).cuda()
    usage = torch.zeros(cfg.E, dtype=torch.int32, device="cuda")
    total = np.zeros(cfg.E, np.int64)
    depth = moe.moe_router_sum_depth(T, cfg.d, cfg.E)
    steps = 3 if T < 1024 else 1
    namb_all, predicted, worst = 0, 0.0, 0.0
    for step in range(steps):
        xb = ms.x_bits(cfg, step, T)
        x = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
        idx, w, s, l = moe.moe_router_topk_logits(x, Wd, bd, cfg.k, usage_ptr=usage.data_ptr())
        torch.cuda.synchronize()
        idx, w, l = _np(idx), _np(w), _np(l)
        worst = max(worst, check_device_logits(xb, Wr, bias, cfg.k, idx, w, l, depth))
        namb, amb = certify_routing(xb, Wr, bias, cfg.k, idx, depth)
        namb_all += namb
        predicted += predicted_near_ties(xb, Wr, bias, cfg.k, depth)
        _, _, ref_s, _ = olayer.route(xb, Wr, bias, cfg.k)
        lx, _ = olayer.router_logits(olayer.bf16_to_f64(xb), Wr, bias)
        assert np.allclose(w, olayer.topk_weights(lx, idx), rtol=0, atol=2e-5)   # weights of its own choice
        assert np.allclose(w.sum(1), 1.0, atol=1e-5)
        assert np.allclose(_np(s), ref_s, rtol=0, atol=2e-6)
        total += np.bincount(idx.ravel(), minlength=cfg.E)
    assert np.array_equal(_np(usage).astype(np.int64), total)
    # tokens whose exact logits sit closer than the certified bound at some
    # rank boundary (every device choice there was checked above against its
    # own logits and the bound): their number must be what the bound's width
    # predicts under exponential spacings of the top logits
    print(f"{name} T={T} depth {depth}: {namb_all} of {steps * T} tokens within the near-tie bound "
          f"(predicted {predicted:.1f}); largest logit error {worst:.3f} of the bound")
    assert namb_all <= 2 * predicted + 2


def test_router_tie_rule_on_device():
    """Identical router rows give identical fp32 logits; the lower index wins."""
    cfg = TINY
    Wr = ms.router_weight(cfg).copy()
    Wr[9] = Wr[2]
    b = np.zeros(cfg.E, np.float32)
    b[2] = b[9] = 40.0
    x = torch.from_numpy(ms.x_bits(cfg, 0).view(np.int16)).cuda().view(torch.bfloat16)
    idx, w, _ = moe.moe_router_topk(x, torch.from_numpy(Wr).cuda(), torch.from_numpy(b).cuda(), 2)
    idx = _np(idx)
    assert (idx[:, 0] == 2).all() and (idx[:, 1] == 9).all()
    assert np.allclose(_np(w), 0.5, atol=1e-6)


@pytest.mark.parametrize("k", [1, 16])
def test_router_k_extremes(k):
    cfg = TINY
    Wr = ms.router_weight(cfg)
    xb = ms.x_bits(cfg, 1)
    x = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
    idx, w, _ = moe.moe_router_topk(x, torch.from_numpy(Wr).cuda(), None, k)
    idx, w = _np(idx), _np(w)
    certify_routing(xb, Wr, None, k, idx, moe.moe_router_sum_depth(cfg.T, cfg.d, cfg.E))
    if k == 1:
        assert (w == 1.0).all()
    else:                                    # k = E: the full softmax
        l, _ = olayer.router_logits(olayer.bf16_to_f64(xb), Wr, None)
        p = np.exp(l - l.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        assert np.allclose(np.take_along_axis(p, idx.astype(np.int64), 1), w, atol=2e-6)


@pytest.mark.parametrize("T", [3, 40])
@pytest.mark.parametrize("E,k", [(256, 80), (1024, 100)])
def test_router_k_above_64(E, k, T):
    """k > 64: the top-k skips its threshold search and ranks every key as a
    candidate; both routers (T = 3 on the per-row GEMVs, T = 40 on the matrix
    cores), under the same certified comparison as test_router_parity."""
    cfg = ms.scaled(ms.CONFIGS["decode80b"], d=512, E=E, k=k, I=64, I_shared=64, n_slots=E)
    _router_parity(cfg, f"E{E}_k{k}", T)


# ---------------------------------------------------------------- bucketing
# (the multi-block scan runs in LDS up to 24576 histogram entries: 4096 x 10
# of 512 is 20480; 2048 x 16 of 1024 is 32768, the scan from global memory)
@pytest.mark.parametrize("T,k,E", [(1, 10, 512), (4, 2, 16), (64, 10, 512), (100, 10, 512),
                                   (700, 3, 1024), (4096, 10, 512), (2048, 16, 1024), (5, 7, 7)])
def test_bucket_bit_exact(T, k, E):
    g = np.random.default_rng(T * 1000 + k)
    idx = np.stack([g.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    if T >= 64:   # skew: many pairs in a few buckets
        hot = g.random(idx.shape) < 0.3
        idx[hot] = np.minimum(idx[hot] % 5, E - 1)
        for t in range(T):       # restore distinctness within a token
            seen = set()
            for r in range(k):
                while int(idx[t, r]) in seen:
                    idx[t, r] = (idx[t, r] + 7) % E
                seen.add(int(idx[t, r]))
    c, o, p = moe.moe_bucket_tokens(torch.from_numpy(idx).cuda(), E)
    rc, ro, rp = obucket.bucket(idx, E)
    assert np.array_equal(_np(c), rc) and np.array_equal(_np(o), ro) and np.array_equal(_np(p), rp)


# ------------------------------------------------------------ decode layer
def test_tiny_layer_parity(tiny):
    worst = 0
    for step in range(TINY.steps):
        rel, _, _, _ = _check_layer_step(tiny, step)
        worst = max(worst, rel)
    print(f"tiny worst rel err {worst:.2e}")


def test_decode35b_parity(l35):
    worst = max(_check_layer_step(l35, s)[0] for s in range(4))
    print(f"35B decode worst rel err {worst:.2e}")


def test_decode80b_parity(l80):
    worst = max(_check_layer_step(l80, s)[0] for s in range(4))
    print(f"80B decode worst rel err {worst:.2e}")


def test_decode80b_small_T(l80):
    for T in (2, 4, 8):
        _check_layer_step(l80, 10 + T, path=moe.MOE_PATH_DECODE, T=T)


def test_batched80b_parity(l80):
    rel, namb, y, idx = _check_layer_step(l80, 0, path=moe.MOE_PATH_BATCHED, T=64)
    print(f"80B batched T=64 rel err {rel:.2e}, ambiguous {namb}")


def test_token_independence(l80):
    """Row t of a T=64 batched call vs a T=1 decode call on x_t: routing
    bit-identical, outputs within tolerance of each other."""
    xb, x = l80.x(5, 64)
    yb, ib, _, _ = moe.moe_layer_forward(l80.layer, x, path=moe.MOE_PATH_BATCHED)
    torch.cuda.synchronize()
    # the two paths sum logits in different orders: tokens inside the
    # certified near-tie bound of either may legitimately route differently
    _, amb = certify_routing(xb, l80.Wr_np, l80.bias_np, l80.cfg.k, _np(ib),
                             moe.moe_router_sum_depth(64, l80.cfg.d, l80.cfg.E))
    for t in [t for t in range(64) if not amb[t]][:6]:
        y1, i1, _, _ = moe.moe_layer_forward(l80.layer, x[t:t + 1].contiguous(), path=moe.MOE_PATH_DECODE)
        torch.cuda.synchronize()
        assert np.array_equal(_np(i1)[0], _np(ib)[t])
        assert_close_y(_np(y1)[0], _np(yb)[t].astype(np.float64))


# ------------------------------------------------------- shape envelope
# The edges of what the kernels accept: intermediates wider than 512 (the
# down GEMVs' extra-group loops), the largest expert count (E = 1024, k = 16:
# the widest top-k), the largest hidden size (d = 8192) and k = E (every
# expert selected).  Each on the decode, batched and prefill paths.
ENVELOPE = {
    "wide_I": dict(d=512, E=32, k=4, I=1024, I_shared=1024, n_slots=32),
    "max_E": dict(d=512, E=1024, k=16, I=128, I_shared=128, n_slots=1024),
    "max_d": dict(d=8192, E=16, k=2, I=128, I_shared=128, n_slots=16),
    "k_eq_E": dict(d=256, E=16, k=16, I=64, I_shared=64, n_slots=16),
    # k steps of the tiled GEMMs a multiple of three (gate/up 12, down 6): the
    # unrolled rounds of three steps with no remainder after them
    "steps_3n": dict(d=768, E=32, k=4, I=384, I_shared=384, n_slots=32),
}


@pytest.mark.parametrize("name", sorted(ENVELOPE))
def test_envelope_decode_and_batched(name):
    L = DeviceLayer(ms.scaled(ms.CONFIGS["decode80b"], alpha=0.0, **ENVELOPE[name]))
    _check_layer_step(L, 0, path=moe.MOE_PATH_DECODE, T=1)
    _check_layer_step(L, 1, path=moe.MOE_PATH_DECODE, T=4)
    _check_layer_step(L, 3, path=moe.MOE_PATH_DECODE, T=8)      # the decode router's widest instance
    _check_layer_step(L, 2, path=moe.MOE_PATH_BATCHED, T=24)
    assert L.pool.check_error() == moe.MOE_OK


@pytest.mark.parametrize("name", sorted(ENVELOPE))
def test_envelope_prefill(name):
    cfg = ms.scaled(ms.CONFIGS["prefill80b"], T=160, **ENVELOPE[name])
    L = DeviceLayer(cfg)
    rel, namb, _ = _prefill_check(L, 0, cfg.T)
    print(f"prefill {name}: rel err {rel:.2e}, near-ties {namb}")


def test_decode_router_preps_every_group_with_few_experts():
    """T = 8 tokens of d = 8192 make T d / 64 = 1024 activation groups, more than
    the threads of the decode router's grid when E = 2 (three blocks): every
    group is still prepared for the GEMVs.  Step 1 would read step 0's
    activations in a group left unprepared."""
    L = DeviceLayer(ms.scaled(ms.CONFIGS["decode80b"], alpha=0.0, d=8192, E=2, k=1, I=128,
                              I_shared=128, n_slots=2))
    for step in range(2):
        _check_layer_step(L, step, path=moe.MOE_PATH_DECODE, T=8)
    assert L.pool.check_error() == moe.MOE_OK


def test_layer_k_above_64():
    """A layer that sends each token to 72 of 128 experts (the top-k's k > 64
    branch inside the decode gate/up kernel, 584 down instances at T = 8) on
    the decode, batched and prefill paths."""
    cfg = ms.scaled(ms.CONFIGS["decode80b"], alpha=0.0, d=256, E=128, k=72, I=64, I_shared=64, n_slots=128)
    L = DeviceLayer(cfg)
    _check_layer_step(L, 0, path=moe.MOE_PATH_DECODE, T=1)
    _check_layer_step(L, 1, path=moe.MOE_PATH_DECODE, T=8)
    _check_layer_step(L, 2, path=moe.MOE_PATH_BATCHED, T=24)
    assert L.pool.check_error() == moe.MOE_OK
    rel, namb, _ = _prefill_check(L, 3, 160)
    print(f"k = 72 prefill: rel err {rel:.2e}, near-ties {namb}")


# ------------------------------------------------------ placement invariance
def test_placement_invariance_bit_identical():
    """Two pools holding the same experts at different slots, and a smaller
    pool refilled step by step through LFU + recency: identical bits."""
    cfg = ms.scaled(ms.CONFIGS["decode80b"], E=64, k=6, steps=12)
    A = DeviceLayer(cfg, table=np.arange(cfg.E))
    B = DeviceLayer(cfg, table=np.random.default_rng(3).permutation(cfg.E))
    C_ = DeviceLayer(cfg, table=None, n_slots=16)        # starts empty
    host = torch.from_numpy(np.stack([A.blob(e) for e in range(cfg.E)])).pin_memory()
    for step in range(cfg.steps):
        xb, x = A.x(step)
        ya, ia, _, _ = moe.moe_layer_forward(A.layer, x)
        yb, ib, _, _ = moe.moe_layer_forward(B.layer, x)
        # partial residency: route, refill the pool, then run the experts
        idx, w, s = moe.moe_router_topk(x, C_.Wr, C_.bias, cfg.k)
        torch.cuda.synchronize()
        C_.pool.refill(_np(idx).ravel(), host, A.pool.stride)
        yc = moe.moe_expert_ffn_int4(C_.pool, C_.shared_blob, cfg.I_shared, x, idx, w, s)
        torch.cuda.synchronize()
        assert np.array_equal(_np(ia), _np(ib)) and np.array_equal(_np(ia), _np(idx))
        assert np.array_equal(_np(ya), _np(yb))
        assert np.array_equal(_np(ya), _np(yc))
    st = C_.pool.stats()
    assert st["misses"] > 0 and st["hits"] > 0
    assert C_.pool.check_error() == moe.MOE_OK


def test_pool_state_after_refill():
    cfg = ms.scaled(TINY, E=16, k=2)
    L = DeviceLayer(cfg, table=None, n_slots=4)
    host = torch.from_numpy(np.stack([L.blob(e) for e in range(cfg.E)])).pin_memory()
    sel_steps = [[3, 5], [3, 9], [1, 2], [5, 3]]
    from oracle import lfu as olfu
    sim = olfu.SlotPoolSim(cfg.E, 4)
    for sel in sel_steps:
        L.pool.refill(sel, host, L.pool.stride)
        sim.plan(sel)
    table, _ = L.pool.read_state()
    assert table.tolist() == sim.slot_of


def test_not_resident_sets_error_word():
    cfg = ms.scaled(TINY, E=16, k=2)
    L = DeviceLayer(cfg, table=np.arange(16), resident=[0, 1, 2])    # most experts absent
    _, x = L.x(0)
    moe.moe_layer_forward(L.layer, x)
    assert L.pool.check_error() == moe.MOE_ERR_NOT_RESIDENT
    assert L.pool.check_error() == moe.MOE_OK        # cleared by the read


def test_shared_intermediate_differs():
    cfg = ms.scaled(TINY, I=64, I_shared=128, d=512)
    L = DeviceLayer(cfg)
    for path in (moe.MOE_PATH_DECODE, moe.MOE_PATH_BATCHED):
        _check_layer_step(L, 1, path=path)


def test_usage_counters_match_selections(l35):
    l35.pool.reset_usage()
    tot = np.zeros(l35.cfg.E, np.int64)
    for step in range(5):
        _, x = l35.x(100 + step)
        _, idx, _, _ = moe.moe_layer_forward(l35.layer, x)
        torch.cuda.synchronize()
        tot += np.bincount(_np(idx).ravel(), minlength=l35.cfg.E)
    _, usage = l35.pool.read_state()
    assert np.array_equal(usage.astype(np.int64), tot)


def test_zero_tokens_is_noop(tiny):
    x = torch.empty((0, TINY.d), dtype=torch.bfloat16, device="cuda")
    y, idx, w, s = moe.moe_layer_forward(tiny.layer, x)
    assert y.shape == (0, TINY.d)


# ----------------------------------------------------------------- prefill
def _prefill_check(L, step, T, sample=None):
    xb, x = L.x(step, T)
    y, idx, w, s = moe.moe_layer_forward(L.layer, x, path=moe.MOE_PATH_PREFILL)
    torch.cuda.synchronize()
    assert L.pool.check_error() == moe.MOE_OK
    idx_np, y_np = _np(idx), _np(y)
    rows = np.arange(T) if sample is None else sample
    depth = moe.moe_router_sum_depth(T, L.cfg.d, L.cfg.E)
    namb, _ = certify_routing(xb[rows], L.Wr_np, L.bias_np, L.cfg.k, idx_np[rows], depth)
    ref = L.oracle(xb[rows], idx=idx_np[rows])
    assert np.allclose(_np(w)[rows], ref["w"], rtol=0, atol=2e-5)
    rel = assert_close_y(y_np[rows], ref["y"])      # one prefill tensor
    return rel, namb, idx_np


def test_prefill_midsize_full_oracle():
    """T=512 tokens, E=32, k=8 (128 tokens per expert on average, several
    chunks per bucket), d=512, I=128: every output against the oracle."""
    cfg = ms.scaled(ms.CONFIGS["prefill80b"], T=512, E=32, k=8, d=512, I=128, I_shared=128,
                    n_slots=32)
    L = DeviceLayer(cfg)
    rel, namb, _ = _prefill_check(L, 0, cfg.T)
    print(f"prefill midsize rel err {rel:.2e}, near-ties {namb}")


def test_prefill_matches_batched_path():
    """The MFMA path and the GEMV path agree within the output tolerance."""
    cfg = ms.scaled(ms.CONFIGS["prefill80b"], T=256, E=64, k=8, d=1024, I=256, I_shared=256,
                    n_slots=64)
    L = DeviceLayer(cfg)
    _, x = L.x(3, cfg.T)
    yp, ip, _, _ = moe.moe_layer_forward(L.layer, x, path=moe.MOE_PATH_PREFILL)
    yb, ib, _, _ = moe.moe_layer_forward(L.layer, x, path=moe.MOE_PATH_BATCHED)
    torch.cuda.synchronize()
    assert np.array_equal(_np(ip), _np(ib))
    assert_close_y(_np(yp), _np(yb).astype(np.float64))


def test_batched_small_d_partial_row_block():
    """d = 192 (not a multiple of the 256-row down tile) on the batched path."""
    cfg = ms.scaled(TINY, d=192, I=64, I_shared=64, T=12, E=16, k=3)
    L = DeviceLayer(cfg)
    _check_layer_step(L, 2, path=moe.MOE_PATH_BATCHED, T=12)


def test_auto_path_choice(l80):
    """MOE_PATH_AUTO: the decode GEMVs up to 8 tokens, the grouped GEMMs
    beyond (bit-identical to the explicit paths), the bucketed GEMVs when d
    is not a multiple of 128."""
    for T, path in ((8, moe.MOE_PATH_DECODE), (9, moe.MOE_PATH_PREFILL), (64, moe.MOE_PATH_PREFILL)):
        _, x = l80.x(30 + T, T)
        ya, ia, _, _ = moe.moe_layer_forward(l80.layer, x)
        ye, ie, _, _ = moe.moe_layer_forward(l80.layer, x, path=path)
        torch.cuda.synchronize()
        assert np.array_equal(_np(ia), _np(ie)) and np.array_equal(_np(ya), _np(ye)), T
    cfg = ms.scaled(TINY, d=192, I=64, I_shared=64, T=12, E=16, k=3)
    L = DeviceLayer(cfg)
    _, x = L.x(1, 12)
    ya, _, _, _ = moe.moe_layer_forward(L.layer, x)
    ye, _, _, _ = moe.moe_layer_forward(L.layer, x, path=moe.MOE_PATH_BATCHED)
    torch.cuda.synchronize()
    assert np.array_equal(_np(ya), _np(ye))


@pytest.mark.parametrize("path", ["batched", "prefill"])
def test_usage_counters_bucketed_paths(l80, path):
    """On the bucketed paths the usage counters are added from the bucket
    counts: the same totals as one count per selection."""
    p = moe.MOE_PATH_BATCHED if path == "batched" else moe.MOE_PATH_PREFILL
    l80.pool.reset_usage()
    tot = np.zeros(l80.cfg.E, np.int64)
    for step, T in ((40, 64), (41, 9), (42, 200)):
        _, x = l80.x(step, T)
        _, idx, _, _ = moe.moe_layer_forward(l80.layer, x, path=p)
        torch.cuda.synchronize()
        tot += np.bincount(_np(idx).ravel(), minlength=l80.cfg.E)
    _, usage = l80.pool.read_state()
    assert np.array_equal(usage.astype(np.int64), tot)


# -------------------------------------------- matrix cores: streaming GEMMs
# The two grouped-GEMM kernel sets of the matrix-core path (tiled: chunks of
# up to 128 tokens staged step by step; streaming: chunks of up to 16 tokens
# whose activations stay in LDS while the weights stream) do the same fp16
# products in the same order, so they give the same bits; both are checked
# against the oracle.  Cases: the 80B shape at 64 tokens, 200 Zipf tokens
# (buckets above 16 tokens split into several chunks), intermediate 1024,
# E = 1024 with k = 16, intermediate 64 (a half tile), a shared expert wider
# than the routed ones, and 8-bit codes.
STREAM = {
    "80b_T64": (dict(), 64),
    "80b_T200": (dict(), 200),
    "wide_I": (dict(d=512, E=32, k=4, I=1024, I_shared=1024, n_slots=32, alpha=0.0), 24),
    "max_E": (dict(d=512, E=1024, k=16, I=128, I_shared=128, n_slots=1024, alpha=0.0), 24),
    "half_tile": (dict(d=256, E=16, k=16, I=64, I_shared=64, n_slots=16, alpha=0.0), 24),
    "shared_wider": (dict(d=512, E=64, k=6, I=64, I_shared=192, n_slots=64, alpha=0.0), 40),
}


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("name", sorted(STREAM))
def test_stream_gemms_match_tiled_and_oracle(name, bits):
    kw, T = STREAM[name]
    base = ms.CONFIGS["decode80b" if bits == 4 else "decode80b_int8"]
    cfg = ms.scaled(base, **{"n_slots": 512, **kw})
    L = DeviceLayer(cfg)
    _, x = L.x(7, T)
    ys, i_s, ws_, ss = moe.moe_layer_forward(L.layer, x, path=moe.MOE_PATH_PREFILL_STREAM)
    yt, it, wt, st = moe.moe_layer_forward(L.layer, x, path=moe.MOE_PATH_PREFILL_TILED)
    torch.cuda.synchronize()
    assert L.pool.check_error() == moe.MOE_OK
    assert torch.equal(i_s, it) and torch.equal(ws_, wt) and torch.equal(ss, st)
    rows = (ys != yt).any(1).nonzero().flatten().tolist()
    if rows:
        idx_np = _np(i_s)
        xb, _ = L.x(7, T)
        ref = L.oracle(xb, idx=idx_np)
        es = np.abs(_np(ys) - ref["y"]).max(1) / np.abs(ref["y"]).max(1)
        et = np.abs(_np(yt) - ref["y"]).max(1) / np.abs(ref["y"]).max(1)
        cnt = np.bincount(idx_np.ravel(), minlength=cfg.E)
        print(f"{name} {bits}-bit: {len(rows)} rows differ, e.g. {rows[:8]}; stream err {es[rows].max():.2e}, "
              f"tiled err {et[rows].max():.2e}; their buckets {[cnt[idx_np[r]].tolist() for r in rows[:3]]}")
    assert not rows
    rel, namb, _, idx = _check_layer_step(L, 7, path=moe.MOE_PATH_PREFILL_STREAM, T=T)
    biggest = np.bincount(idx.ravel(), minlength=cfg.E).max()
    print(f"stream {name} {bits}-bit T={T}: rel err {rel:.2e}, near-ties {namb}, largest bucket {biggest}")


def test_stream_path_is_the_choice_for_few_tokens_per_expert(l80):
    """MOE_PATH_PREFILL (and AUTO above 8 tokens) take the streaming GEMMs
    while T k <= 4 E: the same bits as the forced streaming path; beyond, the
    tiled ones."""
    for T, forced in ((64, moe.MOE_PATH_PREFILL_STREAM), (204, moe.MOE_PATH_PREFILL_STREAM),
                      (206, moe.MOE_PATH_PREFILL_TILED)):
        _, x = l80.x(50 + T, T)
        ya, _, _, _ = moe.moe_layer_forward(l80.layer, x, path=moe.MOE_PATH_AUTO)
        yf, _, _, _ = moe.moe_layer_forward(l80.layer, x, path=forced)
        torch.cuda.synchronize()
        assert torch.equal(ya, yf), T
