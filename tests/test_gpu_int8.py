"""Parity of the 8-bit expert path (MLX affine int8, group 64) with the fp64
CPU oracle, through the C ABI.

Same bars as the 4-bit tests: routing bit-exact up to certified near-ties,
outputs within max|y - y_ref| <= 2e-3 * max|y_ref|, placement invariance
bit-identical.  Shapes: the tiny layer, the 80B decode / batched / prefill
shapes with 8-bit experts, and the envelope edges (intermediate 1024,
E = 1024 with k = 16, d = 8192, k = E).
"""
import numpy as np
import pytest

import moe_synth as ms
from gpu_support import DeviceLayer, certify_routing, assert_close_y

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
moe = pytest.importorskip("sparse_moe_decode_router_amd")

TINY8 = ms.CONFIGS["tiny_int8"]


def _np(t):
    return t.detach().cpu().numpy()


@pytest.fixture(scope="module")
def l80():
    return DeviceLayer(ms.CONFIGS["decode80b_int8"])


def _check(L, step, path=moe.MOE_PATH_AUTO, T=None, sample=None):
    xb, x = L.x(step, T)
    y, idx, w, s = moe.moe_layer_forward(L.layer, x, path=path)
    torch.cuda.synchronize()
    assert L.pool.check_error() == moe.MOE_OK
    rows = np.arange(xb.shape[0]) if sample is None else sample
    idx_np = _np(idx)
    depth = moe.moe_router_sum_depth(xb.shape[0], L.cfg.d, L.cfg.E)
    namb, _ = certify_routing(xb[rows], L.Wr_np, L.bias_np, L.cfg.k, idx_np[rows], depth)
    ref = L.oracle(xb[rows], idx=idx_np[rows])
    assert np.allclose(_np(w)[rows], ref["w"], rtol=0, atol=2e-5)
    if path == moe.MOE_PATH_PREFILL:
        return assert_close_y(_np(y)[rows], ref["y"]), namb
    return max(assert_close_y(_np(y)[t:t + 1], ref["y"][t:t + 1]) for t in range(len(rows))), namb


def test_tiny_int8_layer_parity():
    L = DeviceLayer(TINY8)
    worst = max(_check(L, step)[0] for step in range(TINY8.steps))
    print(f"tiny int8 worst rel err {worst:.2e}")


def test_decode80b_int8_parity(l80):
    worst = max(_check(l80, s, path=moe.MOE_PATH_DECODE)[0] for s in range(4))
    for T in (2, 4, 8):
        _check(l80, 10 + T, path=moe.MOE_PATH_DECODE, T=T)
    print(f"80B int8 decode worst rel err {worst:.2e}")


def test_batched80b_int8_parity(l80):
    rel, namb = _check(l80, 0, path=moe.MOE_PATH_BATCHED, T=64)
    print(f"80B int8 batched T=64 rel err {rel:.2e}, near-ties {namb}")


def test_prefill_int8_midsize_full_oracle():
    cfg = ms.scaled(ms.CONFIGS["prefill80b_int8"], T=512, E=32, k=8, d=512, I=128, I_shared=128,
                    n_slots=32)
    rel, namb = _check(DeviceLayer(cfg), 0, path=moe.MOE_PATH_PREFILL, T=cfg.T)
    print(f"int8 prefill midsize rel err {rel:.2e}, near-ties {namb}")


def test_prefill_int8_matches_batched_path():
    cfg = ms.scaled(ms.CONFIGS["prefill80b_int8"], T=256, E=64, k=8, d=1024, I=256, I_shared=256,
                    n_slots=64)
    L = DeviceLayer(cfg)
    _, x = L.x(3, cfg.T)
    yp, ip, _, _ = moe.moe_layer_forward(L.layer, x, path=moe.MOE_PATH_PREFILL)
    yb, ib, _, _ = moe.moe_layer_forward(L.layer, x, path=moe.MOE_PATH_BATCHED)
    torch.cuda.synchronize()
    assert np.array_equal(_np(ip), _np(ib))
    assert_close_y(_np(yp), _np(yb).astype(np.float64))


ENVELOPE = {
    "wide_I": dict(d=512, E=32, k=4, I=1024, I_shared=1024, n_slots=32),
    "max_E": dict(d=512, E=1024, k=16, I=128, I_shared=128, n_slots=1024),
    "max_d": dict(d=8192, E=16, k=2, I=128, I_shared=128, n_slots=16),
    "k_eq_E": dict(d=256, E=16, k=16, I=64, I_shared=64, n_slots=16),
    "small_d": dict(d=192, E=16, k=3, I=64, I_shared=64, n_slots=16),
    "steps_3n": dict(d=768, E=32, k=4, I=384, I_shared=384, n_slots=32),
}


@pytest.mark.parametrize("name", sorted(ENVELOPE))
def test_int8_envelope_decode_and_batched(name):
    L = DeviceLayer(ms.scaled(ms.CONFIGS["decode80b_int8"], alpha=0.0, **ENVELOPE[name]))
    _check(L, 0, path=moe.MOE_PATH_DECODE, T=1)
    _check(L, 1, path=moe.MOE_PATH_DECODE, T=4)
    _check(L, 2, path=moe.MOE_PATH_BATCHED, T=24)


@pytest.mark.parametrize("name", sorted(set(ENVELOPE) - {"small_d"}))
def test_int8_envelope_prefill(name):
    cfg = ms.scaled(ms.CONFIGS["prefill80b_int8"], T=160, **ENVELOPE[name])
    rel, namb = _check(DeviceLayer(cfg), 0, path=moe.MOE_PATH_PREFILL, T=cfg.T)
    print(f"int8 prefill {name}: rel err {rel:.2e}, near-ties {namb}")


def test_int8_placement_invariance_bit_identical():
    """Permuted slots and an LFU-refilled 16-slot pool give identical bits."""
    cfg = ms.scaled(ms.CONFIGS["decode80b_int8"], E=64, k=6, steps=10)
    A = DeviceLayer(cfg, table=np.arange(cfg.E))
    B = DeviceLayer(cfg, table=np.random.default_rng(5).permutation(cfg.E))
    C_ = DeviceLayer(cfg, table=None, n_slots=16)
    host = torch.from_numpy(np.stack([A.blob(e) for e in range(cfg.E)])).pin_memory()
    for step in range(cfg.steps):
        _, x = A.x(step)
        ya, ia, _, _ = moe.moe_layer_forward(A.layer, x)
        yb, _, _, _ = moe.moe_layer_forward(B.layer, x)
        idx, w, s = moe.moe_router_topk(x, C_.Wr, C_.bias, cfg.k)
        torch.cuda.synchronize()
        C_.pool.refill(_np(idx).ravel(), host, A.pool.stride)
        yc = moe.moe_expert_ffn(C_.pool, C_.shared_blob, cfg.I_shared, x, idx, w, s)
        torch.cuda.synchronize()
        assert np.array_equal(_np(ya), _np(yb)) and np.array_equal(_np(ya), _np(yc))
    assert C_.pool.stats()["misses"] > 0
    assert C_.pool.check_error() == moe.MOE_OK


def test_code_width_checks():
    """The int4-only FFN entry point refuses an 8-bit pool; routed and shared
    experts of different widths are refused (MOE_ERR_UNSUPPORTED) before any
    kernel runs."""
    L = DeviceLayer(TINY8)
    xb, x = L.x(0)
    idx, w, s = moe.moe_router_topk(x, L.Wr, L.bias, TINY8.k)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_expert_ffn_int4(L.pool, L.shared_blob, TINY8.I_shared, x, idx, w, s)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    shared4 = torch.from_numpy(moe.moe_pack_expert(ms.shared_raw(ms.CONFIGS["tiny"]), TINY8.d,
                                                   TINY8.I_shared, 4)).cuda()
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_expert_ffn(L.pool, shared4, TINY8.I_shared, x, idx, w, s, shared_bits=4)
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
    y = moe.moe_expert_ffn(L.pool, L.shared_blob, TINY8.I_shared, x, idx, w, s)
    ref = L.oracle(xb, idx=_np(idx))
    assert_close_y(_np(y), ref["y"])
