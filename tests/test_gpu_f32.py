"""Parity of the unquantised fp32 expert path with the fp64 CPU oracle,
through the C ABI: the decode GEMVs (routing by the top-k kernel) and the
bucketed GEMVs (AUTO above 8 tokens), the shape envelope, placement
invariance, and the matrix-core path refusing f32 experts."""
import numpy as np
import pytest

import moe_synth as ms
from gpu_support import DeviceLayer, certify_routing, assert_close_y

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
moe = pytest.importorskip("sparse_moe_decode_router_amd")

TINY32 = ms.CONFIGS["tiny_f32"]


def _np(t):
    return t.detach().cpu().numpy()


@pytest.fixture(scope="module")
def l80():
    return DeviceLayer(ms.scaled(ms.CONFIGS["decode80b_f32"], E=128, n_slots=128))


def _check(L, step, path=moe.MOE_PATH_AUTO, T=None):
    xb, x = L.x(step, T)
    y, idx, w, s = moe.moe_layer_forward(L.layer, x, path=path)
    torch.cuda.synchronize()
    assert L.pool.check_error() == moe.MOE_OK
    idx_np = _np(idx)
    depth = moe.moe_router_sum_depth(xb.shape[0], L.cfg.d, L.cfg.E)
    namb, _ = certify_routing(xb, L.Wr_np, L.bias_np, L.cfg.k, idx_np, depth)
    ref = L.oracle(xb, idx=idx_np)
    assert np.allclose(_np(w), ref["w"], rtol=0, atol=2e-5)
    return max(assert_close_y(_np(y)[t:t + 1], ref["y"][t:t + 1]) for t in range(xb.shape[0])), namb


def test_tiny_f32_layer_parity():
    L = DeviceLayer(TINY32)
    worst = max(_check(L, step)[0] for step in range(TINY32.steps))
    print(f"tiny f32 worst rel err {worst:.2e}")
    assert worst < 1e-5                     # fp32 products and sums throughout


def test_decode80b_f32_parity(l80):
    worst = max(_check(l80, s, path=moe.MOE_PATH_DECODE)[0] for s in range(3))
    for T in (2, 4, 8):
        worst = max(worst, _check(l80, 10 + T, path=moe.MOE_PATH_DECODE, T=T)[0])
    print(f"80B-shape f32 decode worst rel err {worst:.2e}")


def test_batched_f32_parity(l80):
    rel, namb = _check(l80, 0, T=64)          # AUTO: the bucketed GEMVs for f32
    print(f"f32 batched T=64 rel err {rel:.2e}, near-ties {namb}")


def test_f32_full_80b_decode_shape():
    L = DeviceLayer(ms.CONFIGS["decode80b_f32"])
    rel, _ = _check(L, 0, path=moe.MOE_PATH_DECODE)
    print(f"80B f32 decode rel err {rel:.2e}")


ENVELOPE = {
    "wide_I": dict(d=512, E=32, k=4, I=1024, I_shared=1024, n_slots=32),
    "max_E": dict(d=512, E=1024, k=16, I=128, I_shared=128, n_slots=1024),
    "max_d": dict(d=8192, E=16, k=2, I=128, I_shared=128, n_slots=16),
    "k_eq_E": dict(d=256, E=16, k=16, I=64, I_shared=64, n_slots=16),
    "small_d": dict(d=192, E=16, k=3, I=64, I_shared=64, n_slots=16),
}


@pytest.mark.parametrize("name", sorted(ENVELOPE))
def test_f32_envelope(name):
    L = DeviceLayer(ms.scaled(ms.CONFIGS["decode80b_f32"], alpha=0.0, **ENVELOPE[name]))
    _check(L, 0, path=moe.MOE_PATH_DECODE, T=1)
    _check(L, 1, path=moe.MOE_PATH_DECODE, T=4)
    _check(L, 2, path=moe.MOE_PATH_BATCHED, T=24)


def test_f32_placement_and_refill_bit_identical():
    cfg = ms.scaled(ms.CONFIGS["decode80b_f32"], E=32, k=4, steps=8)
    A = DeviceLayer(cfg, table=np.arange(cfg.E))
    B = DeviceLayer(cfg, table=np.random.default_rng(9).permutation(cfg.E))
    C_ = DeviceLayer(cfg, table=None, n_slots=8)
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
    assert C_.pool.stats()["misses"] > 0 and C_.pool.check_error() == moe.MOE_OK


def test_f32_prefill_path_refused():
    L = DeviceLayer(TINY32)
    _, x = L.x(0, 16)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer_forward(L.layer, x, path=moe.MOE_PATH_PREFILL)
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
