"""Streamed decode steps (moe_layer_forward_streamed): a pool holding only
some experts, refilled by LFU + recency from pinned host memory on a copy
stream while the resident experts compute.  Every output must be
bit-identical to the same step on an all-resident pool (the decode path of
moe_layer_forward), whatever was resident, copied or deferred."""
import numpy as np
import pytest

import moe_synth as ms
from gpu_support import DeviceLayer

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
moe = pytest.importorskip("sparse_moe_decode_router_amd")


def _host_blobs(L):
    return torch.from_numpy(np.stack([L.blob(e) for e in range(L.cfg.E)])).pin_memory()


def _run(cfg, n_slots, T, steps, copy_stream=True):
    twin = DeviceLayer(cfg)                                  # all resident, permuted slots
    part = DeviceLayer(cfg, table=None, n_slots=n_slots)     # starts empty
    host = _host_blobs(twin)
    cs = torch.cuda.Stream() if copy_stream else None
    ws = torch.zeros(part.layer.workspace_bytes(T, moe.MOE_PATH_DECODE), dtype=torch.uint8, device="cuda")
    loads = []
    for step in range(steps):
        _, x = twin.x(step, T)
        y, idx, w, s, nl = moe.moe_layer_forward_streamed(part.layer, x, host, copy_stream=cs, workspace=ws)
        yt, it, wt, st = moe.moe_layer_forward(twin.layer, x, path=moe.MOE_PATH_DECODE)
        torch.cuda.synchronize()
        assert torch.equal(idx, it) and torch.equal(w, wt) and torch.equal(s, st), step
        assert torch.equal(y, yt), (step, float((y - yt).abs().max()))
        loads.append(nl)
    assert part.pool.check_error() == moe.MOE_OK
    stats = part.pool.stats()
    assert stats["misses"] > 0 and sum(loads) == stats["loads"]
    return loads, stats


def test_streamed_small_pool_bit_identical():
    cfg = ms.scaled(ms.CONFIGS["decode80b"], d=256, E=64, k=6, I=64, I_shared=64, alpha=0.0)
    loads, st = _run(cfg, 16, 1, 24)
    assert loads[0] == 6 and st["hits"] > 0               # cold start: every selection is a miss


@pytest.mark.parametrize("T", [2, 4])
def test_streamed_several_tokens(T):
    cfg = ms.scaled(ms.CONFIGS["decode80b"], d=512, E=64, k=4, I=128, I_shared=128, alpha=0.15)
    _run(cfg, 32, T, 12)


def test_streamed_same_stream_and_int8():
    cfg = ms.scaled(ms.CONFIGS["decode80b_int8"], d=256, E=32, k=4, I=64, I_shared=64)
    _run(cfg, 12, 1, 12, copy_stream=False)


def test_streamed_80b_shape():
    cfg = ms.CONFIGS["decode80b"]                           # 256 slots over 512 experts
    loads, st = _run(cfg, cfg.n_slots, 1, 6)
    assert loads[0] == cfg.k


def test_streamed_pool_too_small():
    cfg = ms.scaled(ms.CONFIGS["decode80b"], d=256, E=64, k=6, I=64, I_shared=64, alpha=0.0)
    part = DeviceLayer(cfg, table=None, n_slots=8)
    host = _host_blobs(part)
    _, x = part.x(0, 4)                                     # 4 tokens x 6 picks: more than 8 experts
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer_forward_streamed(part.layer, x, host)
    assert ei.value.status == moe.MOE_ERR_POOL_TOO_SMALL
    torch.cuda.synchronize()


# ------------------------------------------------------------------ offload
def _run_offload(cfg, n_slots, T, steps, host_every=0):
    """Offload steps (plan and copy on the GPU) against the all-resident twin,
    bit for bit; the pool's statistics against the host LFU replayed over the
    same selections.  host_every: every host_every-th step is a host-planned
    streamed step on the same pool (the policy state crosses between the
    device and host copies)."""
    twin = DeviceLayer(cfg)
    part = DeviceLayer(cfg, table=None, n_slots=n_slots)
    host = _host_blobs(twin)
    ws = torch.zeros(part.layer.workspace_bytes(T, moe.MOE_PATH_DECODE), dtype=torch.uint8, device="cuda")
    nl_dev = torch.full((steps,), -1, dtype=torch.int32, device="cuda")
    trace, kinds, host_nl = [], [], {}
    for step in range(steps):
        _, x = twin.x(step, T)
        if host_every and step % host_every == host_every - 1:
            y, idx, w, s, nl = moe.moe_layer_forward_streamed(part.layer, x, host, workspace=ws)
            host_nl[step] = nl
            kinds.append("host")
        else:
            y, idx, w, s = moe.moe_layer_forward_offload(part.layer, x, host, workspace=ws,
                                                         n_loads=nl_dev[step:step + 1])
            kinds.append("dev")
        yt, it, wt, st = moe.moe_layer_forward(twin.layer, x, path=moe.MOE_PATH_DECODE)
        torch.cuda.synchronize()
        assert torch.equal(idx, it) and torch.equal(w, wt) and torch.equal(s, st), step
        assert torch.equal(y, yt), (step, float((y - yt).abs().max()))
        trace.append(idx.flatten().cpu().numpy())
    assert part.pool.check_error() == moe.MOE_OK
    ref = moe.Lfu(cfg.E, n_slots)
    ref_nl = [len(ref.plan(sel)) for sel in trace]
    rs = ref.stats()
    got = part.pool.stats()
    for key in ("steps", "hits", "misses", "evictions"):
        assert got[key] == rs[key], (key, got, rs)
    assert got["loads"] == sum(ref_nl) and got["bytes_loaded"] == sum(ref_nl) * part.pool.stride
    dev_nl = nl_dev.cpu().tolist()
    for step, kind in enumerate(kinds):
        assert (dev_nl[step] if kind == "dev" else host_nl[step]) == ref_nl[step], step
    return ref_nl, got


def test_offload_small_pool_bit_identical():
    cfg = ms.scaled(ms.CONFIGS["decode80b"], d=256, E=64, k=6, I=64, I_shared=64, alpha=0.0)
    loads, st = _run_offload(cfg, 16, 1, 30)
    assert loads[0] == 6 and st["hits"] > 0 and st["evictions"] > 0


def test_offload_several_tokens_int8_and_host_steps_between():
    cfg = ms.scaled(ms.CONFIGS["decode80b_int8"], d=256, E=64, k=4, I=64, I_shared=64, alpha=0.15)
    _run_offload(cfg, 20, 4, 24, host_every=3)


def test_offload_80b_shape():
    cfg = ms.CONFIGS["decode80b"]                           # 256 slots over 512 experts
    loads, st = _run_offload(cfg, cfg.n_slots, 1, 40, host_every=10)
    assert loads[0] == cfg.k


def test_offload_refusals():
    cfg = ms.scaled(ms.CONFIGS["decode80b"], d=256, E=64, k=6, I=64, I_shared=64, alpha=0.0)
    part = DeviceLayer(cfg, table=None, n_slots=8)
    host = _host_blobs(part)
    _, x = part.x(0, 4)                                     # 4 tokens x 6 picks > 8 slots
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer_forward_offload(part.layer, x, host)
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
    with pytest.raises(ValueError):
        moe.moe_layer_forward_offload(part.layer, x[:1], host.clone())   # not pinned
    torch.cuda.synchronize()
    assert part.pool.stats()["steps"] == 0                  # nothing planned
