"""moe_layer_forward_noalloc (the layer with the library's per-GPU scratch as
its workspace, for callers that cannot allocate) against moe_layer_forward
on the same inputs: the same kernels, so the same bits.  Two calls in a row,
the second smaller than the first (the scratch keeps the first call's
contents), then a call too large for the scratch, which must be refused
without touching the outputs."""
import numpy as np
import pytest

import moe_synth as ms
from gpu_support import DeviceLayer

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
moe = pytest.importorskip("sparse_moe_decode_router_amd")


def _outs(T, d, k):
    return (torch.full((T, d), float("nan"), dtype=torch.float32, device="cuda"),
            torch.full((T, k), -7, dtype=torch.int32, device="cuda"),
            torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda"),
            torch.full((T,), float("nan"), dtype=torch.float32, device="cuda"))


def _same(L, step, T, path):
    xb, x = L.x(step, T)
    got = _outs(T, L.cfg.d, L.cfg.k)
    moe.moe_layer_forward_noalloc(L.layer, x, path=path, out=got)
    ref = moe.moe_layer_forward(L.layer, x, path=path)
    torch.cuda.synchronize()
    for a, b, what in zip(got, ref, ("y", "idx", "w", "s")):
        assert torch.equal(a, b), f"T={T} path={path}: {what} differs"
    assert L.pool.check_error() == moe.MOE_OK


def test_noalloc_matches_layer_forward_two_calls():
    cfg = ms.scaled(ms.CONFIGS["batch80b"], E=64, k=8, n_slots=64)
    L = DeviceLayer(cfg)
    assert L.layer.workspace_bytes(64, moe.MOE_PATH_AUTO) <= moe.NOALLOC_SCRATCH_BYTES
    _same(L, 0, 64, moe.MOE_PATH_AUTO)        # grouped GEMMs on the matrix cores
    _same(L, 1, 2, moe.MOE_PATH_AUTO)         # then a smaller decode call on the same scratch
    _same(L, 2, 1, moe.MOE_PATH_DECODE)


def test_noalloc_80b_decode_and_refusal():
    cfg = ms.scaled(ms.CONFIGS["decode80b"], n_slots=512)
    L = DeviceLayer(cfg)
    _same(L, 3, 8, moe.MOE_PATH_DECODE)
    _same(L, 4, 1, moe.MOE_PATH_AUTO)
    T = 4096                                   # a prefill's workspace is far beyond the scratch
    assert L.layer.workspace_bytes(T, moe.MOE_PATH_AUTO) > moe.NOALLOC_SCRATCH_BYTES
    _, x = L.x(0, T)
    got = _outs(T, cfg.d, cfg.k)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer_forward_noalloc(L.layer, x, out=got)
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.isnan(got[0]).all() and (got[1] == -7).all()
