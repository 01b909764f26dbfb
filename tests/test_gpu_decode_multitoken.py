"""Decode down with several rounds of instances (more than 16 per step):
the pipelined kernel (selection slots staged in LDS, the next round's codes
and h records in flight during the compute, h records in a swizzled LDS
layout) does the single-round kernel's arithmetic, so with the routing
given a call on T tokens reproduces each token's own T = 1 call bit for
bit.  The pipelined kernel runs from two rounds (T = 2 at k = 10); the 80B
expert shape (64 experts, all resident) with 4- and 8-bit codes, and a
wide intermediate (groups past the eighth) on a small one."""
import numpy as np
import pytest

import moe_synth as ms
from gpu_support import DeviceLayer

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
moe = pytest.importorskip("sparse_moe_decode_router_amd")


def _np(t):
    return t.detach().cpu().numpy()


CASES = {
    "80b_int4": (ms.scaled(ms.CONFIGS["decode80b"], E=64, n_slots=64), (2, 4, 8)),
    "80b_int8": (ms.scaled(ms.CONFIGS["decode80b_int8"], E=64, n_slots=64), (2, 4, 8)),
    "wide_I_int4": (ms.scaled(ms.CONFIGS["decode80b"], alpha=0.0, d=512, E=32, k=4, I=1024, I_shared=1024,
                              n_slots=32), (4, 8)),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_tokens_match_single_token_calls(name):
    cfg, Ts = CASES[name]
    L = DeviceLayer(cfg)
    for T in Ts:
        _, x = L.x(40 + T, T)
        idx, w, s = moe.moe_router_topk(x, L.Wr, L.bias, cfg.k)
        y = moe.moe_expert_ffn(L.pool, L.shared_blob, cfg.I_shared, x, idx, w, s)
        torch.cuda.synchronize()
        for t in range(T):
            y1 = moe.moe_expert_ffn(L.pool, L.shared_blob, cfg.I_shared, x[t:t + 1].contiguous(),
                                    idx[t:t + 1].contiguous(), w[t:t + 1].contiguous(), s[t:t + 1].contiguous())
            torch.cuda.synchronize()
            assert np.array_equal(_np(y1)[0], _np(y)[t]), (name, T, t)
        assert L.pool.check_error() == moe.MOE_OK


@pytest.mark.parametrize("bits", [4, 8])
def test_wide_intermediate_fallback_kernel(bits):
    """Intermediate 1536: the pipelined kernel's two record buffers exceed
    the LDS, so the decode down pass takes down_decode_kernel (staged
    records, one buffer).  Routing given from the router; outputs against
    the fp64 oracle on that routing, and a T = 4 call against each token's
    own call bit for bit."""
    from gpu_support import assert_close_y
    cfg = ms.scaled(ms.CONFIGS["tiny_int8" if bits == 8 else "tiny"], d=256, E=16, k=2, I=1536, I_shared=1536,
                    n_slots=16)
    L = DeviceLayer(cfg)
    xb, x = L.x(7, 4)
    idx, w, s = moe.moe_router_topk(x, L.Wr, L.bias, cfg.k)
    y = moe.moe_expert_ffn(L.pool, L.shared_blob, cfg.I_shared, x, idx, w, s)
    torch.cuda.synchronize()
    ref = L.oracle(xb, idx=_np(idx))
    for t in range(4):
        assert_close_y(_np(y)[t:t + 1], ref["y"][t:t + 1])
        y1 = moe.moe_expert_ffn(L.pool, L.shared_blob, cfg.I_shared, x[t:t + 1].contiguous(),
                                idx[t:t + 1].contiguous(), w[t:t + 1].contiguous(), s[t:t + 1].contiguous())
        torch.cuda.synchronize()
        assert np.array_equal(_np(y1)[0], _np(y)[t])
    assert L.pool.check_error() == moe.MOE_OK
