"""Chains of MoE layers on the device (moe_chain_forward) against the fp64
oracle, layer by layer on the device's own residual stream: the normalised
input u_l within one bf16 step of the oracle's, the routing certified, and
x_{l+1} = bf16(x_l + y_l) with y_l from the oracle on the device's u_l and
routing, within the layer tolerance plus one bf16 rounding."""
import numpy as np
import pytest

import moe_synth as ms
from oracle import layer as olayer
from gpu_support import DeviceLayer, certify_routing

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
moe = pytest.importorskip("sparse_moe_decode_router_amd")


def _np(t):
    return t.detach().cpu().numpy()


def _bits(t):
    return _np(t.view(torch.int16)).view(np.uint16)


def _layers(cfg, L):
    return [DeviceLayer(ms.scaled(cfg, seed=cfg.seed + 97 * l)) for l in range(L)]


def _check_chain(DL, T, path, step=0, eps=1e-6):
    chain = moe.Chain([D.layer for D in DL], eps)
    xb, x = DL[0].x(step, T)
    x_out, tx, tu, ti = moe.moe_chain_forward(chain, x, path=path, trace=True)
    torch.cuda.synchronize()
    tx, tu, ti = _bits(tx), _bits(tu), _np(ti)
    assert np.array_equal(tx[0], xb) and np.array_equal(_bits(x_out), tx[-1])
    worst = 0.0
    for l, D in enumerate(DL):
        assert D.pool.check_error() == moe.MOE_OK
        # normalised input: the oracle's bf16 value or its neighbour (fp32 sum of squares)
        u_ref = olayer.rms_norm_bf16(tx[l], eps)
        du = np.abs(olayer.bf16_to_f64(tu[l]) - olayer.bf16_to_f64(u_ref))
        assert np.all(du <= np.abs(olayer.bf16_to_f64(u_ref)) * 2.0 ** -7 + 1e-30), l
        depth = moe.moe_router_sum_depth(T, D.cfg.d, D.cfg.E)
        certify_routing(tu[l], D.Wr_np, D.bias_np, D.cfg.k, ti[l], depth)
        y_ref = olayer.moe_layer(tu[l], D.Wr_np, D.bias_np, D.cfg.k, D.raw, D.shared_raw, idx=ti[l])["y"]
        x_l, x_n = olayer.bf16_to_f64(tx[l]), olayer.bf16_to_f64(tx[l + 1])
        err = np.abs(x_n - (x_l + y_ref))
        bound = 2e-3 * np.abs(y_ref).max(axis=1, keepdims=True) + np.abs(x_n) * 2.0 ** -8
        assert np.all(err <= bound), (l, float((err - bound).max()))
        worst = max(worst, float((np.abs(x_n - x_l - y_ref) / np.abs(y_ref).max()).max()))
    return worst


@pytest.mark.parametrize("T,path", [(1, moe.MOE_PATH_DECODE), (4, moe.MOE_PATH_DECODE),
                                    (24, moe.MOE_PATH_AUTO), (24, moe.MOE_PATH_BATCHED)])
def test_chain_small(T, path):
    cfg = ms.scaled(ms.CONFIGS["decode80b"], d=256, E=16, k=2, I=64, I_shared=64, n_slots=16, alpha=0.0)
    worst = _check_chain(_layers(cfg, 4), T, path)
    print(f"chain T={T} path={path}: worst rel {worst:.2e}")


@pytest.mark.parametrize("bits", [8, 32])
def test_chain_other_code_widths(bits):
    cfg = ms.scaled(ms.CONFIGS["decode80b"], d=256, E=16, k=2, I=64, I_shared=64, n_slots=16, alpha=0.0,
                    bits=bits)
    _check_chain(_layers(cfg, 3), 2, moe.MOE_PATH_DECODE)


def test_chain_80b_shape():
    cfg = ms.scaled(ms.CONFIGS["decode80b"], E=128, n_slots=128)
    worst = _check_chain(_layers(cfg, 3), 1, moe.MOE_PATH_DECODE)
    print(f"80B-shape chain of 3: worst rel {worst:.2e}")


def test_chain_graph_replay_matches_eager():
    cfg = ms.scaled(ms.CONFIGS["decode80b"], d=256, E=16, k=2, I=64, I_shared=64, n_slots=16, alpha=0.0)
    DL = _layers(cfg, 3)
    chain = moe.Chain([D.layer for D in DL])
    xs = [DL[0].x(s, 1)[1] for s in range(4)]
    ws = torch.zeros(chain.workspace_bytes(1, moe.MOE_PATH_DECODE), dtype=torch.uint8, device="cuda")
    outs = torch.empty((4, 1, cfg.d), dtype=torch.bfloat16, device="cuda")
    eager = [moe.moe_chain_forward(chain, xs[s], path=moe.MOE_PATH_DECODE).clone() for s in range(4)]
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for s in range(4):
                moe.moe_chain_forward(chain, xs[s], path=moe.MOE_PATH_DECODE, workspace=ws, out=outs[s])
    for _ in range(3):
        outs.zero_()
        g.replay()
        torch.cuda.synchronize()
        for s in range(4):
            assert torch.equal(outs[s], eager[s])


@pytest.mark.parametrize("T,bits,shape", [(1, 4, "small"), (3, 4, "small"), (8, 4, "small"), (2, 8, "small"),
                                          (1, 4, "80b"), (4, 8, "80b")])
def test_chain_traces_do_not_change_results(T, bits, shape):
    """Asking for the traces (or not) gives the same bits.  Without trace_u
    the decode layers hand the residual stream on inside their own kernels;
    with it a separate residual/norm launch runs per layer, whose results the
    oracle checks above: the two must agree bit for bit."""
    if shape == "small":
        cfg = ms.scaled(ms.CONFIGS["decode80b"], d=512, E=32, k=4, I=128, I_shared=128, n_slots=32, alpha=0.0,
                        bits=bits)
    else:
        cfg = ms.scaled(ms.CONFIGS["decode80b"], E=64, n_slots=64, bits=bits)
    DL = _layers(cfg, 4 if shape == "small" else 3)
    chain = moe.Chain([D.layer for D in DL])
    _, x = DL[0].x(5, T)
    xa, txa, _, tia = moe.moe_chain_forward(chain, x, path=moe.MOE_PATH_DECODE, trace=True)
    xb, txb, tub, tib = moe.moe_chain_forward(chain, x, path=moe.MOE_PATH_DECODE, trace=True, trace_u=False)
    xc = moe.moe_chain_forward(chain, x, path=moe.MOE_PATH_DECODE)
    torch.cuda.synchronize()
    assert tub is None
    assert torch.equal(txa, txb) and torch.equal(tia, tib)
    assert torch.equal(xa, xb) and torch.equal(xa, xc)
