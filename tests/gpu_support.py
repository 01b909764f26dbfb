"""Helpers for the GPU parity tests: device layers built from the seeded
generators, and the certified comparison of device routing with the oracle."""
from __future__ import annotations

import numpy as np

import moe_synth as ms
from oracle import layer as olayer


class DeviceLayer:
    """One MoE layer on the device: router weights, optional logit bias, a slot
    pool holding the routed experts (slot of expert e = table[e]) and the
    resident shared expert."""

    def __init__(self, cfg: ms.LayerConfig, table=None, n_slots=None, resident=None, usage=True):
        import torch
        import sparse_moe_decode_router_amd as moe
        self.cfg = cfg
        self.moe = moe
        self.Wr_np = ms.router_weight(cfg)
        self.bias_np = ms.logit_bias(cfg)
        self.Wr = torch.from_numpy(self.Wr_np).cuda()
        self.bias = None if self.bias_np is None else torch.from_numpy(self.bias_np).cuda()
        self.shared_raw = ms.shared_raw(cfg)
        self.shared_blob = torch.from_numpy(
            moe.moe_pack_expert(self.shared_raw, cfg.d, cfg.I_shared, cfg.bits)).cuda()
        n_slots = cfg.E if n_slots is None else n_slots
        self.pool = moe.Pool(cfg.E, n_slots, cfg.d, cfg.I, cfg.bits)
        if table is None:
            table = ms.slot_permutation(cfg) if n_slots == cfg.E else None
        self._raw = {}
        if table is not None:
            table = np.asarray(table, np.int32)
            experts = range(cfg.E) if resident is None else resident
            for e in experts:
                if table[e] >= 0:
                    self.pool.load(int(e), int(table[e]), torch.from_numpy(self.blob(e)).cuda())
            t = np.full(cfg.E, -1, np.int32)
            for e in experts:
                t[e] = table[e]
            self.pool.set_slot_table(t)
        torch.cuda.synchronize()
        self.layer = moe.Layer(self.Wr, self.bias, self.pool, self.shared_blob, cfg.I_shared, cfg.k,
                               usage=usage)

    def raw(self, e: int):
        if e not in self._raw:
            self._raw[e] = ms.expert_raw(self.cfg, e)
        return self._raw[e]

    def blob(self, e: int) -> np.ndarray:
        return self.moe.moe_pack_expert(self.raw(e), self.cfg.d, self.cfg.I, self.cfg.bits)

    def x(self, step: int, T=None):
        import torch
        xb = ms.x_bits(self.cfg, step, T)
        return xb, torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)

    def oracle(self, xb, idx=None):
        return olayer.moe_layer(xb, self.Wr_np, self.bias_np, self.cfg.k, self.raw, self.shared_raw, idx=idx)


def certify_routing(xb, Wr, bias, k, idx_dev, depth):
    """Compare device top-k with the fp64 oracle under the certified bound.

    For each token, r = bound on |device fp32 logit - exact logit|.  Where the
    exact logits around every rank boundary are separated by more than 2r the
    device result is unique and must match bit for bit; otherwise every device
    choice must be consistent with the exact logits within 2r.  Returns
    (number of tokens that were not certified unique, per-token flag)."""
    x = olayer.bf16_to_f64(xb)
    l, _ = olayer.router_logits(x, Wr, bias)
    ref = olayer.select_topk(l, k)
    r = olayer.logit_error_bound(xb, Wr, bias, depth)
    T, E = l.shape
    amb = np.zeros(T, bool)
    for t in range(T):
        order = np.lexsort((np.arange(E), -l[t]))
        top = l[t, order[:min(k + 1, E)]]
        gaps = -np.diff(top)
        if np.all(gaps > 2 * r[t]):
            assert idx_dev[t].tolist() == ref[t].tolist(), (t, idx_dev[t], ref[t])
        else:
            amb[t] = True
            dev = idx_dev[t]
            assert len(set(dev.tolist())) == k
            kth = top[k - 1]
            assert np.all(l[t, dev] >= kth - 2 * r[t])
            assert np.all(np.diff(l[t, dev]) <= 2 * r[t])
    return int(amb.sum()), amb


def assert_close_y(y_dev, y_ref, rel=2e-3):
    err = np.max(np.abs(y_dev.astype(np.float64) - y_ref))
    scale = np.max(np.abs(y_ref))
    assert err <= rel * scale, f"max|err| {err:.3e} > {rel} * {scale:.3e}"
    return err / scale


def check_device_logits(xb, Wr, bias, k, idx_dev, w_dev, l_dev, depth):
    """The device's own logits (exported by moe_router_topk_logits, before the
    bias) against the exact ones and its selection against its own logits:

    * every logit, the shared-gate row included, within the elementwise fp32
      rounding bound for the router's documented summation depth (this pins
      the accumulation model the certified near-tie rule relies on, the matrix
      cores' included);
    * the selection is the exact top k of the device's own fp32 keys
      fp32(logit + bias), ties to the lower index, in rank order: bit for bit
      on every token, near-ties included;
    * the weights are the softmax over those keys.
    Returns the largest |error| / bound."""
    E = Wr.shape[0] - 1
    exact = olayer.bf16_to_f64(xb) @ np.asarray(Wr, np.float64).T
    r = olayer.logit_error_bounds(xb, Wr, depth)
    err = np.abs(l_dev.astype(np.float64) - exact)
    bad = np.argwhere(err > r)
    assert bad.size == 0, f"logit outside the rounding bound at {bad[:4].tolist()}"
    keys = l_dev[:, :E].astype(np.float32)
    if bias is not None:
        keys = (keys + np.asarray(bias, np.float32)[None, :]).astype(np.float32)
    sel = olayer.select_topk(keys.astype(np.float64), k)
    mism = np.nonzero((sel != idx_dev).any(1))[0]
    assert mism.size == 0, f"selection differs from the top k of the device logits at tokens {mism[:4]}"
    w_ref = olayer.topk_weights(keys.astype(np.float64), idx_dev)
    assert np.allclose(w_dev, w_ref, rtol=0, atol=2e-6)
    return float(np.max(err / np.maximum(r, 1e-300)))


def predicted_near_ties(xb, Wr, bias, k, depth):
    """Expected number of tokens the certified rule cannot separate, under the
    exponential-spacing model of the top order statistics: at rank boundary
    i the chance that the exact gap falls below 2 r_t is 1 - exp(-2 r_t / g_i),
    g_i the mean gap at that boundary over these tokens."""
    l, _ = olayer.router_logits(olayer.bf16_to_f64(xb), Wr, bias)
    r = olayer.logit_error_bound(xb, Wr, bias, depth)
    top = -np.sort(-l, axis=1)[:, :min(k + 1, l.shape[1])]
    gaps = -np.diff(top, axis=1)
    if gaps.shape[1] == 0:
        return 0.0
    g = np.maximum(gaps.mean(axis=0), 1e-30)
    p = 1.0 - np.exp(-2.0 * r[:, None] / g[None, :])
    return float((1.0 - np.prod(1.0 - p, axis=1)).sum())
