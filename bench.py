#!/usr/bin/env python3
"""Throughput of the routed-expert MoE layer on one MI355X.

Default workload (the headline): the 80B-shaped batch-1 decode layer (T=1,
d=2048, E=512, top-10, expert and shared intermediate 512, int4 group-64
blobs, Zipf-skewed router), all 512 experts resident in the HBM slot pool
behind a seeded slot permutation.  One step = router -> top-k -> expert
SwiGLU FFNs -> weighted combine with the gated shared expert, for one token.
The layer is replicated R times (pools, router weights, shared experts) and
step s uses replica s mod R, so re-reads do not come from the 256 MB
last-level cache.  Steps are captured in a HIP graph and replayed.

Prints one JSON line: tokens/s of the whole layer (value), the dominant
kernels' achieved HBM bandwidth on algorithmic expert bytes (roofline), and
the CPU oracle timed on a bounded sample of the same steps (cpu_baseline).

--workload selects another configuration (decode35b, refill80b: 256-slot
pool refilled by LFU + recency from pinned host memory, stream80b: the same
with the misses copied on a second stream while the resident experts
compute, batch80b: T=64,
prefill80b / prefill80b_zipf: T=4096 on the matrix cores; decode80b_int8,
batch80b_int8, prefill80b_int8: the same layers with 8-bit experts;
decode80b_f32, batch80b_f32: with unquantised fp32 experts; chain80b: 48
such decode layers per token, as pre-norm residual blocks);
--workload all prints one line per workload, the headline first;
--workload refill_sweep prints the refill run, serial and streamed, for pool
sizes 64..512 (hit rate vs tokens/s).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
METRIC = "routed-MoE layer tokens/s + achieved HBM GB/s on int4 experts (80B shape)"
METRIC8 = "routed-MoE layer tokens/s + achieved HBM GB/s on int8 experts (80B shape)"
DATA = ("synthetic (seeded int4 codes U{0..15}, fp16 scales U[0.002,0.02], bias -8*scale, "
        "x ~ N(0,1) bf16, router N(0,0.02) fp32, Zipf(1.1) logit offset alpha=0.15 where skewed)")
DATA8 = ("synthetic (seeded int8 codes U{0..255}, fp16 scales U[0.002,0.02]/16, bias -128*scale, "
         "x ~ N(0,1) bf16, router N(0,0.02) fp32, Zipf(1.1) logit offset alpha=0.15 where skewed)")
METRIC32 = "routed-MoE layer tokens/s + achieved HBM GB/s on f32 experts (80B shape)"
DATA32 = ("synthetic (seeded fp32 expert weights N(0,0.05), x ~ N(0,1) bf16, router N(0,0.02) fp32, "
          "Zipf(1.1) logit offset alpha=0.15)")


def labels(cfg):
    """(metric, data, weight dtype) of a workload by its code width."""
    if cfg.bits == 8:
        return METRIC8, DATA8, "int8"
    if cfg.bits == 32:
        return METRIC32, DATA32, "f32"
    return METRIC, DATA, "int4"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Ctx:
    def __init__(self):
        import torch
        import moe_synth as ms
        import sparse_moe_decode_router_amd as moe
        from oracle import layer as olayer
        self.torch, self.ms, self.moe, self.olayer = torch, ms, moe, olayer


def packed_experts(c, cfg, pinned=False):
    """All E blobs packed by the library's packer: [E, stride] uint8."""
    torch, ms, moe = c.torch, c.ms, c.moe
    stride = moe.moe_blob_stride(cfg.d, cfg.I, cfg.bits)
    t0 = time.time()
    if pinned:
        out = torch.empty((cfg.E, stride), dtype=torch.uint8, pin_memory=True)
    else:
        out = torch.empty((cfg.E, stride), dtype=torch.uint8, device="cuda")
    for e in range(cfg.E):
        out[e].copy_(torch.from_numpy(moe.moe_pack_expert(ms.expert_raw(cfg, e), cfg.d, cfg.I, cfg.bits)))
        if e % 128 == 127:
            log(f"packed {e + 1}/{cfg.E} experts ({time.time() - t0:.1f}s)")
    return out


def build_layers(c, cfg, R, staging=None):
    torch, ms, moe = c.torch, c.ms, c.moe
    d, I, E = cfg.d, cfg.I, cfg.E
    perm = ms.slot_permutation(cfg)
    if staging is None:
        staging = packed_experts(c, cfg)
    Wr = torch.from_numpy(ms.router_weight(cfg)).cuda()
    b = ms.logit_bias(cfg)
    bias = None if b is None else torch.from_numpy(b).cuda()
    shared = torch.from_numpy(moe.moe_pack_expert(ms.shared_raw(cfg), d, cfg.I_shared, cfg.bits)).cuda()
    layers = []
    for r in range(R):
        pool = moe.Pool(E, E, d, I, cfg.bits)
        for e in range(E):
            pool.load(e, int(perm[e]), staging[e])
        pool.set_slot_table(perm)
        layers.append(moe.Layer(Wr.clone(), None if bias is None else bias.clone(), pool,
                                shared.clone(), cfg.I_shared, cfg.k))
        if r % 8 == 7:
            log(f"replica {r + 1}/{R} ready")
    torch.cuda.synchronize()
    return layers


def x_steps(c, cfg, n, T=None):
    torch, ms = c.torch, c.ms
    xs = np.stack([ms.x_bits(cfg, s % cfg.steps, T) for s in range(n)])
    return torch.from_numpy(xs.view(np.int16)).cuda().view(torch.bfloat16)


def graph_time(c, fn, lo, hi, stream):
    """Capture fn(i) for i in [lo, hi) in one graph; replay once; ms per call."""
    torch = c.torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for i in range(lo, hi):
                fn(i)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (hi - lo)


def cpu_info():
    """Host cores this process may run on and the CPU model."""
    cores = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return cores, model


def cpu_baseline(c, cfg, steps=None, tokens=None):
    """The oracle as it stands (numpy fp64, BLAS threads = the cores this
    process may use) on a bounded sample of the workload: the first `steps`
    seeded steps, or the first `tokens` tokens of step 0.  Expert weights are
    generated before the timed region (they are inputs); dequantisation and
    the products are timed."""
    import threadpoolctl
    ms, olayer = c.ms, c.olayer
    cores, model = cpu_info()
    Wr = ms.router_weight(cfg)
    bias = ms.logit_bias(cfg)
    sh = ms.shared_raw(cfg)
    if steps is not None:
        xs = [ms.x_bits(cfg, s) for s in range(steps)]
        what = f"first {steps} of the {cfg.steps} seeded steps ({steps * cfg.T} tokens)"
    else:
        xs = [ms.x_bits(cfg, 0)[:tokens]]
        what = f"first {tokens} of the {cfg.T} tokens of step 0"
    need = set()
    for xb in xs:
        idx, _, _, _ = olayer.route(xb, Wr, bias, cfg.k)
        need.update(int(e) for e in idx.ravel())
    raws = {e: ms.expert_raw(cfg, e) for e in sorted(need)}     # inputs, generated before timing
    ntok = sum(xb.shape[0] for xb in xs)
    with threadpoolctl.threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        for xb in xs:
            olayer.moe_layer(xb, Wr, bias, cfg.k, raws.__getitem__, sh)
        dt = time.perf_counter() - t0
    return {"value": round(ntok / dt, 3), "unit": "tokens/s", "cores": cores, "cpu": model, "kind": "oracle",
            "sample": f"{what}, numpy fp64 (dequantise + matmul per selected expert, {len(need)} experts), "
                      f"{dt:.1f}s; no dequantised-weight cache"}


def chain_cpu_baseline(c, cfgs, expert_cfg):
    """The oracle through a chain of layers (one residual block per layer)
    for one token, as cpu_baseline: router and shared expert of layer l from
    cfgs[l], the routed experts from expert_cfg (the chain workload packs
    one set of expert blobs into every layer's pool)."""
    import threadpoolctl
    ms, olayer = c.ms, c.olayer
    cores, model = cpu_info()
    layers = []
    xb = ms.x_bits(cfgs[0], 0)
    for cl in cfgs:                                   # inputs first: router, shared and selected experts
        Wr, bias, sh = ms.router_weight(cl), ms.logit_bias(cl), ms.shared_raw(cl)
        layers.append(dict(w_router=Wr, bias=bias, k=cl.k, shared=sh, cfg=cl))
    t_gen = 0.0
    with threadpoolctl.threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        for Ld in layers:
            u = olayer.rms_norm_bf16(xb)
            idx, _, _, _ = olayer.route(u, Ld["w_router"], Ld["bias"], Ld["k"])
            tg = time.perf_counter()
            raws = {int(e): ms.expert_raw(expert_cfg, int(e)) for e in np.unique(idx)}
            t_gen += time.perf_counter() - tg
            Ld["expert"] = raws.__getitem__
            xb, _, _ = olayer.chain_layer(xb, Ld)
        dt = time.perf_counter() - t0 - t_gen
    return {"value": round(1.0 / dt, 4), "unit": "tokens/s", "cores": cores, "cpu": model, "kind": "oracle",
            "sample": f"one token through the {len(cfgs)} layers, numpy fp64, {dt:.1f}s "
                      f"(expert generation, {t_gen:.1f}s, not counted)"}


def measure_ceilings(c, read_bytes=(), three=None, mfma=False):
    """What this MI355X sustains: a one-launch streaming read of each size in
    read_bytes (cold: every launch reads a different window of a 1 GiB
    region, beyond the 256 MB last-level cache), three dependent launches
    reading the sizes in `three` (the minimum a three-phase decode step
    costs at the chip's own read rate and launch gaps), and a loop of dense
    fp16 MFMAs.  HIP events on the launch stream around graph replays.
    (A region of at least twice the largest read keeps every window cold.)"""
    torch, moe = c.torch, c.moe
    out = {}
    stream = torch.cuda.Stream()
    region = max([1 << 30] + [2 * ((nb + 4095) // 4096 * 4096) for nb in read_bytes])
    buf = torch.empty(region, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.empty(65536, dtype=torch.int32, device="cuda")
    n = 40

    def windows(size):
        size = (size + 4095) // 4096 * 4096
        k = region // size
        return [buf[(i % k) * size:(i % k) * size + size] for i in range(n)], size

    grids = (256, 512, 1024, 2048, 16384)        # the best of these workgroup counts
    for nb in read_bytes:
        ws, size = windows(nb)
        best = min((graph_time(c, lambda i: moe.moe_probe_stream_read(ws[i], sink, g), 0, n, stream), g)
                   for g in grids)
        out.setdefault("stream_read", []).append({"bytes": size, "us": round(best[0] * 1e3, 3),
                                                  "GBps": round(size / (best[0] * 1e-3) / 1e9, 1),
                                                  "workgroups": best[1]})
    if three:
        parts = [windows(nb) for nb in three]

        def skel_for(g):
            def skel(i):
                for ws, _ in parts:
                    moe.moe_probe_stream_read(ws[i], sink, g)
            return skel

        best = min((graph_time(c, skel_for(g), 0, n, stream), g) for g in grids)
        out["three_launch"] = {"bytes": [sz for _, sz in parts], "us": round(best[0] * 1e3, 3),
                               "workgroups": best[1]}
    if mfma:
        fsink = torch.empty(1024 * 256, dtype=torch.float32, device="cuda")
        flops = [0.0]

        def mm(i):
            flops[0] = moe.moe_probe_mfma_f16(4000, fsink, 1024)

        ms_ = graph_time(c, mm, 0, 5, stream)
        out["mfma_f16_TFLOPs"] = round(flops[0] / (ms_ * 1e-3) / 1e12, 1)
    del buf
    torch.cuda.empty_cache()
    return out


def ffn_traffic(name):
    """HBM bytes per expert-FFN launch pair from the committed rocprofv3 counter
    record (profiles/decode80b_ffn_traffic.md), scaled by its copy calibration;
    None when there is no record for this workload or the kernels' sources
    changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{name}_ffn_traffic.md")
    if not os.path.exists(path):
        return None
    rec = None
    for line in open(path):
        if line.startswith("traffic-record:"):
            rec = json.loads(line.split(":", 1)[1])
    if rec is None:
        return None
    h = hashlib.sha256()
    for src in rec["sources"]:
        h.update(open(os.path.join(ROOT, src), "rb").read())
    if h.hexdigest() != rec["sources_sha256"]:
        return None
    fs = rec["copy_probe_bytes"] / 1024 / rec["copy_fetch_kib"]
    wsc = rec["copy_probe_bytes"] / 1024 / rec["copy_write_kib"]
    return int(sum(rec["fetch_kib_per_dispatch"].values()) * 1024 * fs
               + sum(rec["write_kib_per_dispatch"].values()) * 1024 * wsc)


def run_decode(c, name, K, W, R, cpu_steps, eager=False):
    torch, ms, moe = c.torch, c.ms, c.moe
    cfg = ms.scaled(ms.CONFIGS[name], n_slots=ms.CONFIGS[name].E)
    nsteps = K + W
    log(f"{name}: all-resident, R={R} replicas, steps={K} warmup={W}")
    layers = build_layers(c, cfg, R)
    xall = x_steps(c, cfg, nsteps)
    ws = torch.zeros(layers[0].workspace_bytes(1, moe.MOE_PATH_DECODE), dtype=torch.uint8, device="cuda")
    y = torch.empty((nsteps, 1, cfg.d), dtype=torch.float32, device="cuda")
    idx = torch.empty((nsteps, 1, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((nsteps, 1, cfg.k), dtype=torch.float32, device="cuda")
    s = torch.empty((nsteps, 1), dtype=torch.float32, device="cuda")

    def step(i):
        moe.moe_layer_forward(layers[i % R], xall[i], path=moe.MOE_PATH_DECODE, workspace=ws,
                              out=(y[i], idx[i], w[i], s[i]))

    for i in range(nsteps):                 # eager reference for the graph replays
        step(i)
    torch.cuda.synchronize()
    y_eager, idx_eager = y.clone(), idx.clone()
    stream = torch.cuda.Stream()
    if eager:
        with torch.cuda.stream(stream):
            for i in range(W):
                step(i)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(W, nsteps):
                step(i)
            e1.record(stream)
            torch.cuda.synchronize()
        ms_step = e0.elapsed_time(e1) / K
    else:
        graph_time(c, step, 0, W, stream)
        ms_step = graph_time(c, step, W, nsteps, stream)
    assert torch.equal(y, y_eager) and torch.equal(idx, idx_eager), "graph replay differs from eager"

    # dominant kernels: the expert FFN (gate/up + down launches) of every
    # timed step, replayed alone from a graph with the routing the layer
    # produced; HIP events on the launch stream
    wsf = torch.zeros(moe.moe_ffn_workspace_bytes(cfg.d, cfg.I, cfg.I_shared, 1, cfg.k, cfg.E,
                                                  moe.MOE_PATH_DECODE, cfg.bits), dtype=torch.uint8, device="cuda")
    yf = torch.empty_like(y)

    def ffn(i):
        L = layers[i % R]
        moe.moe_expert_ffn(L.pool, L.shared_blob, cfg.I_shared, xall[i], idx[i], w[i], s[i],
                           workspace=wsf, out=yf[i])

    ffn_ms = graph_time(c, ffn, W, nsteps, stream)
    assert torch.equal(yf[W:], y[W:]), "FFN-only replay differs from the layer"
    expert_bytes = (cfg.k + 1) * moe.moe_blob_bytes(cfg.d, cfg.I, cfg.bits)
    router_bytes = (cfg.E + 1) * cfg.d * 4
    achieved = expert_bytes / (ffn_ms * 1e-3) / 1e9
    layer_gbs = expert_bytes / (ms_step * 1e-3) / 1e9
    # single-step latency: one step, then a wait for it, 200 times (eager
    # launches through the C ABI; and one-step graph replays)
    lat_e, lat_g = [], []
    with torch.cuda.stream(stream):
        for i in range(200):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step(W + i % K)
            e1.record(stream)
            e1.synchronize()
            lat_e.append(e0.elapsed_time(e1) * 1e3)
        g1 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g1, stream=stream):
            step(W)
        for i in range(200):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g1.replay()
            e1.record(stream)
            e1.synchronize()
            lat_g.append(e0.elapsed_time(e1) * 1e3)
    ceil = measure_ceilings(c, read_bytes=(expert_bytes, expert_bytes + router_bytes),
                            three=(router_bytes, expert_bytes * 2 // 3, expert_bytes // 3))
    read_gbs = ceil["stream_read"][0]["GBps"]
    metric, data, wdt = labels(cfg)
    out = {
        "metric": metric, "value": round(1000.0 / ms_step, 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": f"{wdt} weights, bf16 activations, fp32 accumulate", "data": data,
        "config": {"workload": f"{'80B' if cfg.E == 512 else '35B'}-shape batch-1 decode MoE layer, "
                               f"{wdt} experts, all {cfg.E} experts resident",
                   "T": 1, "d": cfg.d, "E": cfg.E, "k": cfg.k, "I": cfg.I, "I_shared": cfg.I_shared,
                   "group": 64, "bits": cfg.bits, "replicas": R, "hip_graph": not eager},
        "expert_bytes_per_step": expert_bytes,
        "all_bytes_per_step": expert_bytes + router_bytes,
        "layer_expert_GBps": round(layer_gbs, 1),
        "layer_expert_frac_of_hbm_peak": round(layer_gbs / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm",
                     "kernel": ("expert FFN replayed with the routing given (one moe_expert_ffn call: "
                                "gate_up_kernel RAW instance + down_decode_pipe_kernel; inside the layer the "
                                "gate/up instance also selects the experts from the logits)" if cfg.bits != 32
                                else "expert FFN replayed with the routing given (gate_up_f32_kernel + "
                                     "down_decode_f32_kernel, the same kernels the layer runs)"),
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": ffn_traffic(name),
                     "avg_us": round(ffn_ms * 1e3, 3),
                     "measured_peak": read_gbs,
                     "measured_peak_what": f"one-launch streaming read of the same {expert_bytes} bytes, cold",
                     "frac_of_measured": round(achieved / read_gbs, 4)},
        "layer_frac_of_measured_read": round(layer_gbs / read_gbs, 4),
        "p50_step_us": {"eager": round(float(np.median(lat_e)), 2), "graph": round(float(np.median(lat_g)), 2)},
        "ceilings": ceil,
    }
    if cpu_steps > 0:
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(c, cfg, steps=cpu_steps)
    return out


def prefetch_model(moe, trace, E, slots, budgets, lo):
    """What a prefetcher driven by the usage counts could do on this routing
    trace (trace[t] = step t's selections): the pool's own LFU + recency
    policy (moe.Lfu) is replayed over the trace, and before every step t >= lo
    the `b` non-resident experts with the most selections so far (ties: most
    recent) are the candidates a prefetcher would copy into idle link time.
    Reports, per budget b, the fraction of candidates that step t selects and
    the misses of step t they would have covered.  The evictions such
    prefetches would force are not charged, so the coverage is an upper bound."""
    lfu = moe.Lfu(E, slots)
    resident = np.zeros(E, bool)
    count = np.zeros(E, np.int64)
    last = np.full(E, -1, np.int64)
    picked = {b: 0 for b in budgets}
    covered = {b: 0 for b in budgets}
    misses = 0
    n = 0
    for t, sel in enumerate(trace):
        need = np.unique(sel)
        if t >= lo:
            miss = set(need[~resident[need]].tolist())
            misses += len(miss)
            n += 1
            nonres = np.flatnonzero(~resident)
            order = nonres[np.lexsort((-last[nonres], -count[nonres]))]
            for b in budgets:
                cand = set(order[:b].tolist())
                picked[b] += len(cand & set(need.tolist()))
                covered[b] += len(cand & miss)
        for e, _, v in lfu.plan(sel):
            resident[e] = True
            if v >= 0:
                resident[v] = False
        np.add.at(count, sel, 1)
        last[sel] = t
    lfu.close()
    return {"misses_per_step": round(misses / max(1, n), 3),
            "by_budget": [{"experts_prefetched_per_step": b,
                           "fraction_selected_next_step": round(picked[b] / max(1, n * b), 4),
                           "misses_covered_per_step": round(covered[b] / max(1, n), 4)} for b in budgets]}


def run_refill(c, K, W, n_slots=None, host=None, mode="serial"):
    """A pool of n_slots (default 256) over 512 experts, refilled between
    router and experts by LFU + recency from pinned host memory; outputs
    checked bit-identical to an all-resident twin.  mode "serial": router ->
    host plan and refill -> experts in sequence; "streamed": one
    moe_layer_forward_streamed call per step (the misses copy in on a second
    stream while the resident experts compute); "offload": one
    moe_layer_forward_offload call per step (plan and copy on the GPU, no
    host wait).  The serial run adds X steps after the timed ones
    with events around each refill (the pull kernel and the slot-table edit)
    for the link's busy time, and models a usage-count prefetcher on the
    step's routing trace (prefetch_model)."""
    torch, ms, moe = c.torch, c.ms, c.moe
    cfg = ms.CONFIGS["decode80b"]
    if n_slots is not None:
        cfg = ms.scaled(cfg, n_slots=n_slots)
    streamed, offload = mode == "streamed", mode == "offload"
    X = 50 if mode == "serial" else 0
    nsteps = K + W + X
    log(f"refill80b: {cfg.n_slots} slots over {cfg.E} experts, steps={nsteps}")
    if host is None:
        host = packed_experts(c, cfg, pinned=True)
    stride = host.shape[1]
    twin = build_layers(c, ms.scaled(cfg, n_slots=cfg.E), 1, staging=host.cuda())[0]
    pool = moe.Pool(cfg.E, cfg.n_slots, cfg.d, cfg.I)
    xall = x_steps(c, cfg, nsteps)
    wsr = torch.zeros(moe.moe_router_workspace_bytes(1, cfg.d, cfg.E), dtype=torch.uint8, device="cuda")
    wsf = torch.zeros(moe.moe_ffn_workspace_bytes(cfg.d, cfg.I, cfg.I_shared, 1, cfg.k, cfg.E,
                                                  moe.MOE_PATH_DECODE), dtype=torch.uint8, device="cuda")
    y = torch.empty((nsteps, 1, cfg.d), dtype=torch.float32, device="cuda")
    idx = torch.empty((nsteps, 1, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((nsteps, 1, cfg.k), dtype=torch.float32, device="cuda")
    s = torch.empty((nsteps, 1), dtype=torch.float32, device="cuda")
    idx_host = torch.empty((cfg.k,), dtype=torch.int32, pin_memory=True)
    part = moe.Layer(twin.w_router, twin.logit_bias, pool, twin.shared_blob, cfg.I_shared, cfg.k)
    wsl = torch.zeros(part.workspace_bytes(1, moe.MOE_PATH_DECODE), dtype=torch.uint8, device="cuda")
    copy_stream = torch.cuda.Stream()

    def step(i, ev=None):
        if offload:
            moe.moe_layer_forward_offload(part, xall[i], host, workspace=wsl, out=(y[i], idx[i], w[i], s[i]))
            return
        if streamed:
            moe.moe_layer_forward_streamed(part, xall[i], host, copy_stream=copy_stream, workspace=wsl,
                                           out=(y[i], idx[i], w[i], s[i]))
            return
        moe.moe_router_topk(xall[i], twin.w_router, twin.logit_bias, cfg.k, workspace=wsr,
                            out=(idx[i], w[i], s[i]))
        if ev:
            ev[2].record()
        idx_host.copy_(idx[i, 0], non_blocking=True)
        torch.cuda.current_stream().synchronize()
        if ev:
            ev[0].record()
        pool.refill(idx_host.numpy(), host, stride)
        if ev:
            ev[1].record()
        moe.moe_expert_ffn_int4(pool, twin.shared_blob, cfg.I_shared, xall[i], idx[i], w[i], s[i],
                                workspace=wsf, out=y[i])

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    st0 = pool.stats()
    t0 = time.perf_counter()
    for i in range(W, W + K):
        step(i)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    st1 = pool.stats()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(X)]
    for i in range(W + K, nsteps):
        step(i, evs[i - W - K])
    torch.cuda.synchronize()
    st2 = pool.stats()
    assert pool.check_error() == moe.MOE_OK
    # all-resident twin over the same steps: bit-identical outputs
    wst = torch.zeros(twin.workspace_bytes(1, moe.MOE_PATH_DECODE), dtype=torch.uint8, device="cuda")
    yt = torch.empty_like(y)
    it = torch.empty_like(idx)
    for i in range(nsteps):
        moe.moe_layer_forward(twin, xall[i], path=moe.MOE_PATH_DECODE, workspace=wst,
                              out=(yt[i], it[i], torch.empty_like(w[i]), torch.empty_like(s[i])))
    torch.cuda.synchronize()
    identical = bool(torch.equal(yt, y) and torch.equal(it, idx))
    # the workload's contract: every step bit-identical to the all-resident layer
    assert identical, "refilled pool differs from the all-resident layer"
    hits, misses = st1["hits"] - st0["hits"], st1["misses"] - st0["misses"]
    ms_step = dt * 1e3 / K
    link = {}
    if X:
        # the link: busy while the pull kernel reads the missing blobs from
        # pinned host memory; idle for the rest of the step
        pull_us = float(np.mean([a.elapsed_time(b) for a, b, _ in evs])) * 1e3
        # router done -> refill enqueued: selections to the host, the host's
        # wake-up and plan, and the submission of the pull
        host_us = float(np.mean([r.elapsed_time(a) for a, _, r in evs])) * 1e3
        pulled = (st2["bytes_loaded"] - st1["bytes_loaded"]) / X
        rate = pulled / (pull_us * 1e-6) if pull_us > 0 else 0.0
        idle_us = max(0.0, ms_step * 1e3 - pull_us)
        idle_blobs = idle_us * 1e-6 * rate / stride if rate else 0.0
        blob_us = stride / rate * 1e6 if rate else 0.0
        model = prefetch_model(moe, idx[:, 0].cpu().numpy(), cfg.E, cfg.n_slots, (1, 2, 4, 8), W)
        best = max(model["by_budget"], key=lambda r: r["misses_covered_per_step"]
                   if r["experts_prefetched_per_step"] <= max(1, int(idle_blobs)) else -1)
        link = {"link": {"pull_us_per_step": round(pull_us, 1), "pull_GBps": round(rate / 1e9, 1),
                         "host_round_trip_us_per_step": round(host_us, 1),
                         "busy_frac_of_step": round(pull_us / (ms_step * 1e3), 3),
                         "idle_us_per_step": round(idle_us, 1), "idle_blobs_per_step": round(idle_blobs, 2),
                         "us_per_blob": round(blob_us, 1), "steps": X},
                "usage_prefetch_model": {**model,
                                         "best_within_idle_link": best,
                                         "step_us_saved_at_most": round(best["misses_covered_per_step"] * blob_us, 2),
                                         "perfect_predictor_step_us_saved_at_most":
                                             round(min(idle_blobs, misses / max(1, K)) * blob_us, 1)}}
    return {"metric": METRIC, "value": round(K / dt, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
            "warmup": W, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "int4 weights, bf16 activations, fp32 accumulate", "data": DATA,
            "config": {"workload": f"80B-shape batch-1 decode, {cfg.n_slots}-slot HBM pool refilled by "
                                   "LFU+recency from pinned host memory (wall clock incl. PCIe and host policy)"
                                   + {"serial": ", router -> host plan and refill -> experts in sequence",
                                      "streamed": ", misses copied on a second stream while the resident "
                                                  "experts compute",
                                      "offload": ", plan and copy on the GPU (router -> LFU plan kernel -> "
                                                 "copy kernel -> experts, no host wait)"}[mode],
                       "T": 1, "d": cfg.d, "E": cfg.E, "k": cfg.k, "slots": cfg.n_slots, "mode": mode},
            "hit_rate": round(hits / max(1, hits + misses), 4),
            "hit_rate_all_steps": round(st1["hits"] / max(1, st1["hits"] + st1["misses"]), 4),
            "pcie_bytes_per_step": round((st1["bytes_loaded"] - st0["bytes_loaded"]) / K),
            "bit_identical_to_all_resident": identical, **link}


def mfma_kernels(cfg, T):
    """The launches of the matrix-core expert FFN for T tokens (the library
    takes the weight-streaming GEMMs while T k <= 4 E and d <= 4096)."""
    if T * cfg.k <= 4 * cfg.E and cfg.d <= 4096:
        return "prefill_plan_kernel + stream_gate_up_kernel + stream_down_kernel"
    return "prefill_xprep_kernel + prefill_plan_kernel + prefill_gate_up_kernel + prefill_down_kernel"


def ffn_replay(c, cfg, layers, xall, idx, w, s, lo, hi, stream, path):
    """The expert FFN of steps lo..hi-1 replayed alone from a graph (one
    moe_expert_ffn call per step with that step's routing and bucketing, the
    layer's replica), HIP events on the graph's stream; the last step's
    partial outputs, combined, must equal the layer's output bit for bit.
    Returns (ms per call, the launches of one call)."""
    torch, moe = c.torch, c.moe
    T = xall.shape[1]
    R = len(layers)
    buckets = [moe.moe_bucket_tokens(idx[i], cfg.E) for i in range(hi)]
    rpath = moe.MOE_PATH_BATCHED if cfg.bits == 32 else moe.MOE_PATH_PREFILL
    ws = torch.zeros(moe.moe_ffn_workspace_bytes(cfg.d, cfg.I, cfg.I_shared, T, cfg.k, cfg.E, rpath, cfg.bits),
                     dtype=torch.uint8, device="cuda")
    partial = torch.empty((T * cfg.k, cfg.d), dtype=torch.float32, device="cuda")
    shared_out = torch.empty((T, cfg.d), dtype=torch.float32, device="cuda")

    def ffn(i):
        L = layers[i % R]
        _, o, p = buckets[i]
        moe.moe_expert_ffn(L.pool, L.shared_blob, cfg.I_shared, xall[i], idx[i], w[i], s[i], path=rpath,
                           offsets=o, pair_ids=p, workspace=ws, out=(partial, shared_out))

    ms = graph_time(c, ffn, lo, hi, stream)
    return ms, partial, shared_out, (mfma_kernels(cfg, T) if cfg.bits != 32
                                     else "plan_kernel + gate_up_f32_kernel + down_batched_f32_kernel")


def run_batched(c, K, W, R, name="batch80b"):
    """T=64 independent tokens.  The layer runs on the path MOE_PATH_AUTO
    picks for 64 tokens (bucketing, then the grouped GEMMs on the matrix
    cores); the bucketed-GEMV path is timed beside it on the same steps."""
    torch, ms, moe = c.torch, c.ms, c.moe
    cfg = ms.CONFIGS[name]
    T = cfg.T
    nsteps = K + W
    log(f"{name}: T={T}, R={R}, steps={K}")
    layers = build_layers(c, cfg, R)
    xall = x_steps(c, cfg, nsteps)
    y = torch.empty((nsteps, T, cfg.d), dtype=torch.float32, device="cuda")
    idx = torch.empty((nsteps, T, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((nsteps, T, cfg.k), dtype=torch.float32, device="cuda")
    s = torch.empty((nsteps, T), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()
    times = {}
    for path in (moe.MOE_PATH_BATCHED, moe.MOE_PATH_AUTO):
        ws = torch.zeros(layers[0].workspace_bytes(T, path), dtype=torch.uint8, device="cuda")

        def step(i):
            moe.moe_layer_forward(layers[i % R], xall[i], path=path, workspace=ws,
                                  out=(y[i], idx[i], w[i], s[i]))

        graph_time(c, step, 0, W, stream)
        times[path] = graph_time(c, step, W, nsteps, stream)
    ms_step = times[moe.MOE_PATH_AUTO]
    ids = idx.cpu().numpy()
    distinct = float(np.mean([len(np.unique(ids[i])) for i in range(W, nsteps)]))
    expert_bytes = (distinct + 1) * moe.moe_blob_bytes(cfg.d, cfg.I, cfg.bits)
    gbs = expert_bytes / (ms_step * 1e-3) / 1e9
    # dominant kernels: the expert FFN launch group of the AUTO path, replayed
    # with every timed step's own routing and bucketing
    ffn_ms, partial, shared_out, ffn_kernels = ffn_replay(c, cfg, layers, xall, idx, w, s, W, nsteps, stream,
                                                          moe.MOE_PATH_AUTO)
    yc = moe.moe_combine(partial, shared_out, w[nsteps - 1], s[nsteps - 1])
    torch.cuda.synchronize()
    assert torch.equal(yc, y[nsteps - 1]), "FFN-only replay differs from the layer"
    ffn_kernels = "expert FFN replayed with the routing given: " + ffn_kernels
    achieved = expert_bytes / (ffn_ms * 1e-3) / 1e9
    ceil = measure_ceilings(c, read_bytes=(int(expert_bytes),))
    read_gbs = ceil["stream_read"][0]["GBps"]
    metric, data, wdt = labels(cfg)
    return {"metric": metric, "value": round(T * 1000.0 / ms_step, 1), "unit": "tokens/s", "n_gpus": 1,
            "steps": K, "warmup": W, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None,
            "dtype": (f"{wdt} weights -> fp16 MFMA, fp32 accumulate; fp32 router" if cfg.bits != 32
                      else "f32 weights, bf16 activations, fp32 accumulate"), "data": data,
            "config": {"workload": f"80B-shape batched decode, T=64 independent tokens, {wdt} experts, "
                                   "all experts resident",
                       "T": T, "d": cfg.d, "E": cfg.E, "k": cfg.k, "bits": cfg.bits, "replicas": R,
                       "path": ("auto: bucketing + grouped GEMMs on the matrix cores" if cfg.bits != 32
                                else "auto: bucketing + bucketed f32 GEMVs")},
            "distinct_experts_per_step": round(distinct, 1),
            "layer_expert_GBps": round(gbs, 1), "layer_expert_frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "gemv_path_ms_per_step": round(times[moe.MOE_PATH_BATCHED], 5),
            "roofline": {"bound": "hbm", "kernel": ffn_kernels, "achieved": round(achieved, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": ffn_traffic(name), "avg_us": round(ffn_ms * 1e3, 3),
                         "bytes_per_launch": int(expert_bytes),
                         "measured_peak": read_gbs,
                         "measured_peak_what": f"one-launch streaming read of {int(expert_bytes)} bytes, cold",
                         "frac_of_measured": round(achieved / read_gbs, 4)},
            "ceilings": ceil}


def run_prefill(c, name, reps):
    torch, ms, moe = c.torch, c.ms, c.moe
    cfg = ms.CONFIGS[name]
    T = cfg.T
    log(f"{name}: T={T}, reps={reps}")
    L = build_layers(c, ms.scaled(cfg, n_slots=cfg.E), 1)[0]
    x = x_steps(c, cfg, 1, T)[0]
    ws = torch.zeros(L.workspace_bytes(T, moe.MOE_PATH_PREFILL), dtype=torch.uint8, device="cuda")
    out = (torch.empty((T, cfg.d), dtype=torch.float32, device="cuda"),
           torch.empty((T, cfg.k), dtype=torch.int32, device="cuda"),
           torch.empty((T, cfg.k), dtype=torch.float32, device="cuda"),
           torch.empty((T,), dtype=torch.float32, device="cuda"))

    def step(i):
        moe.moe_layer_forward(L, x, path=moe.MOE_PATH_PREFILL, workspace=ws, out=out)

    stream = torch.cuda.Stream()
    graph_time(c, step, 0, 2, stream)
    ms_call = graph_time(c, step, 0, reps, stream)
    assert L.pool.check_error() == moe.MOE_OK
    counts = np.bincount(out[1].cpu().numpy().ravel(), minlength=cfg.E)
    flops = 6.0 * cfg.d * (T * cfg.k * cfg.I + T * cfg.I_shared)
    router_flops = 2.0 * T * cfg.d * (cfg.E + 1)
    tf = flops / (ms_call * 1e-3) / 1e12
    # dominant kernels: the grouped GEMMs' launch group replayed with the routing given
    xs1, id1, w1, s1 = x.unsqueeze(0), out[1].unsqueeze(0), out[2].unsqueeze(0), out[3].unsqueeze(0)
    xr = xs1.expand(reps, -1, -1)
    ffn_ms, partial, shared_out, ffn_kernels = ffn_replay(c, cfg, [L], xr, id1.expand(reps, -1, -1),
                                                          w1.expand(reps, -1, -1), s1.expand(reps, -1), 0, reps,
                                                          stream, moe.MOE_PATH_PREFILL)
    yc = moe.moe_combine(partial, shared_out, out[2], out[3])
    torch.cuda.synchronize()
    assert torch.equal(yc, out[0]), "FFN-only replay differs from the layer"
    ffn_tf = flops / (ffn_ms * 1e-3) / 1e12
    ceil = measure_ceilings(c, mfma=True)
    metric, data, wdt = labels(cfg)
    return {"metric": metric, "value": round(T * 1000.0 / ms_call, 1), "unit": "tokens/s", "n_gpus": 1,
            "steps": reps, "warmup": 2, "ms_per_step": round(ms_call, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None,
            "dtype": f"{wdt} weights -> fp16 MFMA, fp32 accumulate; fp32 router", "data": data,
            "config": {"workload": f"80B-shape prefill layer, T={T}, {wdt} experts, "
                                   f"{'Zipf-skewed' if cfg.alpha else 'unbiased'} router",
                       "T": T, "d": cfg.d, "E": cfg.E, "k": cfg.k, "I": cfg.I, "bits": cfg.bits},
            "expert_gflop": round(flops / 1e9, 1), "router_gflop": round(router_flops / 1e9, 2),
            "layer_expert_TFLOPs": round(tf, 1), "frac_of_mfma_f16_peak": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
            "max_bucket": int(counts.max()),
            "roofline": {"bound": "mfma",
                         "kernel": "expert FFN replayed with the routing given: " + ffn_kernels,
                         "achieved": round(ffn_tf, 1), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(ffn_tf / MFMA_F16_PEAK_TFLOPS, 4), "traffic": ffn_traffic(name),
                         "avg_us": round(ffn_ms * 1e3, 3), "flops_per_launch": flops,
                         "measured_peak": ceil["mfma_f16_TFLOPs"],
                         "measured_peak_what": "loop of dense v_mfma_f32_32x32x16_f16 on register operands",
                         "frac_of_measured": round(ffn_tf / ceil["mfma_f16_TFLOPs"], 4)},
            "ceilings": ceil}


def run_chain(c, K, W, L=48):
    """L layers of the 80B decode shape per token (the 80B model stacks 48
    MoE layers), each layer its own router, shared expert and 512-expert pool
    (distinct HBM, 43 GB in all), applied by moe_chain_forward as pre-norm
    residual blocks; K tokens captured in one HIP graph."""
    torch, ms, moe = c.torch, c.ms, c.moe
    cfg = ms.scaled(ms.CONFIGS["decode80b"], n_slots=512)
    log(f"chain80b: {L} layers, steps={K} warmup={W}")
    staging = packed_experts(c, cfg)
    layers = []
    for l in range(L):
        cl = ms.scaled(cfg, seed=cfg.seed + 97 * l)
        layers.append(build_layers(c, cl, 1, staging=staging)[0])
        if l % 8 == 7:
            log(f"layer {l + 1}/{L} ready")
    del staging
    torch.cuda.empty_cache()
    chain = moe.Chain(layers)
    n = K + W
    xall = x_steps(c, cfg, n)
    ws = torch.zeros(chain.workspace_bytes(1, moe.MOE_PATH_DECODE), dtype=torch.uint8, device="cuda")
    out = torch.empty((n, 1, cfg.d), dtype=torch.bfloat16, device="cuda")

    def step(i):
        moe.moe_chain_forward(chain, xall[i], path=moe.MOE_PATH_DECODE, workspace=ws, out=out[i])

    for i in range(n):
        step(i)
    torch.cuda.synchronize()
    ref = out.clone()
    stream = torch.cuda.Stream()
    graph_time(c, step, 0, W, stream)
    ms_tok = graph_time(c, step, W, n, stream)
    assert torch.equal(out, ref), "graph replay differs from eager"
    for Lr in layers:
        assert Lr.pool.check_error() == moe.MOE_OK
    expert_bytes = L * (cfg.k + 1) * moe.moe_blob_bytes(cfg.d, cfg.I)
    gbs = expert_bytes / (ms_tok * 1e-3) / 1e9
    return {"metric": "MoE-stack decode tokens/s (48 routed-expert layers per token, int4, 80B shape)",
            "value": round(1000.0 / ms_tok, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
            "ms_per_step": round(ms_tok, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "int4 weights, bf16 activations, fp32 accumulate", "data": DATA,
            "config": {"workload": f"chain of {L} 80B-shape MoE layers per token (pre-norm residual blocks), "
                                   "batch-1 decode, every layer's 512 experts resident",
                       "layers": L, "T": 1, "d": cfg.d, "E": cfg.E, "k": cfg.k, "I": cfg.I, "hip_graph": True},
            "us_per_layer": round(ms_tok * 1e3 / L, 2),
            "expert_bytes_per_token": expert_bytes,
            "layer_expert_GBps": round(gbs, 1), "layer_expert_frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


def copy_probe(mb):
    """A plain device-to-device copy of known size, for scaling the
    FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    n = mb << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "copies": 5}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--replicas", type=int, default=32)
    ap.add_argument("--cpu-steps", type=int, default=120)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--eager", action="store_true", help="enqueue decode steps one by one (no HIP graph)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MB",
                    help="only copy an MB-sized device buffer 5 times (calibrates HBM byte counters)")
    ap.add_argument("--workload", default="decode80b",
                    choices=["decode80b", "decode35b", "refill80b", "stream80b", "offload80b", "batch80b", "prefill80b",
                             "prefill80b_zipf", "decode80b_int8", "batch80b_int8", "prefill80b_int8",
                             "decode80b_f32", "batch80b_f32", "chain80b", "all", "refill_sweep", "ceiling"])
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the MoE layer here runs on a single MI355X "
              "(no multi-GPU path is built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe > 0:
        copy_probe(args.copy_probe)
        return
    c = Ctx()
    c.torch.cuda.set_device(0)
    cpu = 0 if args.no_cpu else args.cpu_steps
    todo = ["decode80b", "decode35b", "refill80b", "stream80b", "offload80b", "batch80b", "prefill80b", "prefill80b_zipf",
            "decode80b_int8", "batch80b_int8", "prefill80b_int8", "decode80b_f32", "batch80b_f32",
            "chain80b"] \
        if args.workload == "all" else [args.workload]
    ms = c.ms
    for wl in todo:
        if wl == "ceiling":
            res = {"metric": "measured ceilings of this MI355X", "n_gpus": 1,
                   "ceilings": measure_ceilings(c, read_bytes=(19464192, 23666688, 605 << 20),
                                                three=(4202496, 12976128, 6488064), mfma=True),
                   "spec": {"hbm_GBps": HBM_PEAK_GBS, "mfma_f16_TFLOPs": MFMA_F16_PEAK_TFLOPS}}
            print(json.dumps(res), flush=True)
            continue
        if wl in ("decode80b", "decode35b", "decode80b_int8", "decode80b_f32"):
            # f32 blobs are 12.6 MB: 4 replicas already keep a step's 138 MB
            # out of the 256 MB last-level cache until its next use
            reps = min(args.replicas, 4) if wl.endswith("f32") else args.replicas
            # oracle sample: ~10 s of CPU (wider experts take longer per step)
            csteps = 0 if cpu == 0 else (cpu if wl in ("decode80b", "decode35b")
                                         else max(1, cpu // 2) if wl.endswith("int8") else max(1, cpu // 4))
            res = run_decode(c, wl, args.steps, args.warmup, reps, csteps, args.eager)
        elif wl in ("refill80b", "stream80b", "offload80b"):
            res = run_refill(c, min(args.steps, 300), min(args.warmup, 50),
                             mode={"refill80b": "serial", "stream80b": "streamed", "offload80b": "offload"}[wl])
            if cpu:
                log("timing the CPU oracle")
                res["cpu_baseline"] = cpu_baseline(c, ms.CONFIGS["decode80b"], steps=cpu)
        elif wl == "refill_sweep":
            # hit rate and tokens/s against the pool size (the pages report that
            # pool size barely changes speed on their SSD-backed machine), the
            # serial and the streamed step for each size
            host = packed_experts(c, c.ms.CONFIGS["decode80b"], pinned=True)
            for slots in (64, 128, 192, 256, 384, 512):
                for mode in ("serial", "streamed", "offload"):
                    res = run_refill(c, min(args.steps, 200), min(args.warmup, 50), slots, host, mode)
                    print(json.dumps(res), flush=True)
                    c.torch.cuda.empty_cache()
            continue
        elif wl == "chain80b":
            res = run_chain(c, min(args.steps, 50), min(args.warmup, 5))
            if cpu:
                log("timing the CPU oracle")
                base = ms.scaled(ms.CONFIGS["decode80b"], n_slots=512)
                res["cpu_baseline"] = chain_cpu_baseline(c, [ms.scaled(base, seed=base.seed + 97 * l)
                                                            for l in range(48)], base)
        elif wl in ("batch80b", "batch80b_int8", "batch80b_f32"):
            res = run_batched(c, min(args.steps, 100), min(args.warmup, 10), min(args.replicas, 4), wl)
            if cpu:
                log("timing the CPU oracle")
                res["cpu_baseline"] = cpu_baseline(c, ms.CONFIGS[wl], steps=1)
        else:
            res = run_prefill(c, wl, 10)
            if cpu:
                log("timing the CPU oracle")
                res["cpu_baseline"] = cpu_baseline(c, ms.CONFIGS[wl], tokens=64)
        print(json.dumps(res), flush=True)
        c.torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
