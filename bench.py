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


def cpu_baseline(c, cfg, sample_steps):
    """The oracle as it stands, on the first `sample_steps` decode steps."""
    import threadpoolctl
    ms, olayer = c.ms, c.olayer
    Wr = ms.router_weight(cfg)
    bias = ms.logit_bias(cfg)
    sh = ms.shared_raw(cfg)
    xs = [ms.x_bits(cfg, s) for s in range(sample_steps)]
    need = set()
    for xb in xs:
        idx, _, _, _ = olayer.route(xb, Wr, bias, cfg.k)
        need.update(int(e) for e in idx.ravel())
    raws = {e: ms.expert_raw(cfg, e) for e in sorted(need)}     # inputs, generated before timing
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    t0 = time.perf_counter()
    for xb in xs:
        olayer.moe_layer(xb, Wr, bias, cfg.k, raws.__getitem__, sh)
    dt = time.perf_counter() - t0
    return {"value": round(sample_steps * cfg.T / dt, 3), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"first {sample_steps} of the {cfg.steps} seeded decode steps, numpy fp64 "
                      f"(dequantise + matmul per selected expert), {dt:.1f}s"}


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
                     "kernel": ("expert FFN: gate_up_kernel + down_decode_pipe_kernel" if cfg.bits != 32
                                else "expert FFN: gate_up_f32_kernel + down_decode_f32_kernel"),
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": ffn_traffic(name),
                     "avg_us": round(ffn_ms * 1e3, 3)},
    }
    if cpu_steps > 0:
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(c, cfg, cpu_steps)
    return out


def run_refill(c, K, W, n_slots=None, host=None, streamed=False):
    """A pool of n_slots (default 256) over 512 experts, refilled between
    router and experts by LFU + recency from pinned host memory; outputs
    checked bit-identical to an all-resident twin.  streamed: one
    moe_layer_forward_streamed call per step (the misses copy in on a second
    stream while the resident experts compute) instead of router -> refill
    -> experts in sequence."""
    torch, ms, moe = c.torch, c.ms, c.moe
    cfg = ms.CONFIGS["decode80b"]
    if n_slots is not None:
        cfg = ms.scaled(cfg, n_slots=n_slots)
    nsteps = K + W
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

    def step(i):
        if streamed:
            moe.moe_layer_forward_streamed(part, xall[i], host, copy_stream=copy_stream, workspace=wsl,
                                           out=(y[i], idx[i], w[i], s[i]))
            return
        moe.moe_router_topk(xall[i], twin.w_router, twin.logit_bias, cfg.k, workspace=wsr,
                            out=(idx[i], w[i], s[i]))
        idx_host.copy_(idx[i, 0], non_blocking=True)
        torch.cuda.current_stream().synchronize()
        pool.refill(idx_host.numpy(), host, stride)
        moe.moe_expert_ffn_int4(pool, twin.shared_blob, cfg.I_shared, xall[i], idx[i], w[i], s[i],
                                workspace=wsf, out=y[i])

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    st0 = pool.stats()
    t0 = time.perf_counter()
    for i in range(W, nsteps):
        step(i)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    st1 = pool.stats()
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
    return {"metric": METRIC, "value": round(K / dt, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
            "warmup": W, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "int4 weights, bf16 activations, fp32 accumulate", "data": DATA,
            "config": {"workload": f"80B-shape batch-1 decode, {cfg.n_slots}-slot HBM pool refilled by "
                                   "LFU+recency from pinned host memory (wall clock incl. PCIe and host policy)"
                                   + (", misses copied on a second stream while the resident experts compute"
                                      if streamed else ", router -> refill -> experts in sequence"),
                       "T": 1, "d": cfg.d, "E": cfg.E, "k": cfg.k, "slots": cfg.n_slots, "streamed": streamed},
            "hit_rate": round(hits / max(1, hits + misses), 4),
            "hit_rate_all_steps": round(st1["hits"] / max(1, st1["hits"] + st1["misses"]), 4),
            "pcie_bytes_per_step": round((st1["bytes_loaded"] - st0["bytes_loaded"]) / K),
            "bit_identical_to_all_resident": identical}


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
            "gemv_path_ms_per_step": round(times[moe.MOE_PATH_BATCHED], 5)}


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
            "max_bucket": int(counts.max())}


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
                    choices=["decode80b", "decode35b", "refill80b", "stream80b", "batch80b", "prefill80b",
                             "prefill80b_zipf", "decode80b_int8", "batch80b_int8", "prefill80b_int8",
                             "decode80b_f32", "batch80b_f32", "chain80b", "all", "refill_sweep"])
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
    todo = ["decode80b", "decode35b", "refill80b", "stream80b", "batch80b", "prefill80b", "prefill80b_zipf",
            "decode80b_int8", "batch80b_int8", "prefill80b_int8", "decode80b_f32", "batch80b_f32",
            "chain80b"] \
        if args.workload == "all" else [args.workload]
    for wl in todo:
        if wl in ("decode80b", "decode35b", "decode80b_int8", "decode80b_f32"):
            # f32 blobs are 12.6 MB: 4 replicas already keep a step's 138 MB
            # out of the 256 MB last-level cache until its next use
            reps = min(args.replicas, 4) if wl.endswith("f32") else args.replicas
            res = run_decode(c, wl, args.steps, args.warmup, reps,
                             cpu if wl == "decode80b" else 0, args.eager)
        elif wl in ("refill80b", "stream80b"):
            res = run_refill(c, min(args.steps, 300), min(args.warmup, 50), streamed=wl == "stream80b")
        elif wl == "refill_sweep":
            # hit rate and tokens/s against the pool size (the pages report that
            # pool size barely changes speed on their SSD-backed machine), the
            # serial and the streamed step for each size
            host = packed_experts(c, c.ms.CONFIGS["decode80b"], pinned=True)
            for slots in (64, 128, 192, 256, 384, 512):
                for streamed in (False, True):
                    res = run_refill(c, min(args.steps, 200), min(args.warmup, 50), slots, host, streamed)
                    print(json.dumps(res), flush=True)
                    c.torch.cuda.empty_cache()
            continue
        elif wl == "chain80b":
            res = run_chain(c, min(args.steps, 50), min(args.warmup, 5))
        elif wl in ("batch80b", "batch80b_int8", "batch80b_f32"):
            res = run_batched(c, min(args.steps, 100), min(args.warmup, 10), min(args.replicas, 4), wl)
        else:
            res = run_prefill(c, wl, 10)
        print(json.dumps(res), flush=True)
        c.torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
