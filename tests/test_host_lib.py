"""Host-side checks of libmoe355 that need no GPU: the library loads and
exports every entry point its header declares, the C packer agrees byte for
byte with the oracle's independent packer, the C LFU + recency policy agrees
with the oracle simulation and the hand-derived traces, and argument
validation rejects bad calls before any device work."""
import ctypes as C
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import moe_synth as ms
import sparse_moe_decode_router_amd as moe
from oracle import layer as olayer
from oracle import lfu as olfu
from oracle import quant as oquant
import golden_io

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            src = open(os.path.join(ROOT, "include", h)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names.update(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


_MAPPED_RUNTIMES = r"""
import re, sys
sys.path.insert(0, sys.argv[1])
import sparse_moe_decode_router_amd  # the package before anything imports torch
import torch  # then torch, for the tensors a caller hands over
maps = open("/proc/self/maps").read()
for lib in ("amdhip64", "hsa-runtime64"):
    print(lib, len(set(re.findall(r"(/\S*lib" + lib + r"\S*)", maps))))
"""


def test_one_hip_runtime_whatever_the_import_order():
    """Imported before torch, the package still maps one HIP and one HSA
    runtime (torch's): two in one process leave one of them without a device."""
    out = subprocess.run([sys.executable, "-c", _MAPPED_RUNTIMES, ROOT], capture_output=True, text=True,
                         timeout=300, check=True).stdout.split()
    assert out == ["amdhip64", "1", "hsa-runtime64", "1"], out


def test_library_exports_every_declared_symbol():
    lib = C.CDLL(moe.LIB_PATH)
    names = _header_functions()
    assert len(names) >= 30
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(moe.EXPORTED)


def test_version_and_status_strings():
    assert "gfx950" in moe.version()
    assert moe._lib.moe_status_string(moe.MOE_ERR_POOL_TOO_SMALL).decode().startswith("pool")


@pytest.mark.parametrize("name", ["tiny", "decode35b"])
def test_c_pack_matches_oracle_pack(name):
    cfg = ms.CONFIGS[name]
    for e in (0, 7):
        raw = ms.expert_raw(cfg, e)
        a = moe.moe_pack_expert_int4(raw, cfg.d, cfg.I)
        b = oquant.pack_expert(raw, cfg.d, cfg.I)
        assert a.dtype == np.uint8 and np.array_equal(a, b)
        back = moe.moe_unpack_expert_int4(a, cfg.d, cfg.I)
        for m in oquant.MATS:
            for f in ("codes", "scales", "biases"):
                assert np.array_equal(back[m][f], raw[m][f])
    sh = ms.shared_raw(cfg)
    assert np.array_equal(moe.moe_pack_expert_int4(sh, cfg.d, cfg.I_shared),
                          oquant.pack_expert(sh, cfg.d, cfg.I_shared))


def test_c_pack_golden_layout():
    for d, I, bits, nbytes, stride, codes, sbs, weights in golden_io.blob_layout():
        for mat, row, col, val, off, bits32 in weights:
            raw = {m: {"weights": np.zeros(oquant.mat_dims(d, I)[m], np.float32)} for m in oquant.MATS}
            raw[mat]["weights"][row, col] = val
            blob = moe.moe_pack_expert(raw, d, I, 32)
            assert blob.size == stride and blob[off:off + 4].tobytes() == int(bits32).to_bytes(4, "little")
            assert np.count_nonzero(blob) == np.count_nonzero(blob[off:off + 4])
        assert moe.moe_blob_bytes(d, I, bits) == nbytes and moe.moe_blob_stride(d, I, bits) == stride
        dims = oquant.mat_dims(d, I)
        for mat, row, col, val, off, byte in codes:
            raw = {m: {"codes": np.zeros(dims[m], np.uint8),
                       "scales": np.zeros((dims[m][0], dims[m][1] // 64), np.float16),
                       "biases": np.zeros((dims[m][0], dims[m][1] // 64), np.float16)}
                   for m in oquant.MATS}
            raw[mat]["codes"][row, col] = val
            blob = moe.moe_pack_expert(raw, d, I, bits)
            assert np.nonzero(blob)[0].tolist() == [off] and blob[off] == byte
            back = moe.moe_unpack_expert(blob, d, I, bits)
            assert back[mat]["codes"][row, col] == val and np.count_nonzero(back[mat]["codes"]) == 1


@pytest.mark.parametrize("name", ["tiny_int8", "decode80b_int8", "tiny_f32", "decode80b_f32"])
def test_c_pack_int8_f32_matches_oracle_pack(name):
    cfg = ms.CONFIGS[name]
    for e in (0, 5):
        raw = ms.expert_raw(cfg, e)
        a = moe.moe_pack_expert(raw, cfg.d, cfg.I, cfg.bits)
        b = oquant.pack_expert(raw, cfg.d, cfg.I, cfg.bits)
        assert a.size == oquant.blob_stride(cfg.d, cfg.I, cfg.bits) and np.array_equal(a, b)
        back = moe.moe_unpack_expert(a, cfg.d, cfg.I, cfg.bits)
        for m in oquant.MATS:
            for f in raw[m]:
                assert np.array_equal(back[m][f], raw[m][f])
    assert moe.moe_blob_bytes(2048, 512, 8) == 3342336


def test_c_pack_width_checks():
    """Code width must be 4 or 8 (0 reads as 4); the int4-only entry points
    refuse 8-bit shapes; the generic packer takes 4-bit raws at bits=4."""
    assert moe.moe_blob_bytes(2048, 512, 0) == moe.moe_blob_bytes(2048, 512, 4) == 1769472
    assert moe.moe_blob_bytes(2048, 512, 5) == 0 and moe.moe_blob_stride(2048, 512, 16) == 0
    assert moe.moe_blob_bytes(2048, 512, 32) == 12582912
    cfg = ms.CONFIGS["tiny_int8"]
    raw = ms.expert_raw(cfg, 1)
    out = np.empty(moe.moe_blob_stride(cfg.d, cfg.I, 8), np.uint8)
    cp, sp, bp = (C.c_void_p * 3)(), (C.c_void_p * 3)(), (C.c_void_p * 3)()
    keep = []
    for m, name in enumerate(oquant.MATS):
        c = np.ascontiguousarray(raw[name]["codes"])
        s = np.ascontiguousarray(raw[name]["scales"]).view(np.uint16)
        b = np.ascontiguousarray(raw[name]["biases"]).view(np.uint16)
        keep += [c, s, b]
        cp[m], sp[m], bp[m] = c.ctypes.data, s.ctypes.data, b.ctypes.data
    st = moe._lib.moe_pack_expert_int4(C.byref(moe.shape(cfg.d, cfg.I, 8)), cp, sp, bp, out.ctypes.data)
    assert st == moe.MOE_ERR_INVALID_ARG
    # 8-bit codes above 15 cannot go into a 4-bit blob
    with pytest.raises(moe.MoeError):
        moe.moe_pack_expert(raw, cfg.d, cfg.I, 4)
    raw4 = ms.expert_raw(ms.CONFIGS["tiny"], 1)
    assert np.array_equal(moe.moe_pack_expert(raw4, 256, 64, 4), moe.moe_pack_expert_int4(raw4, 256, 64))
    # the code-width entry points refuse the other widths
    st = moe._lib.moe_pack_expert(C.byref(moe.shape(256, 64, 32)), cp, sp, bp, out.ctypes.data)
    assert st == moe.MOE_ERR_INVALID_ARG
    wp = (C.c_void_p * 3)(cp[0], cp[1], cp[2])
    st = moe._lib.moe_pack_expert_f32(C.byref(moe.shape(256, 64, 8)), wp, out.ctypes.data)
    assert st == moe.MOE_ERR_INVALID_ARG


def test_c_pack_rejects_bad_codes_and_shapes():
    cfg = ms.CONFIGS["tiny"]
    raw = ms.expert_raw(cfg, 0)
    raw["up"]["codes"] = raw["up"]["codes"].copy()
    raw["up"]["codes"][3, 3] = 16
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_pack_expert_int4(raw, cfg.d, cfg.I)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    assert moe.moe_blob_bytes(100, 64) == 0 and moe.moe_blob_stride(64, 96) == 0


def test_c_lfu_golden_traces():
    for name, E, slots, steps in golden_io.lfu_traces():
        lfu = moe.Lfu(E, slots)
        hits = 0
        for sel, loads, h in steps:
            assert lfu.plan(sel) == loads, (name, sel)
            st = lfu.stats()
            assert st["hits"] - hits == h
            hits = st["hits"]


def test_c_lfu_matches_oracle_sim_1000_steps():
    """80B-shape decode, 256-slot pool, Zipf-biased router: the C policy and the
    independent Python simulation agree on every load over 1000 steps, and the
    hit rate sits in the 43-70 % band the pages report."""
    cfg = ms.CONFIGS["decode80b"]
    W = ms.router_weight(cfg).astype(np.float64)
    b = ms.logit_bias(cfg).astype(np.float64)
    X = np.concatenate([olayer.bf16_to_f64(ms.x_bits(cfg, s)) for s in range(cfg.steps)])
    idx = olayer.select_topk(X @ W[:cfg.E].T + b, cfg.k)
    sim = olfu.SlotPoolSim(cfg.E, cfg.n_slots)
    lfu = moe.Lfu(cfg.E, cfg.n_slots)
    for s in range(cfg.steps):
        assert lfu.plan(idx[s]) == sim.plan(idx[s]), s
    st = lfu.stats()
    assert st["hits"] == sim.hits and st["misses"] == sim.misses
    assert 0.43 <= sim.hit_rate <= 0.70


def test_c_lfu_pool_too_small_and_bad_ids():
    lfu = moe.Lfu(4, 1)
    with pytest.raises(moe.MoeError) as ei:
        lfu.plan([0, 1])
    assert ei.value.status == moe.MOE_ERR_POOL_TOO_SMALL
    assert lfu.plan([2, 2]) == [(2, 0, -1)]       # duplicates count once
    with pytest.raises(moe.MoeError):
        lfu.plan([4])
    with pytest.raises(moe.MoeError):
        moe.Lfu(0, 1)


def test_validation_without_device_work():
    """Bad shapes are rejected on the host before any HIP call."""
    lib = moe._lib
    # router: d not a multiple of 64, k > E, E > 1024
    assert lib.moe_router_topk(None, 1, 100, None, None, 16, 2, None, None, None, None, None, 0, None) \
        == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_router_topk(None, 1, 256, None, None, 16, 17, None, None, None, None, None, 0, None) \
        == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_router_topk(None, 1, 256, None, None, 2048, 2, None, None, None, None, None, 0, None) \
        == moe.MOE_ERR_INVALID_ARG
    # T = 0 is a no-op
    assert lib.moe_router_topk(None, 0, 256, None, None, 16, 2, None, None, None, None, None, 0, None) \
        == moe.MOE_OK
    assert lib.moe_combine(None, None, None, None, 0, 2, 256, None, None) == moe.MOE_OK
    assert lib.moe_combine(None, None, None, None, 3, 0, 256, None, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_bucket_tokens(None, 1, 2, 0, None, None, None, None, 0, None) == moe.MOE_ERR_INVALID_ARG
    # pool creation with an invalid shape never reaches hipMalloc
    h = C.c_void_p()
    assert lib.moe_pool_create(16, 4, C.byref(moe.shape(100, 64)), C.byref(h)) == moe.MOE_ERR_INVALID_ARG
    # depth of the device's summation tree: T <= 8 one row per block (d/256
    # per thread, 6 butterfly, 2 tree, 1 bias); T > 8 split-K MFMA with S
    # splits (S = 8 for 64 tokens, 4 for 4096 tokens at E = 512)
    assert lib.moe_router_sum_depth(1, 2048, 512) == 17
    assert lib.moe_router_sum_depth(64, 2048, 512) == 32 + 2 + 8 + 7 + 1
    assert lib.moe_router_sum_depth(4096, 2048, 512) == 32 + 2 + 16 + 3 + 1
    assert lib.moe_router_sum_depth(8, 2048, 0) == -1
    assert lib.moe_router_workspace_bytes(1, 2048, 512) > 0


def test_workspace_sizes_monotone():
    a = moe.moe_ffn_workspace_bytes(2048, 512, 512, 1, 10, 512, moe.MOE_PATH_DECODE)
    b = moe.moe_ffn_workspace_bytes(2048, 512, 512, 64, 10, 512, moe.MOE_PATH_BATCHED)
    assert 0 < a < b


def test_prefill_path_refuses_sizes_past_its_32bit_descriptors():
    """The matrix-core path addresses activations (T d fp16) and the SwiGLU
    intermediate ((T k + T) Imax fp16) through 32-bit buffer descriptors:
    past 4 GiB it is refused (workspace size 0, the call MOE_ERR_UNSUPPORTED)
    and MOE_PATH_AUTO takes the bucketed GEMVs instead."""
    d, I, k, E = 2048, 512, 10, 512
    ws = lambda T, path: moe.moe_ffn_workspace_bytes(d, I, I, T, k, E, path)
    T_ok = 4096
    T_big = (1 << 32) // ((k + 1) * I * 2) + 1          # first T whose intermediate reaches 4 GiB
    assert ((T_big - 1) * (k + 1)) * I * 2 < (1 << 32) <= (T_big * (k + 1)) * I * 2
    assert ws(T_ok, moe.MOE_PATH_PREFILL) > 0
    assert ws(T_big - 1, moe.MOE_PATH_PREFILL) > 0
    assert ws(T_big, moe.MOE_PATH_PREFILL) == 0
    assert ws(T_big, moe.MOE_PATH_AUTO) == ws(T_big, moe.MOE_PATH_BATCHED) > 0
    assert ws(T_big - 1, moe.MOE_PATH_AUTO) == ws(T_big - 1, moe.MOE_PATH_PREFILL)
    # the activation descriptor alone: d = 8192, k = 1, I = 64 -> T d 2 bytes
    T_x = (1 << 32) // (8192 * 2)
    assert moe.moe_ffn_workspace_bytes(8192, 64, 64, T_x, 1, 16, moe.MOE_PATH_PREFILL) == 0
    assert moe.moe_ffn_workspace_bytes(8192, 64, 64, T_x - 1, 1, 16, moe.MOE_PATH_PREFILL) > 0


def test_out_of_memory_has_its_own_status():
    assert moe.MOE_ERR_OUT_OF_MEMORY == -6
    assert moe._lib.moe_status_string(moe.MOE_ERR_OUT_OF_MEMORY).decode() == "host allocation failed"
    assert moe._lib.moe_status_string(moe.MOE_ERR_INVALID_ARG).decode() == "invalid argument"
