"""Python binding for libmoe355 (routed-expert MoE layer on MI355X / gfx950).

Argument marshalling only: every step of the layer runs in the HIP kernels of
``libmoe355.so`` behind the C ABI declared in ``include/moe355.h``.  torch is
used for device memory and streams.  Importing this package does not need a
GPU; calling the device entry points does.  If the shared library has not
been built the import fails loudly (there is no fallback path).

Names follow the C ABI (``moe_router_topk`` etc.).  Device arguments are
torch CUDA tensors; host arguments of the pool calls are numpy arrays.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE355_LIB may name another build of the same library (e.g. an instrumented one)
LIB_PATH = os.environ.get("MOE355_LIB") or os.path.join(_HERE, "libmoe355.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_NOT_RESIDENT = -3
MOE_ERR_POOL_TOO_SMALL = -4
MOE_ERR_HIP = -5
MOE_ERR_OUT_OF_MEMORY = -6

MOE_PATH_AUTO = 0
MOE_PATH_DECODE = 1
MOE_PATH_BATCHED = 2
MOE_PATH_PREFILL = 3
MOE_PATH_PREFILL_TILED = 4
MOE_PATH_PREFILL_STREAM = 5

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libmoe355.so not built at {LIB_PATH}; run "
        "`python sparse_moe_decode_router_amd/build.py` (the HIP library is required; "
        "there is no CPU fallback)")

# torch first: the library's HIP runtime dependency then resolves to the one
# torch has already mapped, so the device memory and streams torch hands over
# belong to the runtime the kernels launch on.  Loaded before torch, it
# would map a second HIP and HSA runtime into the process, and one of the two
# finds no device.
import torch  # noqa: E402,F401

_lib = C.CDLL(LIB_PATH)


class moe_ffn_shape(C.Structure):
    _fields_ = [("d", C.c_int32), ("I", C.c_int32), ("group", C.c_int32), ("bits", C.c_int32)]


class moe_pool_stats(C.Structure):
    _fields_ = [(n, C.c_uint64) for n in ("steps", "hits", "misses", "loads", "evictions", "bytes_loaded")]


class moe_layer_desc(C.Structure):
    _fields_ = [("sh", moe_ffn_shape), ("shared_sh", moe_ffn_shape),
                ("E", C.c_int32), ("k", C.c_int32),
                ("w_router_dev", C.c_void_p), ("logit_bias_dev", C.c_void_p),
                ("pool", C.c_void_p), ("shared_blob_dev", C.c_void_p),
                ("usage_dev", C.c_void_p)]


_P = C.c_void_p
_I = C.c_int32
_S = C.c_size_t
_SIGS = {
    "moe_status_string": (C.c_char_p, [C.c_int]),
    "moe_last_hip_error": (C.c_char_p, []),
    "moe_version": (C.c_char_p, []),
    "moe_blob_bytes": (_S, [_P]),
    "moe_blob_stride": (_S, [_P]),
    "moe_pack_expert": (C.c_int, [_P, _P, _P, _P, _P]),
    "moe_unpack_expert": (C.c_int, [_P, _P, _P, _P, _P]),
    "moe_pack_expert_f32": (C.c_int, [_P, _P, _P]),
    "moe_unpack_expert_f32": (C.c_int, [_P, _P, _P]),
    "moe_pack_expert_int4": (C.c_int, [_P, _P, _P, _P, _P]),
    "moe_unpack_expert_int4": (C.c_int, [_P, _P, _P, _P, _P]),
    "moe_lfu_create": (C.c_int, [_I, _I, _P]),
    "moe_lfu_destroy": (C.c_int, [_P]),
    "moe_lfu_plan": (C.c_int, [_P, _P, _I, _P, _P, _P, _P]),
    "moe_lfu_get_stats": (C.c_int, [_P, _P]),
    "moe_pool_create": (C.c_int, [_I, _I, _P, _P]),
    "moe_pool_destroy": (C.c_int, [_P]),
    "moe_pool_slab": (_P, [_P]),
    "moe_pool_stride": (_S, [_P]),
    "moe_pool_slot_table": (_P, [_P]),
    "moe_pool_usage": (_P, [_P]),
    "moe_pool_num_experts": (_I, [_P]),
    "moe_pool_num_slots": (_I, [_P]),
    "moe_pool_load": (C.c_int, [_P, _I, _I, _P, _P]),
    "moe_pool_load_device": (C.c_int, [_P, _I, _I, _P, _P]),
    "moe_pool_plan": (C.c_int, [_P, _P, _I, _P, _P, _P, _P]),
    "moe_pool_refill": (C.c_int, [_P, _P, _I, _P, _S, _P]),
    "moe_pool_set_slot_table": (C.c_int, [_P, _P, _P]),
    "moe_pool_get_stats": (C.c_int, [_P, _P]),
    "moe_pool_check_error": (C.c_int, [_P, _P, _P]),
    "moe_pool_reset_usage": (C.c_int, [_P, _P]),
    "moe_pool_read_state": (C.c_int, [_P, _P, _P, _P]),
    "moe_router_sum_depth": (_I, [_I, _I, _I]),
    "moe_router_workspace_bytes": (_S, [_I, _I, _I]),
    "moe_router_topk": (C.c_int, [_P, _I, _I, _P, _P, _I, _I, _P, _P, _P, _P, _P, _S, _P]),
    "moe_router_topk_logits": (C.c_int, [_P, _I, _I, _P, _P, _I, _I, _P, _P, _P, _P, _P, _P, _S, _P]),
    "moe_bucket_workspace_bytes": (_S, [_I, _I, _I]),
    "moe_bucket_tokens": (C.c_int, [_P, _I, _I, _I, _P, _P, _P, _P, _S, _P]),
    "moe_ffn_workspace_bytes": (_S, [_P, _P, _I, _I, _I, _I]),
    "moe_expert_ffn": (C.c_int, [_P, _P, _P, _P, _P, _I, _I, _P, _P, _P, _P, _P,
                                 _P, _P, _P, _I, _P, _S, _P]),
    "moe_expert_ffn_int4": (C.c_int, [_P, _P, _P, _P, _P, _I, _I, _P, _P, _P, _P, _P,
                                      _P, _P, _P, _I, _P, _S, _P]),
    "moe_combine": (C.c_int, [_P, _P, _P, _P, _I, _I, _I, _P, _P]),
    "moe_layer_workspace_bytes": (_S, [_P, _I, _I]),
    "moe_layer_forward": (C.c_int, [_P, _P, _I, _P, _P, _P, _P, _I, _P, _S, _P]),
    "moe_layer_forward_noalloc": (C.c_int, [_P, _P, _I, _P, _P, _P, _P, _I, _P]),
    "moe_layer_forward_streamed": (C.c_int, [_P, _P, _S, _P, _I, _P, _P, _P, _P, _P, _S, _P, _P, _P]),
    "moe_layer_forward_offload": (C.c_int, [_P, _P, _S, _P, _I, _P, _P, _P, _P, _P, _S, _P, _P]),
    "moe_probe_stream_read": (C.c_int, [_P, _S, _P, _I, _P]),
    "moe_probe_mfma_f16": (C.c_int, [_I, _P, _I, _P]),
    "moe_probe_mfma_f16_flops": (C.c_double, [_I, _I]),
    "moe_chain_workspace_bytes": (_S, [_P, _I, _I, _I]),
    "moe_chain_forward": (C.c_int, [_P, _I, C.c_float, _P, _I, _P, _P, _P, _P, _I, _P, _S, _P]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGS)


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = _lib.moe_status_string(status).decode()
        if status == MOE_ERR_HIP:
            msg += f" ({_lib.moe_last_hip_error().decode()})"
        super().__init__(f"{where}: {msg} [{status}]")
        self.status = status


def _check(st: int, where: str):
    if st != MOE_OK:
        raise MoeError(st, where)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def version() -> str:
    return _lib.moe_version().decode()


def shape(d: int, I: int, bits: int = 4) -> moe_ffn_shape:
    return moe_ffn_shape(d, I, 64, bits)


# -------------------------------------------------------------- blob layout
def moe_blob_bytes(d: int, I: int, bits: int = 4) -> int:
    return int(_lib.moe_blob_bytes(C.byref(shape(d, I, bits))))


def moe_blob_stride(d: int, I: int, bits: int = 4) -> int:
    return int(_lib.moe_blob_stride(C.byref(shape(d, I, bits))))


_MATS = ("gate", "up", "down")


def moe_pack_expert(raw, d: int, I: int, bits: int = 4) -> np.ndarray:
    """Blob bytes (uint8[stride]) of one expert (4- or 8-bit codes, or bits=32:
    raw[m]["weights"] fp32 [out][in])."""
    if bits == 32:
        keep = [np.ascontiguousarray(raw[name]["weights"], dtype=np.float32) for name in _MATS]
        wp = (C.c_void_p * 3)(*[k.ctypes.data for k in keep])
        out = np.empty(moe_blob_stride(d, I, 32), dtype=np.uint8)
        _check(_lib.moe_pack_expert_f32(C.byref(shape(d, I, 32)), wp, out.ctypes.data), "moe_pack_expert_f32")
        return out
    return _pack(_lib.moe_pack_expert, raw, d, I, bits)


def moe_unpack_expert(blob: np.ndarray, d: int, I: int, bits: int = 4):
    if bits == 32:
        dims = {"gate": (I, d), "up": (I, d), "down": (d, I)}
        raw = {name: {"weights": np.empty(dims[name], np.float32)} for name in _MATS}
        wp = (C.c_void_p * 3)(*[raw[name]["weights"].ctypes.data for name in _MATS])
        blob = np.ascontiguousarray(blob, dtype=np.uint8)
        _check(_lib.moe_unpack_expert_f32(C.byref(shape(d, I, 32)), blob.ctypes.data, wp),
               "moe_unpack_expert_f32")
        return raw
    return _unpack(_lib.moe_unpack_expert, blob, d, I, bits)


def moe_pack_expert_int4(raw, d: int, I: int) -> np.ndarray:
    """Blob bytes (uint8[stride]) of one 4-bit expert from raw MLX-orientation arrays."""
    return _pack(_lib.moe_pack_expert_int4, raw, d, I, 4)


def moe_unpack_expert_int4(blob: np.ndarray, d: int, I: int):
    return _unpack(_lib.moe_unpack_expert_int4, blob, d, I, 4)


def _pack(fn, raw, d: int, I: int, bits: int) -> np.ndarray:
    keep = []
    cp, sp, bp = (C.c_void_p * 3)(), (C.c_void_p * 3)(), (C.c_void_p * 3)()
    for m, name in enumerate(_MATS):
        c = np.ascontiguousarray(raw[name]["codes"], dtype=np.uint8)
        s = np.ascontiguousarray(np.asarray(raw[name]["scales"], np.float16)).view(np.uint16)
        b = np.ascontiguousarray(np.asarray(raw[name]["biases"], np.float16)).view(np.uint16)
        keep += [c, s, b]
        cp[m], sp[m], bp[m] = c.ctypes.data, s.ctypes.data, b.ctypes.data
    out = np.empty(moe_blob_stride(d, I, bits), dtype=np.uint8)
    _check(fn(C.byref(shape(d, I, bits)), cp, sp, bp, out.ctypes.data), fn.__name__)
    return out


def _unpack(fn, blob: np.ndarray, d: int, I: int, bits: int):
    dims = {"gate": (I, d), "up": (I, d), "down": (d, I)}
    raw = {}
    cp, sp, bp = (C.c_void_p * 3)(), (C.c_void_p * 3)(), (C.c_void_p * 3)()
    for m, name in enumerate(_MATS):
        o, i = dims[name]
        raw[name] = {"codes": np.empty((o, i), np.uint8),
                     "scales": np.empty((o, i // 64), np.float16),
                     "biases": np.empty((o, i // 64), np.float16)}
        cp[m] = raw[name]["codes"].ctypes.data
        sp[m] = raw[name]["scales"].ctypes.data
        bp[m] = raw[name]["biases"].ctypes.data
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    _check(fn(C.byref(shape(d, I, bits)), blob.ctypes.data, cp, sp, bp), fn.__name__)
    return raw


# --------------------------------------------------------------------- pool
def _plan(fn, handle, selected):
    sel = np.ascontiguousarray(np.asarray(selected, dtype=np.int32))
    n = sel.size
    le = np.empty(max(n, 1), np.int32)
    ls = np.empty(max(n, 1), np.int32)
    lv = np.empty(max(n, 1), np.int32)
    nl = C.c_int32()
    _check(fn(handle, sel.ctypes.data, n, le.ctypes.data, ls.ctypes.data, lv.ctypes.data, C.byref(nl)),
           fn.__name__)
    return [(int(le[q]), int(ls[q]), int(lv[q])) for q in range(nl.value)]


class Lfu:
    """Host-only LFU + recency slot policy (no device needed)."""

    def __init__(self, E: int, n_slots: int):
        h = C.c_void_p()
        _check(_lib.moe_lfu_create(E, n_slots, C.byref(h)), "moe_lfu_create")
        self.handle = h

    def close(self):
        if self.handle:
            _lib.moe_lfu_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def plan(self, selected):
        return _plan(_lib.moe_lfu_plan, self.handle, selected)

    def stats(self) -> dict:
        st = moe_pool_stats()
        _check(_lib.moe_lfu_get_stats(self.handle, C.byref(st)), "moe_lfu_get_stats")
        return {n: int(getattr(st, n)) for n, _ in moe_pool_stats._fields_}


class Pool:
    """A bounded HBM slot pool of expert blobs (owns its device memory)."""

    def __init__(self, E: int, n_slots: int, d: int, I: int, bits: int = 4):
        self.E, self.n_slots, self.d, self.I, self.bits = E, n_slots, d, I, bits
        h = C.c_void_p()
        _check(_lib.moe_pool_create(E, n_slots, C.byref(shape(d, I, bits)), C.byref(h)), "moe_pool_create")
        self.handle = h
        self.stride = int(_lib.moe_pool_stride(h))

    def close(self):
        if self.handle:
            _lib.moe_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def slab_ptr(self) -> int:
        return int(_lib.moe_pool_slab(self.handle))

    @property
    def slot_table_ptr(self) -> int:
        return int(_lib.moe_pool_slot_table(self.handle))

    @property
    def usage_ptr(self) -> int:
        return int(_lib.moe_pool_usage(self.handle))

    def load(self, expert: int, slot: int, blob, stream=None):
        """blob: a torch CUDA uint8 tensor (device copy) or a numpy/pinned host array."""
        if hasattr(blob, "is_cuda") and blob.is_cuda:
            st = _lib.moe_pool_load_device(self.handle, expert, slot, blob.data_ptr(), _stream(stream))
        else:
            ptr = blob.data_ptr() if hasattr(blob, "data_ptr") else blob.ctypes.data
            st = _lib.moe_pool_load(self.handle, expert, slot, ptr, _stream(stream))
        _check(st, "moe_pool_load")

    def plan(self, selected: Sequence[int]):
        return _plan(_lib.moe_pool_plan, self.handle, selected)

    def refill(self, selected, host_blobs, host_stride: int, stream=None):
        sel = np.ascontiguousarray(np.asarray(selected, dtype=np.int32))
        _check(_lib.moe_pool_refill(self.handle, sel.ctypes.data, sel.size, host_blobs.data_ptr(),
                                    host_stride, _stream(stream)), "moe_pool_refill")

    def set_slot_table(self, table, stream=None):
        t = np.ascontiguousarray(np.asarray(table, dtype=np.int32))
        _check(_lib.moe_pool_set_slot_table(self.handle, t.ctypes.data, _stream(stream)),
               "moe_pool_set_slot_table")

    def stats(self) -> dict:
        st = moe_pool_stats()
        _check(_lib.moe_pool_get_stats(self.handle, C.byref(st)), "moe_pool_get_stats")
        return {n: int(getattr(st, n)) for n, _ in moe_pool_stats._fields_}

    def check_error(self, stream=None) -> int:
        e = C.c_int32()
        _check(_lib.moe_pool_check_error(self.handle, _stream(stream), C.byref(e)), "moe_pool_check_error")
        return e.value

    def reset_usage(self, stream=None):
        _check(_lib.moe_pool_reset_usage(self.handle, _stream(stream)), "moe_pool_reset_usage")

    def read_state(self, stream=None):
        """(slot_table int32[E], usage uint32[E]) copied to host."""
        table = np.empty(self.E, np.int32)
        usage = np.empty(self.E, np.uint32)
        _check(_lib.moe_pool_read_state(self.handle, table.ctypes.data, usage.ctypes.data,
                                        _stream(stream)), "moe_pool_read_state")
        return table, usage


def _ws(nbytes: int):
    import torch
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device="cuda")


# ------------------------------------------------------------------- router
def moe_router_sum_depth(T: int, d: int, E: int) -> int:
    return int(_lib.moe_router_sum_depth(T, d, E))


def moe_router_workspace_bytes(T: int, d: int, E: int) -> int:
    return int(_lib.moe_router_workspace_bytes(T, d, E))


def moe_router_topk(x, w_router, logit_bias, k: int, usage_ptr: Optional[int] = None,
                    workspace=None, out=None, stream=None):
    """x: bf16 [T, d] CUDA; w_router fp32 [E+1, d]; logit_bias fp32 [E] or None.
    Returns (topk_idx int32 [T,k], topk_w fp32 [T,k], shared_gate fp32 [T])."""
    import torch
    T, d = x.shape
    E = w_router.shape[0] - 1
    if out is None:
        out = (torch.empty((T, k), dtype=torch.int32, device=x.device),
               torch.empty((T, k), dtype=torch.float32, device=x.device),
               torch.empty((T,), dtype=torch.float32, device=x.device))
    idx, w, s = out
    if workspace is None:
        workspace = _ws(moe_router_workspace_bytes(T, d, E))
    st = _lib.moe_router_topk(_ptr(x), T, d, _ptr(w_router), _ptr(logit_bias), E, k, _ptr(idx), _ptr(w),
                              _ptr(s), usage_ptr, _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "moe_router_topk")
    return idx, w, s


def moe_router_topk_logits(x, w_router, logit_bias, k: int, usage_ptr: Optional[int] = None,
                           workspace=None, stream=None):
    """moe_router_topk plus the fp32 logits the selection read (before the
    bias).  Returns (topk_idx [T,k], topk_w [T,k], shared_gate [T], logits [T,E+1])."""
    import torch
    T, d = x.shape
    E = w_router.shape[0] - 1
    idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    s = torch.empty((T,), dtype=torch.float32, device=x.device)
    logits = torch.empty((T, E + 1), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = _ws(moe_router_workspace_bytes(T, d, E))
    st = _lib.moe_router_topk_logits(_ptr(x), T, d, _ptr(w_router), _ptr(logit_bias), E, k, _ptr(idx),
                                     _ptr(w), _ptr(s), usage_ptr, _ptr(logits), _ptr(workspace),
                                     workspace.numel(), _stream(stream))
    _check(st, "moe_router_topk_logits")
    return idx, w, s, logits


# ---------------------------------------------------------------- bucketing
def moe_bucket_tokens(topk_idx, E: int, workspace=None, stream=None):
    import torch
    T, k = topk_idx.shape
    counts = torch.empty(E, dtype=torch.int32, device=topk_idx.device)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=topk_idx.device)
    pair_ids = torch.empty(max(T * k, 1), dtype=torch.int32, device=topk_idx.device)
    if workspace is None:
        workspace = _ws(_lib.moe_bucket_workspace_bytes(T, k, E))
    st = _lib.moe_bucket_tokens(_ptr(topk_idx), T, k, E, _ptr(counts), _ptr(offsets), _ptr(pair_ids),
                                _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "moe_bucket_tokens")
    return counts, offsets, pair_ids[:T * k]


# --------------------------------------------------------------- expert FFN
def moe_ffn_workspace_bytes(d, I, Ish, T, k, E, path, bits: int = 4) -> int:
    return int(_lib.moe_ffn_workspace_bytes(C.byref(shape(d, I, bits)), C.byref(shape(d, Ish, bits)),
                                            T, k, E, path))


def moe_expert_ffn_int4(pool: Pool, shared_blob, Ish: int, x, topk_idx, topk_w, shared_gate,
                        path: int = MOE_PATH_DECODE, offsets=None, pair_ids=None,
                        workspace=None, out=None, stream=None):
    """moe_expert_ffn through the 4-bit-only entry point."""
    return _expert_ffn(_lib.moe_expert_ffn_int4, pool, shared_blob, Ish, x, topk_idx, topk_w, shared_gate,
                       path, offsets, pair_ids, workspace, out, stream, 4)


def moe_expert_ffn(pool: Pool, shared_blob, Ish: int, x, topk_idx, topk_w, shared_gate,
                   path: int = MOE_PATH_DECODE, offsets=None, pair_ids=None,
                   workspace=None, out=None, stream=None, shared_bits: Optional[int] = None):
    """DECODE: returns y [T, d] (out: y).  BATCHED/PREFILL: returns (partial [T*k, d], shared_out [T, d])
    (out: that pair).
    The routed experts' code width is the pool's; the shared expert's is shared_bits (default: the same)."""
    return _expert_ffn(_lib.moe_expert_ffn, pool, shared_blob, Ish, x, topk_idx, topk_w, shared_gate,
                       path, offsets, pair_ids, workspace, out, stream,
                       pool.bits if shared_bits is None else shared_bits)


def _expert_ffn(fn, pool, shared_blob, Ish, x, topk_idx, topk_w, shared_gate, path, offsets, pair_ids,
                workspace, out, stream, shared_bits):
    import torch
    T, d = x.shape
    k = topk_idx.shape[1]
    if workspace is None:
        workspace = _ws(moe_ffn_workspace_bytes(d, pool.I, Ish, T, k, pool.E, path, pool.bits))
    y = partial = shared_out = None
    if path == MOE_PATH_DECODE:
        y = torch.empty((T, d), dtype=torch.float32, device=x.device) if out is None else out
    elif out is not None:
        partial, shared_out = out
    else:
        partial = torch.empty((T * k, d), dtype=torch.float32, device=x.device)
        shared_out = torch.empty((T, d), dtype=torch.float32, device=x.device)
    st = fn(pool.handle, C.byref(shape(d, pool.I, pool.bits)), _ptr(shared_blob),
            C.byref(shape(d, Ish, shared_bits)), _ptr(x), T, k, _ptr(topk_idx), _ptr(topk_w),
            _ptr(shared_gate), _ptr(offsets), _ptr(pair_ids), _ptr(y), _ptr(partial),
            _ptr(shared_out), path, _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, fn.__name__)
    return y if path == MOE_PATH_DECODE else (partial, shared_out)


def moe_combine(partial, shared_out, topk_w, shared_gate, stream=None):
    import torch
    T, k = topk_w.shape
    d = partial.shape[1]
    y = torch.empty((T, d), dtype=torch.float32, device=partial.device)
    st = _lib.moe_combine(_ptr(partial), _ptr(shared_out), _ptr(topk_w), _ptr(shared_gate), T, k, d,
                          _ptr(y), _stream(stream))
    _check(st, "moe_combine")
    return y


# -------------------------------------------------------------- whole layer
class Layer:
    """Descriptor of one MoE layer (router, pool of routed experts, shared expert)."""

    def __init__(self, w_router, logit_bias, pool: Pool, shared_blob, Ish: int, k: int,
                 usage: bool = True, shared_bits: Optional[int] = None):
        self.w_router, self.logit_bias, self.pool, self.shared_blob = w_router, logit_bias, pool, shared_blob
        self.k, self.Ish = k, Ish
        self.shared_bits = pool.bits if shared_bits is None else shared_bits
        self.desc = moe_layer_desc(shape(pool.d, pool.I, pool.bits), shape(pool.d, Ish, self.shared_bits),
                                   pool.E, k,
                                   _ptr(w_router), _ptr(logit_bias), pool.handle.value,
                                   _ptr(shared_blob), pool.usage_ptr if usage else None)

    def workspace_bytes(self, T: int, path: int = MOE_PATH_AUTO) -> int:
        return int(_lib.moe_layer_workspace_bytes(C.byref(self.desc), T, path))


def moe_layer_forward(layer: Layer, x, path: int = MOE_PATH_AUTO, workspace=None, out=None,
                      stream=None):
    """Returns (y fp32 [T,d], topk_idx [T,k], topk_w [T,k], shared_gate [T])."""
    import torch
    T, d = x.shape
    k = layer.k
    if out is None:
        out = (torch.empty((T, d), dtype=torch.float32, device=x.device),
               torch.empty((T, k), dtype=torch.int32, device=x.device),
               torch.empty((T, k), dtype=torch.float32, device=x.device),
               torch.empty((T,), dtype=torch.float32, device=x.device))
    y, idx, w, s = out
    if workspace is None:
        workspace = _ws(layer.workspace_bytes(T, path))
    st = _lib.moe_layer_forward(C.byref(layer.desc), _ptr(x), T, _ptr(y), _ptr(idx), _ptr(w), _ptr(s),
                                path, _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "moe_layer_forward")
    return y, idx, w, s


NOALLOC_SCRATCH_BYTES = 32 << 20


def moe_layer_forward_noalloc(layer: Layer, x, path: int = MOE_PATH_AUTO, out=None, stream=None):
    """moe_layer_forward with the library's per-GPU scratch as the workspace
    (the C call allocates nothing).  out: (y, topk_idx, topk_w, shared_gate),
    allocated here when None."""
    import torch
    T, d = x.shape
    k = layer.k
    if out is None:
        out = (torch.empty((T, d), dtype=torch.float32, device=x.device),
               torch.empty((T, k), dtype=torch.int32, device=x.device),
               torch.empty((T, k), dtype=torch.float32, device=x.device),
               torch.empty((T,), dtype=torch.float32, device=x.device))
    y, idx, w, s = out
    st = _lib.moe_layer_forward_noalloc(C.byref(layer.desc), _ptr(x), T, _ptr(y), _ptr(idx), _ptr(w), _ptr(s),
                                        path, _stream(stream))
    _check(st, "moe_layer_forward_noalloc")
    return y, idx, w, s


def moe_layer_forward_streamed(layer: Layer, x, host_blobs, copy_stream=None, workspace=None, out=None,
                               stream=None):
    """One decode step on a partly resident pool, the misses copied in from
    host_blobs (pinned uint8 [E, stride]) on copy_stream while the resident
    experts compute.  Returns (y, topk_idx, topk_w, shared_gate, n_loads);
    blocks the calling thread until the step's selections reach the host."""
    import torch
    T, d = x.shape
    k = layer.k
    if (host_blobs.dtype != torch.uint8 or host_blobs.dim() != 2 or host_blobs.is_cuda
            or not host_blobs.is_pinned() or not host_blobs.is_contiguous()):
        raise ValueError("host_blobs must be a contiguous pinned uint8 host tensor [E, stride]")
    if out is None:
        out = (torch.empty((T, d), dtype=torch.float32, device=x.device),
               torch.empty((T, k), dtype=torch.int32, device=x.device),
               torch.empty((T, k), dtype=torch.float32, device=x.device),
               torch.empty((T,), dtype=torch.float32, device=x.device))
    y, idx, w, s = out
    if workspace is None:
        workspace = _ws(layer.workspace_bytes(T, MOE_PATH_DECODE))
    nl = C.c_int32(0)
    st = _lib.moe_layer_forward_streamed(C.byref(layer.desc), host_blobs.data_ptr(), host_blobs.stride(0),
                                         _ptr(x), T, _ptr(y), _ptr(idx), _ptr(w), _ptr(s), _ptr(workspace),
                                         workspace.numel(), _stream(stream),
                                         _stream(copy_stream) if copy_stream is not None else _stream(stream),
                                         C.byref(nl))
    _check(st, "moe_layer_forward_streamed")
    return y, idx, w, s, int(nl.value)


def moe_layer_forward_offload(layer: Layer, x, host_blobs, workspace=None, out=None, n_loads=None, stream=None):
    """One decode step on a partly resident pool with the refill planned and
    copied by the GPU (router -> LFU + recency plan -> copy of the missing
    blobs from host_blobs, pinned uint8 [E, stride], over PCIe -> experts),
    all on `stream` and without waiting on the host.  n_loads: optional
    device int32 tensor [1] that receives the blobs copied.  Returns
    (y, topk_idx, topk_w, shared_gate)."""
    import torch
    T, d = x.shape
    k = layer.k
    if (host_blobs.dtype != torch.uint8 or host_blobs.dim() != 2 or host_blobs.is_cuda
            or not host_blobs.is_pinned() or not host_blobs.is_contiguous()):
        raise ValueError("host_blobs must be a contiguous pinned uint8 host tensor [E, stride]")
    if n_loads is not None and (n_loads.dtype != torch.int32 or not n_loads.is_cuda or n_loads.numel() < 1):
        raise ValueError("n_loads must be a device int32 tensor")
    if out is None:
        out = (torch.empty((T, d), dtype=torch.float32, device=x.device),
               torch.empty((T, k), dtype=torch.int32, device=x.device),
               torch.empty((T, k), dtype=torch.float32, device=x.device),
               torch.empty((T,), dtype=torch.float32, device=x.device))
    y, idx, w, s = out
    if workspace is None:
        workspace = _ws(layer.workspace_bytes(T, MOE_PATH_DECODE))
    st = _lib.moe_layer_forward_offload(C.byref(layer.desc), host_blobs.data_ptr(), host_blobs.stride(0),
                                        _ptr(x), T, _ptr(y), _ptr(idx), _ptr(w), _ptr(s), _ptr(workspace),
                                        workspace.numel(), _ptr(n_loads) if n_loads is not None else None,
                                        _stream(stream))
    _check(st, "moe_layer_forward_offload")
    return y, idx, w, s


# -------------------------------------------------------------- layer chain
class Chain:
    """L layers applied one after the other (pre-norm residual blocks)."""

    def __init__(self, layers: Sequence[Layer], eps: float = 1e-6):
        self.layers = list(layers)
        self.eps = eps
        self.descs = (moe_layer_desc * len(self.layers))(*[L.desc for L in self.layers])
        self.k = self.layers[0].k

    def workspace_bytes(self, T: int, path: int = MOE_PATH_AUTO) -> int:
        return int(_lib.moe_chain_workspace_bytes(self.descs, len(self.layers), T, path))


def moe_chain_forward(chain: Chain, x, path: int = MOE_PATH_AUTO, trace: bool = False, workspace=None,
                      out=None, stream=None, trace_u: bool = True):
    """Returns x_L (bf16 [T, d]); with trace=True also (trace_x [L+1, T, d],
    trace_u [L, T, d] (None if trace_u=False), topk_idx [L, T, k])."""
    import torch
    T, d = x.shape
    L = len(chain.layers)
    x_out = torch.empty_like(x) if out is None else out
    tx = tu = ti = None
    if trace:
        tx = torch.empty((L + 1, T, d), dtype=x.dtype, device=x.device)
        tu = torch.empty((L, T, d), dtype=x.dtype, device=x.device) if trace_u else None
        ti = torch.empty((L, T, chain.k), dtype=torch.int32, device=x.device)
    if workspace is None:
        workspace = _ws(chain.workspace_bytes(T, path))
    st = _lib.moe_chain_forward(chain.descs, L, C.c_float(chain.eps), _ptr(x), T, _ptr(x_out), _ptr(tx), _ptr(tu),
                                _ptr(ti), path, _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "moe_chain_forward")
    return (x_out, tx, tu, ti) if trace else x_out


# --------------------------------------------------------- measurement probes
def moe_probe_stream_read(buf, sink, blocks: int = 2048, stream=None):
    """One launch reading every byte of the CUDA tensor buf (16-byte multiple)."""
    _check(_lib.moe_probe_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(), blocks,
                                      _stream(stream)), "moe_probe_stream_read")


def moe_probe_mfma_f16(iters: int, sink, blocks: int, stream=None) -> float:
    """A loop of dense fp16 MFMAs; returns the flops of the launch."""
    _check(_lib.moe_probe_mfma_f16(iters, sink.data_ptr(), blocks, _stream(stream)), "moe_probe_mfma_f16")
    return float(_lib.moe_probe_mfma_f16_flops(iters, blocks))
