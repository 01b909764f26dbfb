"""Oracle: int4 / int8 affine group dequantisation and the fixed-stride blob layout.

Dequantisation (MLX affine int4/int8 group quantisation, named on the
Swiftlet pages in the relationship-to-TurboFieldfare section): for an
[out, in] matrix with group size 64 along the input dimension,

    W[o, j] = scale[o, j // 64] * q[o, j] + bias[o, j // 64],
    q in 0..15 (4-bit) or 0..255 (8-bit).

Blob layout (the pages fix only that each routed expert is repacked as one
fixed-stride blob so that fetching it is one read — "How it works"; the byte
layout below is this library's reading, chosen for wide coalesced loads):

  for m in (gate [I x d], up [I x d], down [d x I]):
      codes_m : [in/32][out][16] bytes.  The 16 bytes of (chunk c, row o) hold
                q[o, 32c .. 32c+31], two per byte, element 32c+2b in the low
                nibble of byte b and 32c+2b+1 in the high nibble (the same
                bytes as four little-endian MLX uint32 words, element j of a
                word in bits 4j..4j+3).
      sb_m    : [in/64][out][2] fp16: (scale, bias) of group g of row o.
  sections in the order gate codes, gate sb, up codes, up sb, down codes,
  down sb; blob bytes = 27/16 * d * I; stride = bytes rounded up to 4096,
  zero padded.

8-bit blobs (same sections and order, same sb): codes_m is [in/16][out][16]
bytes, one code per byte; inside every 8 consecutive inputs the bytes hold
inputs (0, 1, 4, 5, 2, 3, 6, 7) of the block, so byte pairs (0, 2) and
(1, 3) of each 32-bit word are the input pairs (i, i+4) the 4-bit layout
forms from nibbles i and i+4.  blob bytes = 51/16 * d * I.

f32 experts (unquantised; the pages validate every layer in f32 as well as
int4 form, correctness section): a raw matrix is {"weights": fp32 [out, in]}
and the blob holds gate, up, down as row-major fp32 [out][in] one after the
other (no scale/bias sections); blob bytes = 12 * d * I.
"""
from __future__ import annotations

import numpy as np

GROUP = 64
CHUNK = 32                   # inputs per 16-byte piece, 4-bit
CHUNK8 = 16                  # inputs per 16-byte piece, 8-bit
MATS = ("gate", "up", "down")
BITS = (4, 8, 32)            # 32: unquantised fp32 weights
PERM8 = np.array([0, 1, 4, 5, 2, 3, 6, 7])   # byte j of an 8-input block holds input PERM8[j]


def dequant(m) -> np.ndarray:
    """fp64 [out, in] from a raw matrix dict {codes, scales, biases} (or the
    weights themselves for an f32 matrix {weights})."""
    if "weights" in m:
        return np.asarray(m["weights"], dtype=np.float32).astype(np.float64)
    q = np.asarray(m["codes"], dtype=np.float64)
    s = np.repeat(np.asarray(m["scales"], dtype=np.float64), GROUP, axis=1)
    b = np.repeat(np.asarray(m["biases"], dtype=np.float64), GROUP, axis=1)
    return s * q + b


def mat_dims(d: int, I: int):
    return {"gate": (I, d), "up": (I, d), "down": (d, I)}


def section_bytes(out: int, inp: int, bits: int = 4):
    """(codes or weights bytes, scale/bias bytes) of one matrix."""
    assert bits in BITS
    if bits == 32:
        return out * inp * 4, 0
    return out * inp * bits // 8, (inp // GROUP) * out * 4


def blob_bytes(d: int, I: int, bits: int = 4) -> int:
    tot = 0
    for o, i in mat_dims(d, I).values():
        c, s = section_bytes(o, i, bits)
        tot += c + s
    return tot


def blob_stride(d: int, I: int, bits: int = 4) -> int:
    b = blob_bytes(d, I, bits)
    return (b + 4095) // 4096 * 4096


def _pack_codes(codes: np.ndarray) -> np.ndarray:
    out, inp = codes.shape
    c = np.asarray(codes, dtype=np.uint8)
    byte = (c[:, 0::2] & 0xF) | ((c[:, 1::2] & 0xF) << 4)       # [out][in/2]
    return byte.reshape(out, inp // CHUNK, 16).transpose(1, 0, 2).ravel()


def _unpack_codes(buf: np.ndarray, out: int, inp: int) -> np.ndarray:
    byte = buf.reshape(inp // CHUNK, out, 16).transpose(1, 0, 2).reshape(out, inp // 2)
    q = np.empty((out, inp), dtype=np.uint8)
    q[:, 0::2] = byte & 0xF
    q[:, 1::2] = byte >> 4
    return q


def _pack_codes8(codes: np.ndarray) -> np.ndarray:
    out, inp = codes.shape
    c = np.asarray(codes, dtype=np.uint8).reshape(out, inp // 8, 8)[:, :, PERM8]
    return c.reshape(out, inp // CHUNK8, 16).transpose(1, 0, 2).ravel()


def _unpack_codes8(buf: np.ndarray, out: int, inp: int) -> np.ndarray:
    b = buf.reshape(inp // CHUNK8, out, 16).transpose(1, 0, 2).reshape(out, inp // 8, 8)
    q = np.empty_like(b)
    q[:, :, PERM8] = b
    return q.reshape(out, inp)


def _pack_sb(scales: np.ndarray, biases: np.ndarray) -> np.ndarray:
    sb = np.stack([np.asarray(scales, np.float16), np.asarray(biases, np.float16)], axis=-1)
    return np.ascontiguousarray(sb.transpose(1, 0, 2)).view(np.uint8).ravel()


def _unpack_sb(buf: np.ndarray, out: int, inp: int):
    sb = np.ascontiguousarray(buf).view(np.float16).reshape(inp // GROUP, out, 2)
    return (np.ascontiguousarray(sb[:, :, 0].T), np.ascontiguousarray(sb[:, :, 1].T))


def pack_expert(raw, d: int, I: int, bits: int = 4) -> np.ndarray:
    """Blob bytes (length = stride) of one expert from its raw matrices."""
    parts = []
    for name in MATS:
        m = raw[name]
        if bits == 32:
            parts.append(np.ascontiguousarray(m["weights"], dtype=np.float32).view(np.uint8).ravel())
            continue
        assert int(np.max(m["codes"])) < (1 << bits)
        parts.append(_pack_codes(m["codes"]) if bits == 4 else _pack_codes8(m["codes"]))
        parts.append(_pack_sb(m["scales"], m["biases"]))
    body = np.concatenate(parts)
    assert body.size == blob_bytes(d, I, bits)
    blob = np.zeros(blob_stride(d, I, bits), dtype=np.uint8)
    blob[:body.size] = body
    return blob


def unpack_expert(blob: np.ndarray, d: int, I: int, bits: int = 4):
    blob = np.asarray(blob, dtype=np.uint8)
    off = 0
    raw = {}
    for name, (o, i) in mat_dims(d, I).items():
        cb, sbb = section_bytes(o, i, bits)
        if bits == 32:
            w = np.ascontiguousarray(blob[off:off + cb]).view(np.float32).reshape(o, i).copy()
            off += cb
            raw[name] = {"weights": w}
            continue
        unpack = _unpack_codes if bits == 4 else _unpack_codes8
        codes = unpack(blob[off:off + cb], o, i)
        off += cb
        sc, bi = _unpack_sb(blob[off:off + sbb], o, i)
        off += sbb
        raw[name] = {"codes": codes, "scales": sc, "biases": bi}
    return raw
