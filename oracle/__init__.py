"""CPU oracle for the routed-expert MoE layer — TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct numpy float64 code.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the library in ``sparse_moe_decode_router_amd`` never does, and the
oracle imports nothing from that library (the two share only the seeded input
generators in ``moe_synth``).

What it computes, and on what authority (Swiftlet pages):
  * routing of every token to k of E experts (10 of 512 / 8 of 256 —
    "How it works"), router and shared expert resident;
  * routed experts as 4-bit (or 8-bit) MLX affine group-quantised weights
    (relationship-to-TurboFieldfare section: MLX affine int4/int8 group
    quantisation with byte-addressed kernels and 64-bit offsets);
  * each expert repacked as one fixed-stride blob so one fetch is one read,
    kept in a bounded pool with LFU + recency eviction ("How it works");
  * placement never changes the answer (correctness section).
The router arithmetic (softmax, top-k with ties to the lower index,
renormalisation over the chosen k), the SwiGLU expert, the sigmoid-gated
shared expert, group size 64 and the blob layout are readings the pages leave
open; each function states the reading it follows.

Modules:
  quant   — dequantisation and the blob layout (pack / unpack)
  layer   — router, expert FFN, whole layer
  bucket  — token -> expert bucketing (counting sort)
  lfu     — LFU + recency slot-pool simulation

Parity status of every function is pinned by ``tests/test_oracle_pins.py``;
none is "parity unpinned".
"""
from . import quant, layer, bucket, lfu  # noqa: F401
