"""Oracle: token -> expert bucketing.

The pages say nothing about batching; the batched-decode and prefill
workloads need (token, rank) pairs grouped by expert.  Reading: a stable
counting sort of the pair indices i = t*k + r by expert id — counts[e],
exclusive prefix offsets[0..E] (offsets[E] = T*k), and pair_ids listing each
bucket's pairs in ascending i.  That is exactly numpy's stable argsort by key.
"""
from __future__ import annotations

import numpy as np


def bucket(topk_idx: np.ndarray, E: int):
    keys = np.asarray(topk_idx, dtype=np.int64).ravel()
    counts = np.bincount(keys, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    pair_ids = np.argsort(keys, kind="stable").astype(np.int32)
    return counts, offsets, pair_ids
