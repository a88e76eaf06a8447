"""Comparison helpers between the HIP path and the CPU oracle.

Margin protocol: a Ward block or a selection must match bit-exactly; a
mismatch is excused only when the oracle's own margin at the decision that
differs is below 1e-3 (the two sides then sit within rounding of a tie).
Every comparison reports units, exact matches, excused and unexcused
mismatches; tests require zero unexcused mismatches and a small mismatch
rate.
"""

from __future__ import annotations

import math
from typing import Dict, List

import numpy as np
import torch

import oracle as O

MARGIN = 1e-3


def gpu_partitions(cache, b: int, g: int) -> List[List[List[int]]]:
    """Per block, the GPU's buckets as sorted entry lists ordered by bucket id."""
    meta = cache.meta()[b, g].cpu().numpy().astype(np.int64)
    mem = cache.members()[b, g].cpu().numpy().astype(np.int64) & 0xFFFF
    nb = mem.shape[0]
    out = []
    for blk in range(nb):
        leaves = []
        for r in range(O.LEAVES_PER_BLOCK):
            m = int(meta[blk * O.LEAVES_PER_BLOCK + r])
            size, off = m & 0xFF, (m >> 8) & 0x3FF
            leaves.append(sorted(mem[blk, off: off + size].tolist()))
        out.append(leaves)
    return out


def ward_first_divergence_margin(E: np.ndarray, gpu_clusters: List[List[int]]) -> float:
    """Oracle margin at its first merge that the GPU partition does not contain."""
    res = O.ward_block(E, margins=True)
    label = np.empty(len(E), dtype=np.int64)
    for ci, c in enumerate(gpu_clusters):
        label[c] = ci
    members = [[i] for i in range(len(E))]
    for (a, b, d, conflict, glob) in res["merges"]:
        merged = members[a] + members[b]
        members[a], members[b] = merged, []
        if len(set(label[merged].tolist())) > 1:
            return min(conflict, res["stop_gap"])
    return res["stop_gap"]


def compare_ward(entries: np.ndarray, oracle_clusters, gpu_clusters) -> Dict:
    """entries: all pooled entries of the head [nb*512, 64]."""
    stats = dict(blocks=len(oracle_clusters), exact=0, excused=0, unexcused=0, margins=[])
    for blk, (oc, gc) in enumerate(zip(oracle_clusters, gpu_clusters)):
        if [list(c) for c in oc] == gc:
            stats["exact"] += 1
            continue
        E = entries[blk * O.BLOCK_ENTRIES:(blk + 1) * O.BLOCK_ENTRIES]
        m = ward_first_divergence_margin(E, gc)
        stats["margins"].append(m)
        if m < MARGIN:
            stats["excused"] += 1
        else:
            stats["unexcused"] += 1
    return stats


def lr_row(lr_idx: np.ndarray, lr_cnt: int) -> np.ndarray:
    return lr_idx[: max(lr_cnt, 0)].astype(np.int64)


def check_lr_wellformed(row: np.ndarray, k: int, t: int, n_blocks: int, n_sinks: int, window: int, cnt: int,
                        flat: bool = True):
    """Properties every long-range list has: sorted, unique, eligible, count
    rule (flat search: min(k, eligible tokens); a tree beam may hold fewer)."""
    nvis, sink_end, l0 = O.query_geometry(t, n_blocks, n_sinks, window)
    total = max(0, l0 - sink_end)
    if flat:
        assert cnt == min(k, total), (cnt, k, total)
    else:
        assert 0 <= cnt <= min(k, total), (cnt, k, total)
    if len(row):
        assert np.all(np.diff(row) > 0)
        assert row[0] >= sink_end and row[-1] < l0


def tol_for(dtype: str) -> float:
    return 2e-2 if dtype == "bf16" else 1e-5
