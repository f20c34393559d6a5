"""MoE token sort and grouped GEMM, written as their plain definitions (test infrastructure).

The Humming announcement's "Results: kernel microbenchmarks" section describes Indexed and
Grouped MoE paths "where tokens are distributed across experts and the amount of work per
expert changes with the load", but does not define the token sort. The reading used here:

moe_align (token sort / expert offsets), for topk_ids [T, topk] over E experts and a row
block size block_m:
  counts[e]   = number of flat entries f = t*topk + j with topk_ids[t, j] == e
  padded[e]   = ceil(counts[e] / block_m) * block_m
  offsets     = exclusive prefix sum of padded (E + 1 entries), num_padded = offsets[E]
  sorted_ids[offsets[e] + i] = the i-th flat entry routed to e in ascending order;
                               padding slots hold the sentinel T*topk
  block_expert[b] = the expert whose range holds row b*block_m
Entries whose expert id is outside [0, E) are routed nowhere.

Grouped GEMM: Y[t*topk + j, :] = X[t, :] . dequant(W_e)^T with e = topk_ids[t, j], optionally
multiplied by topk_weights[t, j]. It does not depend on the order of sorted_ids.
"""
from __future__ import annotations

import numpy as np

from .codecs import decode_bf16, round_to_bf16
from .gemm import dequant_wna16


def ref_moe_align(topk_ids: np.ndarray, E: int, block_m: int):
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    n_flat = ids.size
    counts = np.zeros(E, dtype=np.int64)
    for e in range(E):
        counts[e] = int(np.count_nonzero(ids == e))
    padded = (counts + block_m - 1) // block_m * block_m
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(padded)
    num_padded = int(offsets[E])
    sorted_ids = np.full(num_padded, n_flat, dtype=np.int64)
    for e in range(E):
        members = np.flatnonzero(ids == e)             # ascending flat index = stable order
        sorted_ids[offsets[e]:offsets[e] + members.size] = members
    block_expert = np.empty(num_padded // block_m, dtype=np.int64)
    for b in range(block_expert.size):
        row = b * block_m
        block_expert[b] = int(np.searchsorted(offsets, row, side="right") - 1)
    return {
        "counts": counts, "expert_offsets": offsets, "num_padded": num_padded,
        "sorted_ids": sorted_ids, "block_expert": block_expert,
    }


def ref_moe_gemm(x_bf16: np.ndarray, topk_ids: np.ndarray, expert_weights, N: int, E: int,
                 g: int, topk_weights: np.ndarray | None = None, rows=None, cols=None):
    """Grouped WNA16 GEMM over routed rows. ``expert_weights(e)`` returns the standard-format
    dict (wq, scales[, zeros]) of expert e. Returns (y float64 [R, N'], y bf16 bits, valid),
    R = T*topk (or len(rows)), N' = N (or len(cols)); rows routed to an expert id outside
    [0, E) have no defined output: they are NaN in y and False in ``valid``."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, topk = ids.shape
    flat = np.arange(T * topk) if rows is None else np.asarray(rows, dtype=np.int64)
    x = decode_bf16(x_bf16)
    n_cols = N if cols is None else len(cols)
    y = np.full((flat.size, n_cols), np.nan, dtype=np.float64)
    experts = ids.reshape(-1)[flat]
    for e in np.unique(experts):
        if e < 0 or e >= E:
            continue
        sel = np.flatnonzero(experts == e)
        wd = expert_weights(int(e))
        w = dequant_wna16(wd["wq"], wd["scales"], wd.get("zeros"), g, cols)
        y[sel] = x[flat[sel] // topk] @ w.T
    if topk_weights is not None:
        tw = np.asarray(topk_weights, dtype=np.float32).astype(np.float64).reshape(-1)[flat]
        y = y * tw[:, None]
    valid = ~np.isnan(y[:, 0]) if n_cols else np.ones(flat.size, dtype=bool)
    bits = round_to_bf16(np.where(np.isnan(y), 0.0, y))
    return y, bits, valid
