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

Grouped GEMM: Y[t*topk + j, :] = X[t, :] . dequant(W_e)^T with e = topk_ids[t, j] (W_e INT4
group-quantized with bf16 scales, or MXFP4 with e8m0 block scales), optionally
multiplied by topk_weights[t, j]. It does not depend on the order of sorted_ids.
"""
from __future__ import annotations

import numpy as np

from .codecs import decode_bf16, decode_e4m3, decode_e8m0, decode_int8, round_to_bf16
from .gemm import dequant_mxfp4, dequant_wna16, dequant_wna2, dequant_wna3


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


def _values(a: np.ndarray) -> np.ndarray:
    """bf16 bits (uint16) decoded, or float64 values taken as they are (the exact chain)."""
    a = np.asarray(a)
    return decode_bf16(a) if a.dtype == np.uint16 else a.astype(np.float64)


def _dequant_expert(wd, g: int, cols):
    """An expert's standard-format weights -> float64 [N, K]: INT4 groups with bf16 scales
    (uint16 bits), MXFP4 blocks with e8m0 scales (uint8), or 8-bit codes with an fp32 scale per
    channel ({"wq", "s_ch", "fp8"}: INT8, or e4m3 when fp8 is true), or 2-bit codes with group
    scales and zero-points ({"wq", "scales", "zeros", "bits": 2})."""
    if wd.get("bits") == 2:
        return dequant_wna2(wd["wq"], wd["scales"], wd["zeros"], g, cols)
    if wd.get("bits") == 3:
        return dequant_wna3(wd["wq"], wd["scales"], wd["zeros"], g, cols)
    if "s_ch" in wd:
        c = np.asarray(wd["wq"]) if cols is None else np.asarray(wd["wq"])[np.asarray(cols)]
        q = decode_e4m3(c) if wd.get("fp8") else decode_int8(c).astype(np.float64)
        s = np.asarray(wd["s_ch"], dtype=np.float32).astype(np.float64)
        return q * (s if cols is None else s[np.asarray(cols)])[:, None]
    if np.asarray(wd["scales"]).dtype == np.uint8:
        return dequant_mxfp4(wd["wq"], wd["scales"], cols)
    return dequant_wna16(wd["wq"], wd["scales"], wd.get("zeros"), g, cols)


def ref_moe_gemm(x_bf16: np.ndarray, topk_ids: np.ndarray, expert_weights, N: int, E: int,
                 g: int, topk_weights: np.ndarray | None = None, rows=None, cols=None):
    """Grouped WNA16 GEMM over routed rows. ``expert_weights(e)`` returns the standard-format
    dict (wq, scales[, zeros]) of expert e. Returns (y float64 [R, N'], y bf16 bits, valid),
    R = T*topk (or len(rows)), N' = N (or len(cols)); rows routed to an expert id outside
    [0, E) have no defined output: they are NaN in y and False in ``valid``."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, topk = ids.shape
    flat = np.arange(T * topk) if rows is None else np.asarray(rows, dtype=np.int64)
    x = _values(x_bf16)
    n_cols = N if cols is None else len(cols)
    y = np.full((flat.size, n_cols), np.nan, dtype=np.float64)
    experts = ids.reshape(-1)[flat]
    for e in np.unique(experts):
        if e < 0 or e >= E:
            continue
        sel = np.flatnonzero(experts == e)
        w = _dequant_expert(expert_weights(int(e)), g, cols)
        y[sel] = x[flat[sel] // topk] @ w.T
    if topk_weights is not None:
        tw = np.asarray(topk_weights, dtype=np.float32).astype(np.float64).reshape(-1)[flat]
        y = y * tw[:, None]
    valid = ~np.isnan(y[:, 0]) if n_cols else np.ones(flat.size, dtype=bool)
    bits = round_to_bf16(np.where(np.isnan(y), 0.0, y))
    return y, bits, valid


def ref_grouped_gemm(x_bf16: np.ndarray, expert_offsets: np.ndarray, expert_weights, N: int, E: int,
                     g: int, cols=None):
    """Grouped GEMM over activation rows already grouped by expert (the "Grouped" MoE path of the
    announcement's section "Results: kernel microbenchmarks"): rows [offsets[e], offsets[e+1])
    of X belong to expert e, and Y[r, :] = X[r, :] . dequant(W_e)^T for each of them. The
    offsets are meant to be non-decreasing; a range is read as its intersection with [0, R), so
    a decreasing pair or a bound past R gives fewer rows. Rows in no range have no defined output
    (NaN in y, False in ``valid``). Returns (y float64 [R, N'], y bf16 bits, valid)."""
    x = _values(x_bf16)
    R = x.shape[0]
    offs = np.asarray(expert_offsets, dtype=np.int64)
    n_cols = N if cols is None else len(cols)
    y = np.full((R, n_cols), np.nan, dtype=np.float64)
    for e in range(E):
        lo, hi = min(max(int(offs[e]), 0), R), min(max(int(offs[e + 1]), 0), R)
        if hi <= lo:
            continue
        w = _dequant_expert(expert_weights(e), g, cols)
        y[lo:hi] = x[lo:hi] @ w.T
    valid = ~np.isnan(y[:, 0]) if n_cols else np.ones(R, dtype=bool)
    bits = round_to_bf16(np.where(np.isnan(y), 0.0, y))
    return y, bits, valid


def ref_moe_gemm_q(xq: np.ndarray, s_tok: np.ndarray, topk_ids: np.ndarray, expert_weights, N: int, E: int,
                   act: str, topk_weights: np.ndarray | None = None, rows=None, cols=None):
    """Grouped GEMM with 8-bit per-token activations: act "e4m3" (W4A8: MXFP4 experts) or "int8"
    (W8A8: int8 experts with an fp32 scale per channel, expert dict {"wq", "s_ch"}).
    Y[t*topk + j, :] = s_tok[t] * (X_q[t, :] . W_e^T) (* s_ch for INT8) (* topk_weights[t, j]),
    exact in float64 (the INT8 sum is an exact integer). Returns (y float64 [R, N'], y bf16 bits,
    valid) like ref_moe_gemm."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, topk = ids.shape
    flat = np.arange(T * topk) if rows is None else np.asarray(rows, dtype=np.int64)
    x = decode_e4m3(xq) if act == "e4m3" else decode_int8(xq)
    st = np.asarray(s_tok, dtype=np.float32).astype(np.float64)
    n_cols = N if cols is None else len(cols)
    cidx = np.arange(N) if cols is None else np.asarray(cols)
    y = np.full((flat.size, n_cols), np.nan, dtype=np.float64)
    experts = ids.reshape(-1)[flat]
    for e in np.unique(experts):
        if e < 0 or e >= E:
            continue
        sel = np.flatnonzero(experts == e)
        wd = expert_weights(int(e))
        tok = flat[sel] // topk
        if act == "e4m3":
            w = dequant_mxfp4(wd["wq"], wd["scales"], cols)
            y[sel] = (x[tok] @ w.T) * st[tok][:, None]
        else:
            w = decode_int8(np.asarray(wd["wq"])[cidx]).astype(np.float64)
            sc = np.asarray(wd["s_ch"], dtype=np.float32).astype(np.float64)[cidx]
            y[sel] = (x[tok] @ w.T) * st[tok][:, None] * sc[None, :]
    if topk_weights is not None:
        tw = np.asarray(topk_weights, dtype=np.float32).astype(np.float64).reshape(-1)[flat]
        y = y * tw[:, None]
    valid = ~np.isnan(y[:, 0]) if n_cols else np.ones(flat.size, dtype=bool)
    bits = round_to_bf16(np.where(np.isnan(y), 0.0, y))
    return y, bits, valid


def ref_moe_gemm_fp8_block(xq: np.ndarray, xs: np.ndarray, topk_ids: np.ndarray, expert_weights, N: int,
                           E: int, topk_weights: np.ndarray | None = None, rows=None, cols=None):
    """Grouped GEMM with block-scaled FP8 experts and tokens (the page's FP8 W8A8 with blockwise
    scaling in its MoE form, section "W8A8 / W4A8 / W4A4", Indexed and Grouped layouts): expert
    dict {"wq": e4m3 [N, K], "ws": fp32 [N/128, K/128]}, tokens e4m3 [T, K] with fp32 scales
    xs [T, K/128]. For routed row (t, j) with expert e and 128-k blocks g:
        Y[t*topk + j, n] = sum_g xs[t, g] * ws_e[n // 128, g] * sum_{k in g} xq[t, k] * wq_e[n, k]
    (* topk_weights[t, j]), in float64. Returns (y float64 [R, N'], y bf16 bits, valid) like
    ref_moe_gemm."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, topk = ids.shape
    flat = np.arange(T * topk) if rows is None else np.asarray(rows, dtype=np.int64)
    x = decode_e4m3(xq)
    sa = np.asarray(xs, dtype=np.float32).astype(np.float64)
    G = x.shape[1] // 128
    cidx = np.arange(N) if cols is None else np.asarray(cols)
    y = np.full((flat.size, cidx.size), np.nan, dtype=np.float64)
    experts = ids.reshape(-1)[flat]
    for e in np.unique(experts):
        if e < 0 or e >= E:
            continue
        sel = np.flatnonzero(experts == e)
        wd = expert_weights(int(e))
        tok = flat[sel] // topk
        w = decode_e4m3(np.asarray(wd["wq"])[cidx])
        sw = np.asarray(wd["ws"], dtype=np.float32).astype(np.float64)[cidx // 128]   # [N', G]
        acc = np.zeros((sel.size, cidx.size))
        for g in range(G):
            blk = slice(128 * g, 128 * (g + 1))
            acc += (x[tok, blk] @ w[:, blk].T) * sa[tok, g][:, None] * sw[None, :, g]
        y[sel] = acc
    if topk_weights is not None:
        tw = np.asarray(topk_weights, dtype=np.float32).astype(np.float64).reshape(-1)[flat]
        y = y * tw[:, None]
    valid = ~np.isnan(y[:, 0]) if cidx.size else np.ones(flat.size, dtype=bool)
    bits = round_to_bf16(np.where(np.isnan(y), 0.0, y))
    return y, bits, valid


def ref_moe_gemm_mx(xq: np.ndarray, xs: np.ndarray, topk_ids: np.ndarray, expert_weights, N: int, E: int,
                    act: str, topk_weights: np.ndarray | None = None, rows=None, cols=None):
    """Grouped GEMM with MX-scaled tokens and MXFP4 experts (the page's W4A4 and W4A8 with
    microscaling formats, section "W8A8 / W4A8 / W4A4", whose Indexed and Grouped paths it
    names): tokens are MXFP4 (act "mxfp4": packed e2m1 [T, K/2]) or MXFP8 (act "mxfp8": e4m3
    [T, K]) with an e8m0 scale byte per 32 k in xs [T, K/32]; experts {"wq", "scales"} as MXFP4.
        Y[t*topk + j, :] = x_t . dequant_mxfp4(W_e)^T (* topk_weights[t, j]),
    x_t[k] = decode(xq[t, k]) * 2^(xs[t, k // 32] - 127), exact in float64. Returns
    (y float64 [R, N'], y bf16 bits, valid) like ref_moe_gemm."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, topk = ids.shape
    flat = np.arange(T * topk) if rows is None else np.asarray(rows, dtype=np.int64)
    if act == "mxfp4":
        x = dequant_mxfp4(xq, xs)
    else:
        xc = decode_e4m3(xq)
        x = xc * decode_e8m0(xs)[:, np.arange(xc.shape[1]) // 32]
    n_cols = N if cols is None else len(cols)
    y = np.full((flat.size, n_cols), np.nan, dtype=np.float64)
    experts = ids.reshape(-1)[flat]
    for e in np.unique(experts):
        if e < 0 or e >= E:
            continue
        sel = np.flatnonzero(experts == e)
        wd = expert_weights(int(e))
        w = dequant_mxfp4(wd["wq"], wd["scales"], cols)
        y[sel] = x[flat[sel] // topk] @ w.T
    if topk_weights is not None:
        tw = np.asarray(topk_weights, dtype=np.float32).astype(np.float64).reshape(-1)[flat]
        y = y * tw[:, None]
    valid = ~np.isnan(y[:, 0]) if n_cols else np.ones(flat.size, dtype=bool)
    bits = round_to_bf16(np.where(np.isnan(y), 0.0, y))
    return y, bits, valid


def ref_silu_mul(gate_up_bf16: np.ndarray):
    """Gated activation of the MoE expert MLP: for each routed row, the first half of the
    gate_up output is the gate g, the second half the up projection u, and
    act = silu(g) * u = g / (1 + exp(-g)) * u, evaluated in float64 on the bf16 inputs and
    rounded once to bf16. Returns (act float64 [R, I], act bf16 bits)."""
    gu = _values(gate_up_bf16)
    I = gu.shape[1] // 2
    g, u = gu[:, :I], gu[:, I:]
    act = g / (1.0 + np.exp(-g)) * u
    return act, round_to_bf16(act)


def ref_moe_combine(y_bf16: np.ndarray, topk_ids: np.ndarray, E: int):
    """Top-k combine: out[t, :] = sum over k of y[t*topk + k, :] for the k routed to an expert in
    [0, E) (a row routed elsewhere has no output and is left out), float64 sum of the bf16 rows,
    rounded once to bf16. The router weights were applied by the Down GEMM. Returns
    (out float64 [T, N], out bf16 bits)."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, topk = ids.shape
    y = _values(y_bf16).reshape(T, topk, -1)
    valid = ((ids >= 0) & (ids < E))[:, :, None]
    out = np.where(valid, y, 0.0).sum(axis=1)
    return out, round_to_bf16(out)


def ref_moe_layer(x_bf16: np.ndarray, topk_ids: np.ndarray, topk_weights: np.ndarray,
                  gate_up_weights, down_weights, I: int, H: int, E: int, g: int, exact: bool = False):
    """One MoE layer: per routed row (t, k) with expert e = topk_ids[t, k],
        gu  = bf16(x[t] . Wgu_e^T)          (gate_up GEMM, N = 2I)
        a   = bf16(silu(gu[:I]) * gu[I:])    (gated activation)
        d   = bf16(w[t, k] * a . Wd_e^T)      (Down GEMM, N = H, router weight in its epilogue)
        out[t] = bf16(sum_k d)                (top-k combine)
    Each stage is exact float64 arithmetic on its bf16 inputs, rounded once to bf16 at the stage
    boundary -- the tensors a layer hands on are bf16. Returns the bf16 bits of every stage
    (gate_up [T*topk, 2I], act [T*topk, I], down [T*topk, H], out [T, H]).

    exact=True keeps every stage boundary in float64 instead (the same chain with no rounding;
    rows routed nowhere are 0) and returns float64 values: the distance between the two chains
    is the rounding noise that the bf16 boundaries alone put into the layer."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, topk = ids.shape
    pick = (lambda r: np.nan_to_num(r[0], nan=0.0)) if exact else (lambda r: r[1])
    gu = pick(ref_moe_gemm(x_bf16, ids, gate_up_weights, 2 * I, E, g))
    act = pick(ref_silu_mul(gu))
    d = pick(ref_moe_gemm(act, ids.reshape(-1, 1), down_weights, H, E, g,
                          topk_weights=np.asarray(topk_weights).reshape(-1, 1)))
    out = pick(ref_moe_combine(d, ids, E))
    return {"gate_up": gu, "act": act, "down": d, "out": out}


def ref_moe_layer_w4a8(x_bf16: np.ndarray, topk_ids: np.ndarray, topk_weights: np.ndarray,
                       gate_up_weights, down_weights, I: int, H: int, E: int):
    """The MoE layer with MXFP4 experts and tokenwise FP8 activations -- the page's end-to-end
    W4A8 setting (section "End-to-end inference performance": the model's MXFP4 weights kept,
    activations quantized per token to FP8). Per routed row (t, k) with expert e:
        xq, xs = per-token e4m3 quantization of x            (each token row)
        gu  = bf16(xs[t] * xq[t] . Wgu_e^T)
        a   = bf16(silu(gu[:I]) * gu[I:])
        aq, as = per-token e4m3 quantization of a           (each routed row)
        d   = bf16(w[t, k] * as[r] * aq[r] . Wd_e^T)
        out[t] = bf16(sum_k d)
    Stages as in ref_moe_layer, with the quantizer of actquant.quantize_per_token before each
    GEMM. Returns the bf16 bits of every stage and the activation codes and scales."""
    from .actquant import quantize_per_token
    ids = np.asarray(topk_ids, dtype=np.int64)
    xq, xs = quantize_per_token(x_bf16, "e4m3")
    gu = ref_moe_gemm_q(xq, xs, ids, gate_up_weights, 2 * I, E, "e4m3")[1]
    act = ref_silu_mul(gu)[1]
    aq, as_ = quantize_per_token(act, "e4m3")
    d = ref_moe_gemm_q(aq, as_, ids.reshape(-1, 1), down_weights, H, E, "e4m3",
                       topk_weights=np.asarray(topk_weights).reshape(-1, 1))[1]
    out = ref_moe_combine(d, ids, E)[1]
    return {"xq": xq, "xs": xs, "gate_up": gu, "act": act, "aq": aq, "as": as_, "down": d, "out": out}
