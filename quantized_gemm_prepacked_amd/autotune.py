"""Offline autotuner: time every kernel configuration that fits a dense shape on this GPU and
write the fastest per M as a tuning table that the library loads ahead of its built-in one.

The Humming announcement's roadmap (section "Roadmap", "Adding autotune") plans to benchmark
candidate configurations on the target device because heuristics cannot pick the best one for
every shape; this is that step, run offline. Usage:

    python -m quantized_gemm_prepacked_amd.autotune --format w4a16a --N 14336 --K 4096 \\
        --M 1,16,128,1024,8192 --out table.txt
    HQ_TUNING_FILE=table.txt python app.py        # or hq_load_tuning_table("table.txt")

Inputs are random codes and scales of the format (the kernels' time does not depend on the
values); every launch reads a different copy of the weights, cycled through more than the
256 MB Infinity Cache, and each candidate is a HIP graph of back-to-back launches, so the times
are those of weights streamed from HBM. A candidate whose output differs from the built-in
choice's by more than a relative L2 of 4e-3 (two kernels each within the float bar of the
exact result) is rejected and reported.
"""
from __future__ import annotations

import argparse
import math
import os
import sys
import time

import numpy as np
import torch

from . import (DESC_W4A16_ASYM, DESC_W4A16_MXFP4, DESC_W4A16_SYM, DESC_W4A4_MXFP4, DESC_W4A8_MXFP4,
               DESC_W4A8_MXFP8, DESC_W8A8, DESC_W8A8_FP8_BLOCK, DESC_W8A16_FP8, DESC_W8A16_INT8, DESC_W2A16_ASYM, DESC_W3A16_ASYM,
               HQError, hq_gemm, hq_gemm_plan, hq_gemm_workspace_bytes, hq_kernel_config_count,
               hq_load_tuning_table, hq_prepack_weights, hq_prepacked_bytes)

# format -> (descriptor, table family name, asym)
FORMATS = {
    "w4a16": (DESC_W4A16_SYM, "wna16", 0),
    "w4a16a": (DESC_W4A16_ASYM, "wna16", 1),
    "w8a8": (DESC_W8A8, "w8a8", 0),
    "w4a8": (DESC_W4A8_MXFP4, "w4a8", 0),
    "w4a4": (DESC_W4A4_MXFP4, "w4a4", 0),
    "w4a8mx": (DESC_W4A8_MXFP8, "w4a8mx", 0),
    "w4a16mx": (DESC_W4A16_MXFP4, "mxw4a16", 0),
    "fp8block": (DESC_W8A8_FP8_BLOCK, "fp8b", 0),
    "w8a16": (DESC_W8A16_INT8, "w8a16", 0),
    "f8a16": (DESC_W8A16_FP8, "f8a16", 0),
    "w2a16": (DESC_W2A16_ASYM, "wna2", 1),
    "w3a16": (DESC_W3A16_ASYM, "wna3", 1),
}
INF_M = 1 << 40


def _weights(fmt: str, N: int, K: int, g: np.random.Generator):
    """Standard-format random weights: (wq, scales, zeros)."""
    if fmt in ("w4a16", "w4a16a"):
        wq = g.integers(0, 256, (N, K // 2), dtype=np.uint8)
        s = (0.01 * (1 + 0.1 * g.standard_normal((N, K // 128)))).astype(np.float32)
        scales = (s.view(np.uint32) >> 16).astype(np.uint16)
        zeros = g.integers(0, 16, (N, K // 128), dtype=np.uint8) if fmt == "w4a16a" else None
        return wq, scales, zeros
    if fmt in ("w2a16", "w3a16"):
        s = (0.01 * (1 + 0.1 * g.standard_normal((N, K // 128)))).astype(np.float32)
        b2 = fmt == "w2a16"
        return (g.integers(0, 256, (N, K // 4 if b2 else 3 * K // 8), dtype=np.uint8),
                (s.view(np.uint32) >> 16).astype(np.uint16), g.integers(0, 4 if b2 else 8, (N, K // 128), dtype=np.uint8))
    if fmt in ("w8a8", "w8a16"):
        return (g.integers(-127, 128, (N, K)).astype(np.int8),
                (0.001 * (1 + g.random(N))).astype(np.float32), None)
    if fmt == "f8a16":
        return (g.integers(0, 0x78, (N, K)).astype(np.uint8) | (g.integers(0, 2, (N, K)).astype(np.uint8) << 7),
                (0.001 * (1 + g.random(N))).astype(np.float32), None)
    if fmt == "fp8block":
        return (g.integers(0, 0x78, (N, K)).astype(np.uint8),
                (0.001 * (1 + g.random((N // 128, K // 128)))).astype(np.float32), None)
    return (g.integers(0, 256, (N, K // 2), dtype=np.uint8),
            g.integers(118, 124, (N, K // 32)).astype(np.uint8), None)


def _activations(fmt: str, M: int, K: int, g: np.random.Generator):
    """(a bytes, a_scale) in the format's activation layout."""
    if fmt in ("w4a16", "w4a16a", "w4a16mx", "w8a16", "f8a16", "w2a16", "w3a16"):
        x = g.standard_normal((M, K)).astype(np.float32)
        return (x.view(np.uint32) >> 16).astype(np.uint16).view(np.uint8), None
    if fmt == "w8a8":
        return g.integers(-127, 128, (M, K)).astype(np.int8).view(np.uint8), (0.01 * (1 + g.random(M))).astype(np.float32)
    if fmt == "w4a8":
        return g.integers(0, 0x78, (M, K)).astype(np.uint8), (0.01 * (1 + g.random(M))).astype(np.float32)
    if fmt == "fp8block":
        return g.integers(0, 0x78, (M, K)).astype(np.uint8), (0.01 * (1 + g.random((M, K // 128)))).astype(np.float32)
    if fmt == "w4a4":
        return (g.integers(0, 256, (M, K // 2), dtype=np.uint8),
                g.integers(124, 130, (M, K // 32)).astype(np.uint8).reshape(-1))
    return g.integers(0, 0x78, (M, K)).astype(np.uint8), g.integers(118, 124, (M, K // 32)).astype(np.uint8).reshape(-1)


def _candidates(kinds, splits, max_cfgs=None):
    out = []
    for kind in kinds:
        n = hq_kernel_config_count(kind)
        for cfg in range(n if max_cfgs is None else min(n, max_cfgs)):
            for split in (splits if kind == 0 else (1,)):
                out.append((kind, cfg, split))
    return out


def tune(fmt: str, N: int, K: int, Ms, kinds=(0, 1, 2, 3), splits=(-1,), max_cfgs=None, target_us=300.0,
         replays=5, log=print, verbose=False):
    """Time every fitting candidate per M; returns [{M, kind, cfg, split, us, default_us,
    default}] with the fastest candidate of each M."""
    desc, _, _ = FORMATS[fmt]
    dev = torch.device("cuda:0")
    g = np.random.default_rng(2024)
    hq_load_tuning_table(None)                # the built-in choice is the baseline
    wq, scales, zeros = _weights(fmt, N, K, g)
    packed = np.zeros(hq_prepacked_bytes(desc, 1, N, K), np.uint8)
    hq_prepack_weights(desc, 1, N, K, wq, scales, zeros, packed)
    w0 = torch.from_numpy(packed).to(dev)
    n_copies = max(2, math.ceil(768e6 / packed.nbytes))
    weights = [w0] + [w0.clone() for _ in range(n_copies - 1)]
    cands = _candidates(kinds, splits, max_cfgs)
    results = []
    saved = os.environ.pop("HQ_TUNE", None)
    try:
        for M in Ms:
            a, s = _activations(fmt, M, K, g)
            at = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
            st = None if s is None else torch.from_numpy(np.ascontiguousarray(s)).to(dev)
            y = torch.empty((M, N), dtype=torch.int16, device=dev)

            def run_one(tune_str):
                if tune_str is None:
                    os.environ.pop("HQ_TUNE", None)
                else:
                    os.environ["HQ_TUNE"] = tune_str
                nb = hq_gemm_workspace_bytes(desc, M, N, K)
                ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
                ctr = [0]

                def launch():
                    hq_gemm(desc, M, N, K, at, st, weights[ctr[0] % n_copies], y, ws, nb)
                    ctr[0] += 1
                launch()
                torch.cuda.synchronize()
                out = y.clone()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(3):
                    launch()
                e1.record()
                torch.cuda.synchronize()
                est = e0.elapsed_time(e1) * 1e3 / 3
                reps = max(1, min(32, int(math.ceil(target_us / max(est, 1e-3)))))
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph):
                    for _ in range(reps):
                        launch()
                graph.replay()
                torch.cuda.synchronize()
                times = []
                for _ in range(replays):
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    graph.replay()
                    e1.record()
                    torch.cuda.synchronize()
                    times.append(e0.elapsed_time(e1) * 1e3 / reps)
                return float(np.median(times)), out

            # warm the clocks with ~0.3 s of the built-in choice before the first timing, so the
            # baseline is not measured colder than the candidates after it
            run_one(None)
            t_end = time.perf_counter() + 0.3
            while time.perf_counter() < t_end:
                run_one(None)
            base_us, base_out = run_one(None)
            base = base_out.view(torch.bfloat16).float()
            default = hq_gemm_plan(desc, M, N, K)
            best = (base_us, default)
            for kind, cfg, split in cands:
                t = f"kind={kind},cfg={cfg},split={split}"
                try:
                    us, out = run_one(t)
                except HQError:
                    continue                      # does not fit this shape
                o = out.view(torch.bfloat16).float()
                rel = float((o - base).norm() / max(float(base.norm()), 1e-30))
                if not math.isfinite(rel) or rel > 4e-3:
                    log(f"  M={M} {t}: output differs from the built-in choice (rel L2 {rel:.2e}), rejected")
                    continue
                if verbose:
                    log(f"  M={M} {t}: {us:.2f} us")
                if us < best[0]:
                    best = (us, (kind, cfg, split))
            kind, cfg, split = best[1]
            results.append(dict(M=M, kind=kind, cfg=cfg, split=split, us=round(best[0], 3),
                                default_us=round(base_us, 3), default=default))
            log(f"M={M}: built-in {default} {base_us:.2f} us -> best ({kind}, {cfg}, {split}) {best[0]:.2f} us")
    finally:
        if saved is None:
            os.environ.pop("HQ_TUNE", None)
        else:
            os.environ["HQ_TUNE"] = saved
    return results


def table_lines(fmt: str, N: int, K: int, results):
    """Table entries: each measured M covers up to the geometric midpoint to the next one."""
    _, fam, asym = FORMATS[fmt]
    rs = sorted(results, key=lambda r: r["M"])
    lines = []
    for i, r in enumerate(rs):
        max_m = INF_M if i + 1 == len(rs) else int(math.sqrt(r["M"] * rs[i + 1]["M"]))
        lines.append(f"{fam} {asym} {N} {K} {max_m} {r['kind']} {r['cfg']} {r['split']}"
                     f"  # M={r['M']}: {r['us']} us (built-in {r['default_us']} us)")
    return lines


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--format", required=True, choices=sorted(FORMATS))
    ap.add_argument("--N", type=int, required=True)
    ap.add_argument("--K", type=int, required=True)
    ap.add_argument("--M", required=True, help="comma-separated M values")
    ap.add_argument("--kinds", default="0,1,2,3")
    ap.add_argument("--splits", default="-1", help="skinny K splits to try (-1 = heuristic)")
    ap.add_argument("--out", default=None)
    ap.add_argument("--verbose", action="store_true", help="print every candidate's time")
    args = ap.parse_args(argv)
    Ms = [int(m) for m in args.M.split(",")]
    res = tune(args.format, args.N, args.K, Ms, kinds=[int(k) for k in args.kinds.split(",")],
               splits=[int(s) for s in args.splits.split(",")], log=lambda m: print(m, file=sys.stderr, flush=True),
               verbose=args.verbose)
    text = "\n".join(["# <family> <asym> <N> <K> <max_m> <kind> <cfg> <split>"] + table_lines(args.format, args.N, args.K, res)) + "\n"
    if args.out:
        with open(args.out, "a") as f:
            f.write(text)
    else:
        sys.stdout.write(text)


if __name__ == "__main__":
    main()
