#!/usr/bin/env python3
"""Throughput of the fused-dequantization quantized GEMM on one MI355X.

Default workload: dense W4A16 M-sweep, N=14336, K=4096, asymmetric UINT4 weights with a bf16
scale and a uint4 zero-point per (channel, group of 128), bf16 N(0,1) activations, bf16 output,
M in {1, 16, 128, 1024, 8192}. One step = one GEMM at every M of the sweep. The default run then
times the MoE gate_up workload (E=256, top-8, N=4096, K=7168, T in {1, 32, 512, 4096}: token sort
+ grouped GEMM, tokens/s) the same way and reports it under "moe" (--no-moe leaves it out). Other
workloads:
--config w8a8 | w4a8 | w4a4 | w4a16mx | fp8block | w8a16 | f8a16 | w2a16 | w3a16 | moe | moe_mx | moe_fp8b |
moe_layer | moe_layer_w4a8.

Timing follows the Humming announcement's microbenchmark protocol (section "Results: kernel
microbenchmarks": M over powers of two, kernels warmed up and timed independently with cold
caches): every launch reads a different copy of the weights, cycled through more than 3x the
MI355X's 256 MB Infinity Cache, so weight bytes come from HBM. Each M point is a HIP graph of R
back-to-back launches (so small launches are not separated by host gaps; R gives a replay of about
0.5 ms, at most 32 launches), replayed between HIP events on the stream it runs on; per-launch
time = event time / R. One step replays every M
point's graph; `value` = (sum over the M points of one launch's flops) / (sum of the per-launch
times), i.e. the sweep's throughput with each M point counted once.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quantized GEMM TFLOPS and HBM GB/s vs roofline over M=1..8192; MoE tokens/s"
HBM_PEAK_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2500.0, "int8": 5000.0, "fp8": 5000.0, "fp4": 10100.0}

WORKLOADS = {
    "w4a16": dict(name="dense W4A16 M-sweep", N=14336, K=4096, Ms=[1, 16, 128, 1024, 8192], cfg=2,
                  dtype="bf16", peak="bf16"),
    "w8a8": dict(name="dense W8A8 INT8", N=8192, K=8192, Ms=[1, 64, 512, 4096], cfg=3,
                 dtype="int8", peak="int8"),
    "w4a8": dict(name="dense W4A8-MXFP4", N=4096, K=7168, Ms=[1, 32, 256, 2048, 8192], cfg=4,
                 dtype="fp8", peak="fp8"),
    "w4a4": dict(name="dense W4A4-MXFP4", N=4096, K=7168, Ms=[1, 32, 256, 2048, 8192], cfg=4,
                 dtype="fp4", peak="fp4"),
    "w4a16mx": dict(name="dense W4A16-MXFP4 M-sweep", N=14336, K=4096, Ms=[1, 16, 128, 1024, 8192], cfg=2,
                    dtype="bf16", peak="bf16"),
    "fp8block": dict(name="dense FP8 W8A8 with 128x128 / 1x128 block scales", N=8192, K=8192,
                     Ms=[1, 64, 512, 4096], cfg=3, dtype="fp8", peak="fp8"),
    "w8a16": dict(name="dense W8A16 INT8 M-sweep", N=14336, K=4096, Ms=[1, 16, 128, 1024, 8192], cfg=2,
                  dtype="bf16", peak="bf16"),
    "w2a16": dict(name="dense W2A16 M-sweep", N=14336, K=4096, Ms=[1, 16, 128, 1024, 8192], cfg=2,
                  dtype="bf16", peak="bf16"),
    "w3a16": dict(name="dense W3A16 M-sweep", N=14336, K=4096, Ms=[1, 16, 128, 1024, 8192], cfg=2,
                  dtype="bf16", peak="bf16"),
    "f8a16": dict(name="dense W8A16 FP8 e4m3 M-sweep", N=14336, K=4096, Ms=[1, 16, 128, 1024, 8192], cfg=2,
                  dtype="bf16", peak="bf16"),
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def per_launch_stats(ms_per_replay, reps: int) -> dict:
    """Per-launch microseconds from the replays' event times: median (the reported time), min and
    90th percentile over the timed replays."""
    import numpy as np
    us = np.asarray(ms_per_replay, dtype=np.float64) * 1e3 / reps
    return {"median": float(np.median(us)), "min": float(us.min()), "p90": float(np.percentile(us, 90))}


def kernel_sources_sha(files=None) -> str:
    """sha256 over HIP/C++ sources of the library (file names and contents, sorted): the files
    named (those the measured kernel is built from), or every source."""
    import hashlib
    d = os.path.join(ROOT, "quantized_gemm_prepacked_amd", "csrc")
    names = sorted(files) if files else sorted(f for f in os.listdir(d) if f.endswith((".hip", ".h", ".cpp")))
    h = hashlib.sha256()
    for f in names:
        h.update(f.encode())
        with open(os.path.join(d, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str, point: str, plan=None):
    """HBM bytes per launch of the dominant kernel from the FETCH_SIZE / WRITE_SIZE counter passes
    recorded in profiles/traffic_<workload>.json (each counter scaled by what it reads for a copy of
    known size). None when there is no record for this point, when the sources the kernel is built
    from (the record's kernel_files) have changed since the counters were taken, or when the
    library would now run another configuration there (plan, for dense calls)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    try:
        with open(path) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("point") != point or rec.get("kernel_sources_sha256") != kernel_sources_sha(rec.get("kernel_files")):
        return None
    if plan is not None and rec.get("plan") is not None and list(plan) != list(rec["plan"]):
        return None
    return int(rec["hbm_bytes_per_launch"])


def alg_bytes(wl: str, M: int, N: int, K: int) -> int:
    """Bytes the method must move once: packed weights with scales/zeros, activations (+ per-token
    scales), output."""
    if wl == "w4a16":
        w = N * K // 2 + N * (K // 128) * 2 + N * (K // 128) // 2
        return w + M * K * 2 + M * N * 2
    if wl == "w8a8":
        return N * K + N * 4 + M * K + M * 4 + M * N * 2
    if wl == "w4a4":
        return N * K // 2 + N * (K // 32) + M * K // 2 + M * (K // 32) + M * N * 2
    if wl == "w4a16mx":
        return N * K // 2 + N * (K // 32) + M * K * 2 + M * N * 2
    if wl == "fp8block":
        return N * K + (N // 128) * (K // 128) * 4 + M * K + M * (K // 128) * 4 + M * N * 2
    if wl in ("w8a16", "f8a16"):
        return N * K + N * 4 + M * K * 2 + M * N * 2
    if wl == "w2a16":
        return N * K // 4 + N * (K // 128) * 2 + N * (K // 128) // 2 + M * K * 2 + M * N * 2
    if wl == "w3a16":
        return N * K * 3 // 8 + N * (K // 128) * 2 + N * (K // 128) // 2 + M * K * 2 + M * N * 2
    return N * K // 2 + N * (K // 32) + M * K + M * 4 + M * N * 2


def make_inputs(wl: str, spec: dict):
    import numpy as np

    import synth
    N, K, cfg = spec["N"], spec["K"], spec["cfg"]
    import quantized_gemm_prepacked_amd as hq
    if wl == "w4a16":
        d = synth.make_wna16(cfg, 1, N, K, asym=True)
        desc = hq.DESC_W4A16_ASYM
        std = (d["wq"], d["scales"], d["zeros"])
        acts = {M: (synth.normal_bf16(synth.rng(cfg, M), (M, K)), None) for M in spec["Ms"]}
    elif wl == "w8a8":
        d = synth.make_w8a8(cfg, 1, N, K)
        desc = hq.DESC_W8A8
        std = (d["wq"], d["s_ch"], None)
        acts = {}
        for M in spec["Ms"]:
            a = synth.make_w8a8_activations(cfg, M, K)
            acts[M] = (a["xq"], a["s_tok"])
    elif wl == "fp8block":
        d = synth.make_w8a8_fp8_block(cfg, 1, N, K)
        desc = hq.DESC_W8A8_FP8_BLOCK
        std = (d["wq"], d["ws"], None)
        acts = {}
        for M in spec["Ms"]:
            a = synth.make_w8a8_fp8_block(cfg, M, 128, K)          # activations only (N unused)
            acts[M] = (a["xq"], a["xs"])
    elif wl in ("w2a16", "w3a16"):
        d = synth.make_wna2(cfg, 1, N, K) if wl == "w2a16" else synth.make_wna3(cfg, 1, N, K)
        desc = hq.DESC_W2A16_ASYM if wl == "w2a16" else hq.DESC_W3A16_ASYM
        std = (d["wq"], d["scales"], d["zeros"])
        acts = {M: (synth.normal_bf16(synth.rng(cfg, M), (M, K)), None) for M in spec["Ms"]}
    elif wl in ("w8a16", "f8a16"):
        d = synth.make_w8a16(cfg, 1, N, K, fp8=wl == "f8a16")
        desc = hq.DESC_W8A16_FP8 if wl == "f8a16" else hq.DESC_W8A16_INT8
        std = (d["wq"], d["s_ch"], None)
        acts = {M: (synth.normal_bf16(synth.rng(cfg, M), (M, K)), None) for M in spec["Ms"]}
    elif wl == "w4a16mx":
        d = synth.make_w4a16mx(cfg, 1, N, K)
        desc = hq.DESC_W4A16_MXFP4
        std = (d["wq"], d["scales"], None)
        acts = {M: (synth.normal_bf16(synth.rng(cfg, M), (M, K)), None) for M in spec["Ms"]}
    elif wl == "w4a4":
        d = synth.make_w4a4(cfg, 1, N, K)
        desc = hq.DESC_W4A4_MXFP4
        std = (d["wq"], d["scales"], None)
        acts = {}
        for M in spec["Ms"]:
            a = synth.make_w4a4_activations(cfg, M, K)
            acts[M] = (a["xq"], a["xs"])      # the e8m0 block scales travel as a_scale
    else:
        d = synth.make_w4a8(cfg, 1, N, K)
        desc = hq.DESC_W4A8_MXFP4
        std = (d["wq"], d["scales"], None)
        acts = {}
        for M in spec["Ms"]:
            a = synth.make_w4a8_activations(cfg, M, K)
            acts[M] = (a["xq"], a["s_tok"])
    packed = np.zeros(hq.hq_prepacked_bytes(desc, 1, N, K), np.uint8)
    hq.hq_prepack_weights(desc, 1, N, K, *std, packed)
    return desc, std, packed, acts


def oracle_threads() -> int:
    """Threads the CPU oracle's numpy calls run on (its BLAS pool), for cpu_baseline.cores."""
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline(wl: str, spec: dict, std, acts):
    """The CPU oracle, untuned, on a bounded sample of the same workload."""
    import numpy as np

    import oracle
    threads = oracle_threads()
    N, K = spec["N"], spec["K"]
    flops = 0.0
    secs = 0.0
    parts = []
    for M in spec["Ms"]:
        x, s = acts[M]
        rows = None if M <= 1024 else np.arange(1024)
        m_eff = M if rows is None else len(rows)
        t0 = time.perf_counter()
        if wl == "w4a16":
            oracle.ref_wna16(x, std[0], std[1], std[2], 128, rows=rows)
        elif wl == "w8a8":
            oracle.ref_w8a8(x, s, std[0], std[1], rows=rows)
        elif wl == "w4a4":
            oracle.ref_w4a4(x, s, std[0], std[1], rows=rows)
        elif wl == "w4a16mx":
            oracle.ref_w4a16_mx(x, std[0], std[1], rows=rows)
        elif wl in ("w8a16", "f8a16"):
            oracle.ref_w8a16(x, std[0], std[1], fp8=wl == "f8a16", rows=rows)
        elif wl == "w2a16":
            oracle.ref_wna2(x, std[0], std[1], std[2], 128, rows=rows)
        elif wl == "w3a16":
            oracle.ref_wna3(x, std[0], std[1], std[2], 128, rows=rows)
        elif wl == "fp8block":
            oracle.ref_w8a8_fp8_block(x, s, std[0], std[1], rows=rows)
        else:
            oracle.ref_w4a8(x, s, std[0], std[1], rows=rows)
        dt = time.perf_counter() - t0
        secs += dt
        flops += 2.0 * m_eff * N * K
        parts.append(f"M={M}" + ("" if rows is None else f" (first {m_eff} rows)"))
    return {
        "value": round(flops / secs / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
        "kind": "oracle",
        "sample": f"{spec['name']}: " + ", ".join(parts) + f"; fp64 dequantize + matmul, {secs:.1f} s",
    }


def run_dense(args, wl: str):
    import numpy as np
    import torch

    import quantized_gemm_prepacked_amd as hq

    spec = WORKLOADS[wl]
    N, K, Ms = spec["N"], spec["K"], spec["Ms"]
    dev = torch.device("cuda:0")
    log(f"[bench] {spec['name']} N={N} K={K} M={Ms}: generating inputs")
    desc, std, packed, acts = make_inputs(wl, spec)
    if args.stream_k:
        desc = hq.with_flags(desc, hq.HQ_COMPUTE_STREAM_K)
    w0 = torch.from_numpy(packed).to(dev)
    n_copies = max(2, int(np.ceil(768e6 / packed.nbytes)))
    weights = [w0] + [w0.clone() for _ in range(n_copies - 1)]
    dev_acts, outs, wss = {}, {}, {}
    for M in Ms:
        x, s = acts[M]
        xt = torch.from_numpy(np.ascontiguousarray(x).view(np.uint8)).to(dev)
        st = None if s is None else torch.from_numpy(np.ascontiguousarray(s).reshape(-1)).to(dev)
        dev_acts[M] = (xt, st)
        outs[M] = torch.empty((M, N), dtype=torch.int16, device=dev)
        nb = hq.hq_gemm_workspace_bytes(desc, M, N, K)
        wss[M] = (torch.empty(max(nb, 16), dtype=torch.uint8, device=dev), nb)
    stream = torch.cuda.current_stream()
    ctr = [0]

    def launch(M, strm=None):
        w = weights[ctr[0] % n_copies]
        ctr[0] += 1
        xt, st = dev_acts[M]
        ws, nb = wss[M]
        hq.hq_gemm(desc, M, N, K, xt, st, w, outs[M], ws, nb, strm)

    # Launch-bound small calls would be timed with host gaps in between; so each M point is a HIP
    # graph of R back-to-back launches (consecutive launches read different weight copies), and
    # the graph replay is bracketed by events on the capturing stream. R is chosen so that one
    # replay holds about 0.5 ms of launches (from an eager estimate, an upper bound), which
    # amortizes the replay's own start-up cost, between 1 and 32 launches.
    eager = {}
    est = {}
    for M in Ms:
        launch(M, stream)
        torch.cuda.synchronize()
        eager[M] = outs[M].clone()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(3):
            launch(M, stream)
        b.record(stream)
        torch.cuda.synchronize()
        est[M] = a.elapsed_time(b) * 1e3 / 3
    reps = {M: max(1, min(32, int(np.ceil(500.0 / max(est[M], 1e-3))))) for M in Ms}
    graphs = {}
    for M in Ms:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps[M]):
                launch(M)           # current stream = the capture stream
        graphs[M] = g
    for M in Ms:                     # a replay must reproduce the eager result bit for bit
        graphs[M].replay()
        torch.cuda.synchronize()
        if not torch.equal(outs[M], eager[M]):
            raise RuntimeError(f"graph replay differs from the eager result at M={M}")
    log(f"[bench] warmup {args.warmup} steps ({n_copies} weight copies rotate; launches per graph {reps})")
    for _ in range(args.warmup):
        for M in Ms:
            graphs[M].replay()
    torch.cuda.synchronize()
    evs = {M: [] for M in Ms}
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for M in Ms:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            graphs[M].replay()
            b.record(stream)
            evs[M].append((a, b))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sweep = []
    tot_flops = 0.0
    tot_s = 0.0
    for M in Ms:
        st = per_launch_stats([a.elapsed_time(b) for a, b in evs[M]], reps[M])
        us = st["median"]
        fl = 2.0 * M * N * K
        by = alg_bytes(wl, M, N, K)
        tf = fl / (us * 1e-6) / 1e12
        gbs = by / (us * 1e-6) / 1e9
        peak = PEAK_TFLOPS[spec["peak"]]
        frac_c, frac_m = tf / peak, gbs / HBM_PEAK_GBS
        sweep.append({"M": M, "launches_per_graph": reps[M], "us": round(us, 3), "us_min": round(st["min"], 3),
                      "us_p90": round(st["p90"], 3), "tflops": round(tf, 3), "gbps": round(gbs, 1),
                      "bound": "hbm" if frac_m >= frac_c else "mfma",
                      "frac": round(max(frac_c, frac_m), 4), "bytes": by, "flops": fl})
        tot_flops += fl
        tot_s += us * 1e-6
    if wl in ("w8a8", "w4a8", "w4a4", "fp8block"):
        # The step before these GEMMs (dynamic quantization of bf16 activations), timed the same
        # way for context; it is not part of `value`.
        act = {"w8a8": hq.HQ_ACT_INT8_PER_TOKEN, "w4a8": hq.HQ_ACT_FP8E4M3_PER_TOKEN,
               "w4a4": hq.HQ_ACT_MXFP4, "fp8block": hq.HQ_ACT_FP8E4M3_BLOCK128}[wl]
        for row in sweep:
            M = row["M"]
            xb = torch.randn(M, K, device=dev).to(torch.bfloat16)
            xq = torch.empty(M, K, dtype=torch.uint8, device=dev)
            sq = torch.empty(max(M, M * K // 128), dtype=torch.float32, device=dev)
            r = 32
            gq = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gq):
                for _ in range(r):
                    hq.hq_quantize_activations(act, M, K, xb, xq, sq)
            gq.replay()
            torch.cuda.synchronize()
            qe = []
            for _ in range(max(3, args.steps)):
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(stream)
                gq.replay()
                b.record(stream)
                qe.append((a, b))
            torch.cuda.synchronize()
            row["act_quant_us"] = round(per_launch_stats([a.elapsed_time(b) for a, b in qe], r)["median"], 3)
    dom = max(sweep, key=lambda r: r["us"])
    if dom["bound"] == "mfma":
        roof = {"bound": "mfma", "achieved": dom["tflops"], "peak": PEAK_TFLOPS[spec["peak"]],
                "unit": "TFLOP/s", "frac": round(dom["tflops"] / PEAK_TFLOPS[spec["peak"]], 4)}
    else:
        roof = {"bound": "hbm", "achieved": dom["gbps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(dom["gbps"] / HBM_PEAK_GBS, 4)}
    roof["traffic"] = measured_traffic(wl, f"M={dom['M']}", plan=hq.hq_gemm_plan(desc, dom["M"], N, K))
    roof["kernel"] = f"M={dom['M']}"
    line = {
        "metric": METRIC, "value": round(tot_flops / tot_s / 1e12, 4), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": spec["dtype"], "data": "synthetic",
        "config": {"workload": spec["name"], "N": N, "K": K, "M": Ms,
                   **({"compute": "stream_k"} if args.stream_k else {}),
                   "weights": {"w4a16": "uint4 asym g128 bf16 scale + uint4 zero",
                               "w8a8": "int8 per-channel fp32 scale, int8 per-token act",
                               "w4a8": "mxfp4 e2m1 + e8m0 per 32, fp8 e4m3 per-token act",
                               "w4a4": "mxfp4 e2m1 + e8m0 per 32, mxfp4 act (e8m0 per 32)",
                               "w4a16mx": "mxfp4 e2m1 + e8m0 per 32, bf16 act",
                               "fp8block": "e4m3 + fp32 per 128x128 block, e4m3 act + fp32 per 1x128",
                               "w8a16": "int8 per-channel fp32 scale, bf16 act",
                               "f8a16": "fp8 e4m3 per-channel fp32 scale, bf16 act",
                               "w2a16": "uint2 asym g128 bf16 scale + uint2 zero",
                               "w3a16": "uint3 asym g128 bf16 scale + uint3 zero"}[wl]},
        "roofline": roof,
        "sweep": sweep,
    }
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline (bounded sample)")
        line["cpu_baseline"] = cpu_baseline(wl, spec, std, acts)
    else:
        line["cpu_baseline"] = None
    return line


MOE = dict(name="MoE grouped GEMM W4A16 (DeepSeek-V3-shaped gate_up)", E=256, topk=8, N=4096,
           K=7168, Ts=[1, 32, 512, 4096], cfg=5)


def _random_mxfp4_expert(g, N: int, K: int):
    """Standard-format MXFP4 weights with uniformly random codes and e8m0 scales near those of
    N(0, 0.02) blocks (only the data volume matters for throughput)."""
    import numpy as np
    return {"wq": g.integers(0, 256, (N, K // 2), dtype=np.uint8),
            "scales": g.integers(119, 123, (N, K // 32)).astype(np.uint8)}


def workload_name(config: str) -> str:
    """The `config.workload` label of a --config value's bench line."""
    if config in WORKLOADS:
        return WORKLOADS[config]["name"]
    return {
        "moe": MOE["name"],
        "moe_mx": MOE["name"].replace("W4A16", "W4A16-MXFP4"),
        "moe_fp8b": MOE["name"].replace("W4A16", "FP8 W8A8 block-scaled (128x128 weights, 1x128 tokens)"),
        "moe_layer": MOE_LAYER["name"],
        "moe_layer_w4a8": MOE_LAYER["name"].replace("W4A16", "W4A8-MXFP4, tokenwise FP8 activations"),
    }[config]


def run_moe(args, mx=False):
    """Token sort + grouped GEMM per T. tokens/s = T / (t_align + t_gemm). mx: True for MXFP4
    experts (W4A16-MXFP4) instead of INT4 group-128, "fp8b" for block-scaled FP8 experts and
    tokens (the token quantization happens before the timed region)."""
    import numpy as np
    import torch

    import quantized_gemm_prepacked_amd as hq
    import synth

    E, topk, N, K, Ts, cfg = (MOE[k] for k in ("E", "topk", "N", "K", "Ts", "cfg"))
    dev = torch.device("cuda:0")
    fp8b = mx == "fp8b"
    name = workload_name("moe_fp8b" if fp8b else "moe_mx" if mx else "moe")
    if fp8b:
        desc, expert_gen = hq.DESC_W8A8_FP8_BLOCK, synth.random_fp8b_expert
    else:
        desc = hq.DESC_W4A16_MXFP4 if mx else hq.DESC_W4A16_SYM
        expert_gen = _random_mxfp4_expert if mx else synth.random_int4_sym_expert
    peak = "fp8" if fp8b else "bf16"
    stride = hq.hq_prepacked_bytes(desc, 1, N, K)
    log(f"[bench] {name}: {E} experts x {stride / 1e6:.1f} MB prepacked (random codes)")
    w0 = torch.empty(stride * E, dtype=torch.uint8, device=dev)
    g = synth.rng(cfg, 0)
    std = {}
    host = np.zeros(stride, np.uint8)
    for e in range(E):
        d = expert_gen(g, N, K)
        if e < 16:
            std[e] = d
        hq.hq_prepack_weights(desc, 1, N, K, d["wq"], d["ws"] if fp8b else d["scales"], None, host)
        w0[e * stride:(e + 1) * stride].copy_(torch.from_numpy(host))
    n_copies = 4                      # > 256 MB Infinity Cache between reuses even at T = 1
    weights = [w0] + [w0.clone() for _ in range(n_copies - 1)]
    state = {}
    for T in Ts:
        inp = synth.make_moe_inputs(cfg, T, K, E, topk)
        bm = hq.hq_moe_block_m(desc, T, topk, E, N, K)
        cap = hq.hq_moe_align_capacity(T, topk, E, bm)
        hist = np.bincount(inp["topk_ids"].reshape(-1), minlength=E)
        if fp8b:   # tokens quantized to e4m3 with an fp32 scale per 128 k (outside the timed region)
            xq, xs = synth.quantize_fp8_blocks(synth.bf16_bits_to_f32(inp["x"]), 1, 128)
            inp = dict(inp, xq=xq, xs=xs)
            xdev, sdev = torch.from_numpy(xq).to(dev), torch.from_numpy(xs.reshape(-1)).to(dev)
        else:
            xdev, sdev = torch.from_numpy(inp["x"].view(np.int16)).to(dev), None
        state[T] = dict(
            x=xdev, xs=sdev,
            ids=torch.from_numpy(inp["topk_ids"]).to(dev), bm=bm,
            sorted=torch.empty(cap, dtype=torch.int32, device=dev),
            bexp=torch.empty(max(cap // bm, 1), dtype=torch.int32, device=dev),
            offs=torch.empty(E + 1, dtype=torch.int32, device=dev),
            npad=torch.empty(1, dtype=torch.int32, device=dev),
            y=torch.empty((T * topk, N), dtype=torch.int16, device=dev),
            wsb=hq.hq_moe_gemm_workspace_bytes(desc, T, topk, E, N, K, bm),
            active=int((hist > 0).sum()), top=int(hist.max()), inp=inp)
    for T in Ts:
        state[T]["ws"] = torch.empty(max(state[T]["wsb"], 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    ctr = [0]

    def align(T):
        s = state[T]
        hq.hq_moe_align(s["ids"], T, topk, E, s["bm"], s["sorted"], s["bexp"], s["offs"], s["npad"],
                        None, 0, None)

    def gemm(T):
        s = state[T]
        w = weights[ctr[0] % n_copies]
        ctr[0] += 1
        hq.hq_moe_grouped_gemm(desc, T, topk, E, N, K, s["x"], s["xs"], w, s["sorted"], s["bexp"],
                               s["npad"], s["bm"], None, s["y"], s["ws"], s["wsb"], None)

    # One HIP graph of R back-to-back launches per (T, stage); the sort's outputs persist, so R
    # sorts then R grouped GEMMs over rotating weight copies time each stage without host gaps.
    reps = {T: max(1, min(16, int(4e5 // max(T, 1)))) for T in Ts}
    for T in Ts:
        align(T)
        gemm(T)
    torch.cuda.synchronize()
    ga, gg = {}, {}
    for T in Ts:
        ga[T] = torch.cuda.CUDAGraph()
        with torch.cuda.graph(ga[T]):
            for _ in range(reps[T]):
                align(T)
        gg[T] = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gg[T]):
            for _ in range(reps[T]):
                gemm(T)
    for _ in range(args.warmup):
        for T in Ts:
            ga[T].replay()
            gg[T].replay()
    torch.cuda.synchronize()
    rec = {T: [] for T in Ts}
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for T in Ts:
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            evs[0].record(stream)
            ga[T].replay()
            evs[1].record(stream)
            gg[T].replay()
            evs[2].record(stream)
            rec[T].append(evs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sweep = []
    tot_t = 0.0
    tot_tok = 0
    for T in Ts:
        sa = per_launch_stats([e[0].elapsed_time(e[1]) for e in rec[T]], reps[T])
        sg = per_launch_stats([e[1].elapsed_time(e[2]) for e in rec[T]], reps[T])
        ta, tg = sa["median"], sg["median"]
        s = state[T]
        fl = 2.0 * T * topk * N * K
        by = s["active"] * stride + (T * K + T * (K // 128) * 4 if fp8b else T * K * 2) + T * topk * N * 2
        tf = fl / (tg * 1e-6) / 1e12
        gbs = by / (tg * 1e-6) / 1e9
        fc, fm = tf / PEAK_TFLOPS[peak], gbs / HBM_PEAK_GBS
        sweep.append({"T": T, "launches_per_graph": reps[T], "block_m": s["bm"], "active_experts": s["active"], "top_expert_rows": s["top"],
                      "align_us": round(ta, 3), "gemm_us": round(tg, 3), "gemm_us_min": round(sg["min"], 3),
                      "gemm_us_p90": round(sg["p90"], 3),
                      "tokens_per_s": round(T / ((ta + tg) * 1e-6), 1), "tflops": round(tf, 3),
                      "gbps": round(gbs, 1), "bound": "hbm" if fm >= fc else "mfma",
                      "frac": round(max(fc, fm), 4)})
        tot_t += (ta + tg) * 1e-6 * reps[T]
        tot_tok += T * reps[T]
    dom = max(sweep, key=lambda r: r["gemm_us"])
    if dom["bound"] == "mfma":
        roof = {"bound": "mfma", "achieved": dom["tflops"], "peak": PEAK_TFLOPS[peak], "unit": "TFLOP/s",
                "frac": round(dom["tflops"] / PEAK_TFLOPS[peak], 4)}
    else:
        roof = {"bound": "hbm", "achieved": dom["gbps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(dom["gbps"] / HBM_PEAK_GBS, 4)}
    wl_name = "moe_fp8b" if fp8b else "moe_mx" if mx else "moe"
    roof.update(traffic=measured_traffic(wl_name, f"T={dom['T']}"), kernel=f"grouped GEMM T={dom['T']}")
    line = {
        "metric": METRIC, "value": round(tot_tok / tot_t, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": peak,
        "data": "synthetic",
        "config": {"workload": name, "E": E, "topk": topk, "N": N, "K": K, "T": Ts,
                   "routing": "N(0,1) logits + Zipf(1.1) log-prior, softmax top-8"},
        "roofline": roof, "sweep": sweep, "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        inp = state[1]["inp"]
        ids = inp["topk_ids"]
        need = [int(e) for e in np.unique(ids)]
        rg = synth.rng(cfg, 0)
        ws = {}
        for e in range(max(need) + 1):      # regenerate the same random experts in order
            d = expert_gen(rg, N, K)
            if e in need:
                ws[e] = d
        t0 = time.perf_counter()
        if fp8b:
            oracle.ref_moe_gemm_fp8_block(inp["xq"], inp["xs"], ids, lambda e: ws[e], N, E)
        else:
            oracle.ref_moe_gemm(inp["x"], ids, lambda e: ws[e], N, E, 128)
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": round(1 / dt, 3), "unit": "tokens/s", "cores": oracle_threads(),
                                "kind": "oracle", "sample": f"T=1 ({len(need)} experts), {dt:.1f} s"}
    return line


MOE_LAYER = dict(name="MoE layer W4A16 (DeepSeek-V3-shaped: gate_up, SiLU*mul, Down, top-k combine)",
                 E=256, topk=8, H=7168, I=2048, Ts=[1, 32, 512, 4096], cfg=5)


def run_moe_layer(args, w4a8=False):
    """One MoE layer per T: token sort -> gate_up grouped GEMM [T*8, 4096] -> SiLU*mul ->
    Down grouped GEMM [T*8, 7168] with router weights -> top-k combine. The Humming
    announcement times MoE as gate_up plus Down (section "Results: kernel microbenchmarks").
    tokens/s = T / (one layer's time); each stage is also timed on its own. w4a8: MXFP4 experts
    with tokenwise FP8 activations (the announcement's end-to-end W4A8 setting): the tokens and
    the SiLU output are quantized per row to e4m3 before the GEMMs (the latter fused with the
    gated activation: hq_moe_silu_mul_quantize)."""
    import numpy as np
    import torch

    import quantized_gemm_prepacked_amd as hq
    import synth

    E, topk, H, I, Ts, cfg = (MOE_LAYER[k] for k in ("E", "topk", "H", "I", "Ts", "cfg"))
    dev = torch.device("cuda:0")
    desc = hq.DESC_W4A8_MXFP4 if w4a8 else hq.DESC_W4A16_SYM
    name = workload_name("moe_layer_w4a8" if w4a8 else "moe_layer")
    gen = _random_mxfp4_expert if w4a8 else synth.random_int4_sym_expert
    peak = "fp8" if w4a8 else "bf16"
    n_copies = 4                      # > 256 MB Infinity Cache between reuses even at T = 1
    g = synth.rng(cfg, 0)
    std = {}

    def experts(N, K, tag):
        stride = hq.hq_prepacked_bytes(desc, 1, N, K)
        w0 = torch.empty(stride * E, dtype=torch.uint8, device=dev)
        host = np.zeros(stride, np.uint8)
        for e in range(E):
            d = gen(g, N, K)
            if e < 16:
                std[(tag, e)] = d
            hq.hq_prepack_weights(desc, 1, N, K, d["wq"], d["scales"], None, host)
            w0[e * stride:(e + 1) * stride].copy_(torch.from_numpy(host))
        return [w0] + [w0.clone() for _ in range(n_copies - 1)], stride

    log(f"[bench] {name}: preparing {E} gate_up and {E} Down experts (random codes)")
    w_gu, st_gu = experts(2 * I, H, "gu")
    log("[bench] gate_up experts ready")
    w_dn, st_dn = experts(H, I, "dn")
    log("[bench] Down experts ready")
    state = {}
    for T in Ts:
        inp = synth.make_moe_inputs(cfg, T, H, E, topk)
        R = T * topk
        bm = hq.hq_moe_block_m(desc, T, topk, E, 2 * I, H)
        cap = hq.hq_moe_align_capacity(T, topk, E, bm)
        hist = np.bincount(inp["topk_ids"].reshape(-1), minlength=E)
        ws1 = hq.hq_moe_gemm_workspace_bytes(desc, T, topk, E, 2 * I, H, bm)
        ws2 = hq.hq_moe_gemm_workspace_bytes(desc, R, 1, E, H, I, bm)
        state[T] = dict(
            x=torch.from_numpy(inp["x"].view(np.int16)).to(dev),
            ids=torch.from_numpy(inp["topk_ids"]).to(dev),
            tw=torch.from_numpy(inp["topk_weights"].reshape(-1).astype(np.float32)).to(dev), bm=bm,
            sorted=torch.empty(cap, dtype=torch.int32, device=dev),
            bexp=torch.empty(max(cap // bm, 1), dtype=torch.int32, device=dev),
            offs=torch.empty(E + 1, dtype=torch.int32, device=dev),
            npad=torch.empty(1, dtype=torch.int32, device=dev),
            xq=torch.empty((T, H), dtype=torch.uint8, device=dev), xs=torch.empty(T, dtype=torch.float32, device=dev),
            aq=torch.empty((R, I), dtype=torch.uint8, device=dev), as_=torch.empty(R, dtype=torch.float32, device=dev),
            gu=torch.empty((R, 2 * I), dtype=torch.int16, device=dev),
            act=torch.empty((R, I), dtype=torch.int16, device=dev),
            dn=torch.empty((R, H), dtype=torch.int16, device=dev),
            out=torch.empty((T, H), dtype=torch.int16, device=dev),
            ws1=ws1, ws2=ws2, ws=torch.empty(max(ws1, ws2, 16), dtype=torch.uint8, device=dev),
            active=int((hist > 0).sum()), inp=inp)
    stream = torch.cuda.current_stream()
    ctr = [0, 0]

    def align(T):
        s = state[T]
        hq.hq_moe_align(s["ids"], T, topk, E, s["bm"], s["sorted"], s["bexp"], s["offs"], s["npad"],
                        None, 0, None)

    def quant_x(T):
        s = state[T]
        hq.hq_quantize_activations(hq.HQ_ACT_FP8E4M3_PER_TOKEN, T, H, s["x"], s["xq"], s["xs"], None)

    def silu_quant(T):     # the gated activation and its per-row e4m3 quantization in one launch
        s = state[T]
        hq.hq_moe_silu_mul_quantize(hq.HQ_ACT_FP8E4M3_PER_TOKEN, T * topk, I, s["gu"], s["aq"], s["as_"], None)

    def gate_up(T):
        s = state[T]
        w = w_gu[ctr[0] % n_copies]
        ctr[0] += 1
        a, sa = (s["xq"], s["xs"]) if w4a8 else (s["x"], None)
        hq.hq_moe_grouped_gemm(desc, T, topk, E, 2 * I, H, a, sa, w, s["sorted"], s["bexp"],
                               s["npad"], s["bm"], None, s["gu"], s["ws"], s["ws1"], None)

    def silu(T):
        s = state[T]
        hq.hq_moe_silu_mul(T * topk, I, s["gu"], s["act"], None)

    def down(T):
        s = state[T]
        w = w_dn[ctr[1] % n_copies]
        ctr[1] += 1
        a, sa = (s["aq"], s["as_"]) if w4a8 else (s["act"], None)
        hq.hq_moe_grouped_gemm(desc, T * topk, 1, E, H, I, a, sa, w, s["sorted"], s["bexp"],
                               s["npad"], s["bm"], s["tw"], s["dn"], s["ws"], s["ws2"], None)

    def combine(T):
        s = state[T]
        hq.hq_moe_combine(T, topk, E, H, s["ids"], s["dn"], s["out"], None)

    if w4a8:
        stages = {"align": align, "quant_x": quant_x, "gate_up": gate_up, "silu_quant": silu_quant,
                  "down": down, "combine": combine}
    else:
        stages = {"align": align, "gate_up": gate_up, "silu_mul": silu, "down": down, "combine": combine}

    def layer(T):
        for f in stages.values():
            f(T)

    # HIP graphs of R back-to-back layers per T (the whole layer), and of R launches per stage
    reps = {T: max(1, min(16, int(4e5 // max(T, 1)))) for T in Ts}
    for T in Ts:
        layer(T)
    torch.cuda.synchronize()
    graphs = {}
    for T in Ts:
        for stage, f in [("layer", layer)] + list(stages.items()):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                for _ in range(reps[T]):
                    f(T)
            graphs[(T, stage)] = gr
    names = ["layer"] + list(stages)
    for _ in range(args.warmup):
        for gr in graphs.values():
            gr.replay()
    torch.cuda.synchronize()
    rec = {k: [] for k in graphs}
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for T in Ts:
            for stage in names:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                graphs[(T, stage)].replay()
                b.record(stream)
                rec[(T, stage)].append((a, b))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sweep, tot_t, tot_tok = [], 0.0, 0
    for T in Ts:
        us = {n: per_launch_stats([a.elapsed_time(b) for a, b in rec[(T, n)]], reps[T])["median"] for n in names}
        s = state[T]
        R = T * topk
        pt = {}
        for n, (N, K, st) in (("gate_up", (2 * I, H, st_gu)), ("down", (H, I, st_dn))):
            fl = 2.0 * R * N * K
            by = s["active"] * st + (R * (K + 4) if w4a8 else R * K * 2) + R * N * 2
            tf, gbs = fl / (us[n] * 1e-6) / 1e12, by / (us[n] * 1e-6) / 1e9
            fc, fm = tf / PEAK_TFLOPS[peak], gbs / HBM_PEAK_GBS
            pt[n] = {"us": round(us[n], 3), "tflops": round(tf, 3), "gbps": round(gbs, 1),
                     "bound": "hbm" if fm >= fc else "mfma", "frac": round(max(fc, fm), 4)}
        sweep.append({"T": T, "launches_per_graph": reps[T], "block_m": s["bm"], "active_experts": s["active"],
                      "layer_us": round(us["layer"], 3),
                      "stage_us": {n: round(us[n], 3) for n in stages},
                      "tokens_per_s": round(T / (us["layer"] * 1e-6), 1), "gemms": pt})
        tot_t += us["layer"] * 1e-6
        tot_tok += T
    dom_T, dom_n = max(((r["T"], n) for r in sweep for n in ("gate_up", "down")),
                       key=lambda k: next(r for r in sweep if r["T"] == k[0])["gemms"][k[1]]["us"])
    d = next(r for r in sweep if r["T"] == dom_T)["gemms"][dom_n]
    if d["bound"] == "mfma":
        roof = {"bound": "mfma", "achieved": d["tflops"], "peak": PEAK_TFLOPS[peak], "unit": "TFLOP/s",
                "frac": round(d["tflops"] / PEAK_TFLOPS[peak], 4)}
    else:
        roof = {"bound": "hbm", "achieved": d["gbps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(d["gbps"] / HBM_PEAK_GBS, 4)}
    roof.update(traffic=measured_traffic("moe_layer_w4a8" if w4a8 else "moe_layer", f"{dom_n} T={dom_T}"),
                kernel=f"{dom_n} grouped GEMM T={dom_T}")
    line = {
        "metric": METRIC, "value": round(tot_tok / tot_t, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": peak,
        "data": "synthetic",
        "config": {"workload": name, "E": E, "topk": topk, "H": H, "I": I, "T": Ts,
                   "routing": "N(0,1) logits + Zipf(1.1) log-prior, softmax top-8"},
        "roofline": roof, "sweep": sweep, "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        inp = state[1]["inp"]
        ids = inp["topk_ids"]
        need = sorted(int(e) for e in np.unique(ids))
        rg = synth.rng(cfg, 0)
        gu_w, dn_w = {}, {}
        for tag, (N, K), dst in (("gu", (2 * I, H), gu_w), ("dn", (H, I), dn_w)):
            for e in range(E):           # regenerate the same random experts in order
                dd = gen(rg, N, K)
                if e in need:
                    dst[e] = dd
        t0 = time.perf_counter()
        if w4a8:
            oracle.ref_moe_layer_w4a8(inp["x"], ids, inp["topk_weights"], lambda e: gu_w[e], lambda e: dn_w[e],
                                      I, H, E)
        else:
            oracle.ref_moe_layer(inp["x"], ids, inp["topk_weights"], lambda e: gu_w[e], lambda e: dn_w[e],
                                 I, H, E, 128)
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": round(1 / dt, 3), "unit": "tokens/s", "cores": oracle_threads(),
                                "kind": "oracle", "sample": f"T=1 ({len(need)} experts), {dt:.1f} s"}
    return line


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="w4a16", choices=sorted(WORKLOADS) + ["moe", "moe_mx", "moe_fp8b", "moe_layer", "moe_layer_w4a8"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stream-k", action="store_true",
                    help="dense workloads: set HQ_COMPUTE_STREAM_K (small-M calls balanced over the CUs)")
    ap.add_argument("--no-moe", action="store_true",
                    help="default workload only: leave out the MoE gate_up sweep that follows the dense one")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this library has no "
              "multi-GPU path: every box here has a single MI355X.", file=sys.stderr)
        sys.exit(2)
    if args.config == "moe":
        line = run_moe(args)
    elif args.config == "moe_mx":
        line = run_moe(args, mx=True)
    elif args.config == "moe_fp8b":
        line = run_moe(args, mx="fp8b")
    elif args.config == "moe_layer":
        line = run_moe_layer(args)
    elif args.config == "moe_layer_w4a8":
        line = run_moe_layer(args, w4a8=True)
    else:
        line = run_dense(args, args.config)
        if args.config == "w4a16" and not args.no_moe:
            # The metric's second half: MoE tokens/s on the DeepSeek-V3-shaped gate_up (token sort +
            # grouped GEMM per T), timed the same way in the same run. `value` stays the dense
            # sweep's TFLOP/s; the MoE line rides along under "moe".
            moe = run_moe(argparse.Namespace(**{**vars(args), "no_cpu_baseline": True}))
            line["moe"] = {k: moe[k] for k in ("value", "unit", "ms_per_step", "config", "roofline", "sweep")}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
