"""Measured ceilings on this GPU, as context for the GEMM's roofline fractions.

Two kinds of reference numbers, timed the way bench.py times the library (a HIP graph of
back-to-back launches, each launch reading a different copy of its operands, cycled through more
than the MI355X's 256 MB Infinity Cache, so the bytes come from HBM):

  read ceiling   the fastest one streaming-read kernel (csrc/read_probe.hip: 16-byte non-temporal
                 loads, grid-stride or a contiguous share per workgroup, 1, 4 or 16 loads in flight
                 per thread, workgroups of 256 or 1024 threads, best of these and of a few grid
                 sizes)
                 reads a fresh buffer of the sizes the decode calls stream: 15.6 MB (the W4A8-MXFP4 weights), 30.5 MB (W4A16, N=14336
                 K=4096), 67 MB (W8A8, N=K=8192) -- the practical bound of an M=1 call, below the
                 8 TB/s data-sheet figure; torch's copy (read + write) beside it.
  vendor GEMMs   torch's unquantized GEMMs (hipBLASLt) at the large-M shapes (bf16 at M=8192
                 N=14336 K=4096, int8 at M=4096 N=K=8192, fp8 at M=8192 N=4096 K=7168) and the
                 bf16 GEMM at the decode shapes: the analogue of the cuBLAS baseline the Humming
                 announcement compares its kernels with (section "Results: kernel
                 microbenchmarks"). They read unquantized operands, so at small M they move 2x
                 (int8/fp8) to 4x (bf16) the weight bytes of the 4-bit library calls.

Usage:  python -m quantized_gemm_prepacked_amd.ceilings [--out file.json]
"""
from __future__ import annotations

import argparse
import json
import math
import sys

import numpy as np
import torch

CACHE_BYTES = 256e6


def _graph_time(fns, reps, iters=20):
    """Median microseconds per launch of fns[i % len(fns)] over a graph of `reps` launches."""
    fns[0]()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(reps):
            fns[i % len(fns)]()
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(iters):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b) * 1e3 / reps)
    return float(np.median(ts))


def _copies(nbytes):
    return max(2, int(math.ceil(3 * CACHE_BYTES / nbytes)))


def _probe_lib():
    import ctypes
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhq_probe.so")
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with quantized_gemm_prepacked_amd/build.py")
    lib = ctypes.CDLL(path)
    f = lib.hqp_stream_read
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int, ctypes.c_void_p]
    return f


def read_ceilings(sizes_mb=(15.6, 30.5, 67.1), wgs_list=(224, 256, 512, 1024, 2048, 4096, 8192)):
    """Best time of the streaming-read probe over a few grid sizes, both ways of dealing the buffer
    to the workgroups and three load depths, and torch's copy (read + write) for comparison."""
    probe = _probe_lib()
    out = []
    for mb in sizes_mb:
        n = int(mb * 1e6) // 16 * 16
        k = _copies(n)
        src = [torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda") for _ in range(k)]
        sink = torch.empty(max(wgs_list), dtype=torch.int32, device="cuda")
        best = None
        for threads in (256, 1024):
            for blocked in (0, 1):
                for loads in (1, 4, 16):
                    for wgs in wgs_list:
                        def rd(s, wgs=wgs, threads=threads, blocked=blocked, loads=loads):
                            assert probe(s.data_ptr(), n, sink.data_ptr(), wgs, threads, blocked, loads,
                                         torch.cuda.current_stream().cuda_stream) == 0
                        us = _graph_time([lambda s=s: rd(s) for s in src], reps=2 * k)
                        if best is None or us < best[0]:
                            best = (us, wgs, blocked, loads, threads)
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        cp = _graph_time([lambda s=s: dst.copy_(s) for s in src], reps=2 * k)
        out.append({"MB": mb, "read_us": round(best[0], 2), "read_GBps": round(n / best[0] / 1e3, 1),
                    "read_workgroups": best[1], "read_layout": "blocked" if best[2] else "grid-stride",
                    "read_loads_in_flight_per_thread": best[3], "read_threads_per_workgroup": best[4],
                    "torch_copy_us": round(cp, 2), "torch_copy_traffic_GBps": round(2 * n / cp / 1e3, 1)})
        del src
    return out


def vendor_gemms():
    rows = []

    def run(name, M, N, K, make, fn, flops_per=2):
        k = _copies(N * K * (2 if "bf16" in name else 1))
        ws = [make() for _ in range(min(k, 8 if M >= 1024 else k))]
        x = ws[0][0]
        us = _graph_time([lambda w=w: fn(x, w[1]) for w in ws], reps=max(len(ws), 4) if M >= 1024 else 2 * len(ws))
        fl = flops_per * M * N * K
        wbytes = N * K * (2 if "bf16" in name else 1)
        rows.append({"gemm": name, "M": M, "N": N, "K": K, "us": round(us, 2),
                     "TFLOPs": round(fl / us / 1e6, 1), "weight_GBps": round(wbytes / us / 1e3, 1)})

    for M, N, K in ((1, 14336, 4096), (16, 14336, 4096), (8192, 14336, 4096)):
        run("bf16 torch.mm", M, N, K,      # weights stored [K, N]: no transposed operand
            lambda M=M, N=N, K=K: (torch.randn(M, K, device="cuda", dtype=torch.bfloat16),
                                   torch.randn(K, N, device="cuda", dtype=torch.bfloat16)),
            lambda x, w: torch.mm(x, w))
    for M in (64, 4096):
        N = K = 8192
        run("int8 torch._int_mm", M, N, K,
            lambda M=M: (torch.randint(-127, 127, (M, K), dtype=torch.int8, device="cuda"),
                         torch.randint(-127, 127, (K, N), dtype=torch.int8, device="cuda")),
            lambda x, w: torch._int_mm(x, w))
    one = torch.ones((), device="cuda")
    for M in (32, 8192):
        N, K = 4096, 7168
        run("fp8 e4m3 torch._scaled_mm", M, N, K,
            lambda M=M: (torch.randn(M, K, device="cuda").to(torch.float8_e4m3fn),
                         torch.randn(N, K, device="cuda").to(torch.float8_e4m3fn)),
            lambda x, w: torch._scaled_mm(x, w.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16))
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=None)
    args = ap.parse_args()
    res = {"device": torch.cuda.get_device_name(0), "torch": torch.__version__,
           "read_ceilings": read_ceilings(), "vendor_gemms": vendor_gemms()}
    text = json.dumps(res, indent=1)
    print(text)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text + "\n")


if __name__ == "__main__":
    sys.exit(main())
