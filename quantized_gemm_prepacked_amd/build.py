"""Ahead-of-time build of libhq.so for gfx950 with hipcc (no JIT, no torch extension machinery).

Every HIP source is compiled for ``--offload-arch=gfx950`` only; the host-only prepack and the C
ABI are compiled by the same driver. Objects go to ``_build/`` next to this file, the shared
library to ``libhq.so`` in the package directory.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libhq.so")
PROBE_OUT = os.path.join(PKG, "libhq_probe.so")
BUILD = os.path.join(PKG, "_build")

SOURCES = ["hq_api.cpp", "prepack.cpp", "gemm_dispatch.hip", "gemm_skinny.hip", "gemm_tiled.hip", "gemm_pipe.hip", "gemm_pingpong.hip", "moe_align.hip", "moe_layer.hip", "act_quant.hip", "tuning_table.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _hip_runtime_dir() -> str:
    """Directory of the HIP runtime to link against.

    PyTorch-ROCm ships its own libamdhip64/libhsa-runtime64. Device memory and streams come from
    PyTorch, so the kernels must be registered with that same runtime: a second HIP runtime in
    the process opens its own HSA instance and sees no device. The library records the
    runtime's SONAME, so when PyTorch is loaded first (the binding imports it before opening
    libhq.so) the loader reuses PyTorch's copy; loaded on its own, it resolves to ROCm's.
    """
    try:
        import importlib.util
        spec = importlib.util.find_spec("torch")
        if spec and spec.origin:
            d = os.path.join(os.path.dirname(spec.origin), "lib")
            if os.path.exists(os.path.join(d, "libamdhip64.so")):
                return d
    except Exception:
        pass
    return "/opt/rocm/lib"


COMMON = ["-O3", "-fPIC", "-std=c++17", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-function"]
# Device code: gfx950 only; keep the compiler from forming packed-fp32 instructions.
# MFMA results stay in ordinary VGPRs: the WNA16 group scale is applied to the accumulators with
# VALU FMAs, which would otherwise shuttle every value between AGPRs and VGPRs.
DEVICE = ["-x", "hip", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-rdc", "-munsafe-fp-atomics", "-mllvm", "-amdgpu-mfma-vgpr-form=true"]


def _compile(src: str) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC, *COMMON]
    if src.endswith(".hip"):
        cmd += DEVICE
    else:
        cmd += ["-D__HIP_PLATFORM_AMD__"]
    cmd += ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(errs))
    if errs:
        sys.stderr.write("\n".join(errs) + "\n")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libhq.so. Always rebuilds. Returns the library path."""
    if os.path.isdir(BUILD):
        shutil.rmtree(BUILD)
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    rt = _hip_runtime_dir()
    cmd = ["g++", "-shared", "-fPIC", "-o", tmp, *objs, f"-L{rt}", "-l:libamdhip64.so",
           f"-Wl,-rpath,{rt}", "-Wl,--no-undefined"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    # the streaming-read probe of ceilings.py: its own small library, not part of libhq.so
    pobj = _compile("read_probe.hip")
    ptmp = PROBE_OUT + ".tmp"
    r = subprocess.run(["g++", "-shared", "-fPIC", "-o", ptmp, pobj, f"-L{rt}", "-l:libamdhip64.so",
                        f"-Wl,-rpath,{rt}", "-Wl,--no-undefined"], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("probe link failed:\n" + r.stdout + r.stderr)
    os.replace(ptmp, PROBE_OUT)
    if verbose:
        print(f"built {PROBE_OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
