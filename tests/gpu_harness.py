"""Shared plumbing for the GPU parity tests: upload standard-format inputs, prepack, call the
library through its C ABI, and compare with the CPU oracle under the stated tolerances."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import quantized_gemm_prepacked_amd as hq

DEV = "cuda:0"

# Float paths: relative L2 <= 2e-3 and max-abs <= 2e-2 * max|ref| against the unrounded fp64
# oracle. W8A8: int32 accumulator bit-exact, bf16 output within 1 ulp of bf16(oracle).
REL_L2_TOL = 2e-3
MAX_ABS_FRAC = 2e-2


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def prepack(desc, E, N, K, wq, scales, zeros=None) -> torch.Tensor:
    out = np.zeros(hq.hq_prepacked_bytes(desc, E, N, K), np.uint8)
    hq.hq_prepack_weights(desc, E, N, K, wq, scales, zeros, out)
    return to_dev(out)


def workspace(nbytes: int):
    if nbytes == 0:
        return None, 0
    return torch.empty(nbytes, dtype=torch.uint8, device=DEV), nbytes


# Sentinels an output keeps when the library never writes it: a bf16 NaN (check_float's finite
# check catches it) or, for int32 outputs, INT32_MIN (outside every W8A8 accumulator's range).
BF16_NAN_BITS = 0x7FC0
I32_SENTINEL = -(2 ** 31)


def gemm(desc, M, N, K, a, a_scale, w_dev, out_dtype=torch.int16):
    fill = BF16_NAN_BITS if out_dtype == torch.int16 else I32_SENTINEL
    y = torch.full((max(M, 1), N), fill, dtype=out_dtype, device=DEV)
    ws, wsb = workspace(hq.hq_gemm_workspace_bytes(desc, M, N, K))
    hq.hq_gemm(desc, M, N, K, a, a_scale, w_dev, y, ws, wsb)
    torch.cuda.synchronize()
    return y[:M].cpu().numpy()


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_float(y_bits: np.ndarray, ref64: np.ndarray, what: str, rounding_floor: bool = False):
    """The float bar. rounding_floor: for outputs so heavy-tailed that rounding the exact result
    once to bf16 already moves it by more than the relative-L2 bar (a few dominant elements, as
    with block scales spread over 2^+-40), the bar is 1.1x that rounding's own error -- no
    bf16-output implementation can do better than the exact result rounded once."""
    y = bf16_to_f64(y_bits.view(np.uint16))
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    err = y - ref64
    rel = np.linalg.norm(err) / max(np.linalg.norm(ref64), 1e-300)
    mx = np.abs(err).max() / max(np.abs(ref64).max(), 1e-300)
    tol = REL_L2_TOL
    if rounding_floor:
        rounded = bf16_to_f64(oracle.round_to_bf16(ref64))
        floor = np.linalg.norm(rounded - ref64) / max(np.linalg.norm(ref64), 1e-300)
        tol = max(REL_L2_TOL, 1.1 * floor)
        say(f"  {what}: exact result rounded once to bf16: rel_l2={floor:.3e}")
    say(f"  {what}: rel_l2={rel:.3e} max_abs/max_ref={mx:.3e}")
    assert rel <= tol, f"{what}: relative L2 {rel:.3e} > {tol:.3e}"
    assert mx <= MAX_ABS_FRAC, f"{what}: max abs err {mx:.3e} x max|ref| > {MAX_ABS_FRAC}"
    return rel, mx


def bf16_ordered(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> integers whose order is the numeric order (+0 and -0 -> 0)."""
    b = bits.astype(np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def check_ulp(y_bits: np.ndarray, ref_bits: np.ndarray, what: str, max_ulp: int = 1):
    d = np.abs(bf16_ordered(y_bits.view(np.uint16)) - bf16_ordered(ref_bits))
    say(f"  {what}: max ulp {d.max()}, exact {np.mean(d == 0) * 100:.2f}%")
    assert d.max() <= max_ulp, f"{what}: bf16 differs by {d.max()} ulp"


def every_configuration(desc, M, N, K, run, check, monkeypatch):
    """Run every configuration of every kernel kind that fits the shape (the tuning table may
    name any of them) and check each output; returns {kind: configurations run}."""
    ran = {}
    for kind in (0, 1, 2, 3):
        for cfg in range(hq.hq_kernel_config_count(kind)):
            monkeypatch.setenv("HQ_TUNE", f"kind={kind},cfg={cfg},split=1")
            try:
                plan = hq.hq_gemm_plan(desc, M, N, K)
            except hq.HQError:
                continue            # the configuration does not fit this shape
            assert plan[:2] == (kind, cfg), f"forced kind={kind} cfg={cfg}, planned {plan}"
            say(f"[every configuration] kind={kind} cfg={cfg} plan={plan}")
            check(run(), f"kind={kind} cfg={cfg}")
            ran[kind] = ran.get(kind, 0) + 1
    monkeypatch.delenv("HQ_TUNE")
    say(f"[every configuration] configurations run per kind: {ran}")
    return ran


def moe_random_shapes(seed: int, n: int, n_multiple: int = 16):
    """n seeded MoE problems (T, topk, E, N, K, block_m, with_router_weights) over few-token,
    mid and large T, every top-k up to 8 and block size 16..128 (128-row blocks only where N
    allows them), small enough for the fp64 oracle."""
    g = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        T = int(g.choice([g.integers(1, 16), g.integers(16, 200), g.integers(200, 700)]))
        topk = int(g.choice([1, 2, 4, 8]))
        E = int(g.integers(max(2, topk), 65))
        N = int(n_multiple * g.integers(1, 768 // n_multiple + 1))
        K = int(128 * g.integers(1, 13))
        bm = int(g.choice([16, 32, 64, 128]))
        if (bm == 128 and N % 128) or T * topk * N * K > 2e8:
            continue
        out.append((T, topk, E, N, K, bm, bool(g.integers(0, 2))))
    return out
