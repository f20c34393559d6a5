"""GPU parity of the skinny kernel's few-row forms (M <= 4: one activation copy per unit, the
other MFMA rows repeating the live ones, only live rows reduced and stored) for every dense
format, forced through the tuning override, against the CPU oracle; and their refusal above four
rows."""
import numpy as np
import pytest

import oracle
import quantized_gemm_prepacked_amd as hq

from gpu_harness import check_float, check_ulp, gemm, prepack, say, to_dev
from test_gpu_invariant import _inputs

pytestmark = pytest.mark.gpu

FEW_CFGS = range(30, 35)   # the few-row entries of the skinny configuration table
FMTS = ["w4a16", "w4a16a", "w8a8", "w4a8", "w4a4", "w4a8mx", "w4a16mx", "fp8block",
        "w8a16", "f8a16", "w2a16", "w3a16"]


def _check(fmt, x, s, std, y, what):
    if fmt in ("w4a16", "w4a16a"):
        ref, _ = oracle.ref_wna16(x, std[0], std[1], std[2], 128)
    elif fmt == "w8a8":
        _, _, bits = oracle.ref_w8a8(x, s, std[0], std[1])
        check_ulp(y, bits, what)
        return
    elif fmt == "w4a8":
        ref, _ = oracle.ref_w4a8(x, s, std[0], std[1])
    elif fmt == "w4a4":
        ref, _ = oracle.ref_w4a4(x, s, std[0], std[1])
    elif fmt == "w4a16mx":
        ref, _ = oracle.ref_w4a16_mx(x, std[0], std[1])
    elif fmt == "fp8block":
        ref, _ = oracle.ref_w8a8_fp8_block(x, s, std[0], std[1])
    elif fmt == "w3a16":
        ref, _ = oracle.ref_wna3(x, std[0], std[1], std[2], 128)
    elif fmt == "w2a16":
        ref, _ = oracle.ref_wna2(x, std[0], std[1], std[2], 128)
    elif fmt in ("w8a16", "f8a16"):
        ref, _ = oracle.ref_w8a16(x, std[0], std[1], fp8=fmt == "f8a16")
    else:
        ref, _ = oracle.ref_w4a8_mx(x, s, std[0], std[1])
    check_float(y, ref, what)


@pytest.mark.parametrize("fmt", FMTS)
def test_few_row_forms(fmt, monkeypatch):
    N, K = 512, 1024
    desc, std, x4, s4 = _inputs(fmt, 4, N, K)
    w = prepack(desc, 1, N, K, *std)
    ran = 0
    for M in (1, 3, 4):
        x = np.ascontiguousarray(x4[:M])
        s = None if s4 is None else np.ascontiguousarray(s4[:M])
        for cfg in FEW_CFGS:
            for split in ((1, 2) if cfg == 30 else (1,)):
                monkeypatch.setenv("HQ_TUNE", f"kind=0,cfg={cfg},split={split}")
                plan = hq.hq_gemm_plan(desc, M, N, K)
                assert plan == (0, cfg, split), plan
                say(f"[few rows] {fmt} M={M} cfg={cfg} split={split}")
                y = gemm(desc, M, N, K, to_dev(x), None if s is None else to_dev(s), w)
                _check(fmt, x, s, std, y, f"few rows {fmt} M={M} cfg={cfg} split={split}")
                ran += 1
    assert ran == 18
    # above four rows a forced few-row form is refused like any override that does not fit, and
    # the built-in choice is never one
    monkeypatch.setenv("HQ_TUNE", "kind=0,cfg=30,split=1")
    with pytest.raises(hq.HQError):
        hq.hq_gemm_plan(desc, 5, N, K)
    monkeypatch.delenv("HQ_TUNE")
    assert hq.hq_gemm_plan(desc, 5, N, K)[1] not in FEW_CFGS
