"""The offline autotuner on the GPU: it times the fitting candidates of a small shape, its table
loads, the library then runs the chosen kernels, and their results still meet the oracle bar."""
import numpy as np
import pytest

import oracle
import quantized_gemm_prepacked_amd as hq
import synth
from quantized_gemm_prepacked_amd import autotune

from gpu_harness import check_float, gemm, prepack, say, to_dev

pytestmark = pytest.mark.gpu


def test_autotune_small_shape(tmp_path):
    N, K, Ms = 512, 1024, [1, 300]
    say("[autotune] w4a16a N=512 K=1024 M=1,300")
    res = autotune.tune("w4a16a", N, K, Ms, kinds=(0, 3), max_cfgs=3, target_us=50.0, replays=3, log=say)
    assert [r["M"] for r in res] == Ms and all(r["us"] <= r["default_us"] for r in res)
    path = tmp_path / "table.txt"
    path.write_text("\n".join(autotune.table_lines("w4a16a", N, K, res)) + "\n")
    try:
        hq.hq_load_tuning_table(str(path))
        d = synth.make_wna16(800, 1, N, K, asym=True)
        w = prepack(hq.DESC_W4A16_ASYM, 1, N, K, d["wq"], d["scales"], d["zeros"])
        for r in res:
            assert hq.hq_gemm_plan(hq.DESC_W4A16_ASYM, r["M"], N, K)[:2] == (r["kind"], r["cfg"])
            x = synth.normal_bf16(synth.rng(800, r["M"]), (r["M"], K))
            y = gemm(hq.DESC_W4A16_ASYM, r["M"], N, K, to_dev(x), None, w)
            ref, _ = oracle.ref_wna16(x, d["wq"], d["scales"], d["zeros"], 128)
            check_float(y, ref, f"tuned M={r['M']} {r['kind']},{r['cfg']},{r['split']}")
    finally:
        hq.hq_load_tuning_table(None)
