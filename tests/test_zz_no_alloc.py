"""GPU test of hq_gemm_noalloc, the dense GEMM entry point that allocates nothing: its split-K
partials and activation group sums live in the library's own per-GPU scratch array. Through the
C ABI it must give hq_gemm's output bit for bit (same kernels, same plan), and meet the oracle bar,
on two calls in a row with the second one smaller -- the array then still holds the first call's
bytes, which must not leak into the second result."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_prepacked_amd as hq
import synth

from gpu_harness import BF16_NAN_BITS, DEV, check_float, gemm, prepack, say, to_dev

pytestmark = pytest.mark.gpu


def _noalloc(desc, M, N, K, a, a_scale, w):
    y = torch.full((M, N), BF16_NAN_BITS, dtype=torch.int16, device=DEV)
    hq.hq_gemm_noalloc(desc, M, N, K, a, a_scale, w, y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


# (first call, second smaller call) of each kind of scratch use:
#   WNA16 on the LDS kernels: the activation group sums (rows x groups)
#   WNA16 / W4A8 on the small-M kernel with a K split across workgroups: fp32 partials
@pytest.mark.parametrize("desc_name,first,second", [
    ("DESC_W4A16_ASYM", (600, 512, 1024), (300, 256, 512)),
    ("DESC_W4A16_SYM", (20, 256, 16384), (4, 128, 8192)),
    ("DESC_W4A8_MXFP4", (2, 256, 16384), (1, 64, 8192)),
])
def test_noalloc_matches_hq_gemm_twice(desc_name, first, second):
    desc = getattr(hq, desc_name)
    for i, (M, N, K) in enumerate((first, second)):
        ws = hq.hq_gemm_workspace_bytes(desc, M, N, K)
        say(f"[noalloc] {desc_name} call {i}: M={M} N={N} K={K} workspace {ws} B")
        assert 0 < ws <= hq.HQ_NOALLOC_SCRATCH_BYTES      # the case really uses the scratch
        if desc_name == "DESC_W4A8_MXFP4":
            d = synth.make_w4a8(900 + i, M, N, K)
            w = prepack(desc, 1, N, K, d["wq"], d["scales"])
            a, s = to_dev(d["xq"]), to_dev(d["s_tok"])
            ref, _ = oracle.ref_w4a8(d["xq"], d["s_tok"], d["wq"], d["scales"])
        else:
            asym = desc_name.endswith("ASYM")
            d = synth.make_wna16(900 + i, M, N, K, asym=asym)
            w = prepack(desc, 1, N, K, d["wq"], d["scales"], d.get("zeros"))
            a, s = to_dev(d["x"]), None
            ref, _ = oracle.ref_wna16(d["x"], d["wq"], d["scales"], d.get("zeros"), 128)
        y_ws = gemm(desc, M, N, K, a, s, w)
        y_na = _noalloc(desc, M, N, K, a, s, w)
        assert np.array_equal(y_na, y_ws), "hq_gemm_noalloc differs from hq_gemm"
        check_float(y_na, ref, f"noalloc {desc_name} M={M}")


def test_noalloc_rejects_calls_beyond_its_scratch():
    desc = hq.DESC_W4A16_SYM
    M, N, K = 65536, 256, 65536          # group sums: 65536 rows x 512 groups x 4 bytes = 128 MiB
    need = hq.hq_gemm_workspace_bytes(desc, M, N, K)
    assert need > hq.HQ_NOALLOC_SCRATCH_BYTES
    dummy = torch.zeros(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(hq.HQError) as e:
        hq.hq_gemm_noalloc(desc, M, N, K, dummy, None, dummy, dummy)
    assert e.value.status == hq.HQ_ERR_WORKSPACE and "scratch" in str(e.value)
