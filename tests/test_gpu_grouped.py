"""GPU parity of the grouped GEMM (rows pre-grouped by expert offsets) against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_prepacked_amd as hq
import synth

from gpu_harness import DEV, check_float, prepack, say, to_dev

pytestmark = pytest.mark.gpu

DESC = hq.DESC_W4A16_SYM
NAN_BF16 = 0x7FC0


def _run(x_bits, offs, E, N, K, experts):
    R = x_bits.shape[0]
    stride = hq.hq_prepacked_bytes(DESC, 1, N, K)
    w = torch.zeros(stride * E, dtype=torch.uint8, device=DEV)
    for e, wd in experts.items():
        w[e * stride:(e + 1) * stride] = prepack(DESC, 1, N, K, wd["wq"], wd["scales"])
    wsb = hq.hq_grouped_gemm_workspace_bytes(DESC, R, E, N, K)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=DEV)
    y = torch.full((max(R, 1), N), NAN_BF16, dtype=torch.int16, device=DEV)
    say(f"[grouped] R={R} E={E} N={N} K={K} offsets[:8]={offs[:8].tolist()}")
    hq.hq_grouped_gemm(DESC, R, E, N, K, to_dev(x_bits.view(np.int16)), None, w, to_dev(offs.astype(np.int32)),
                       y, ws, wsb)
    torch.cuda.synchronize()
    return y[:R].cpu().numpy().view(np.uint16)


def _case(R, E, N, K, counts, seed, lead=0, random_codes=False, cols=None):
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64) + lead
    x = synth.normal_bf16(synth.rng(seed, R), (R, K))
    active = [e for e in range(E) if counts[e] > 0]
    if random_codes:
        experts = {e: synth.random_int4_sym_expert(synth.rng(seed, 7, e), N, K) for e in active}
    else:
        experts = {e: synth.make_moe_weights_expert(seed, e, N, K) for e in active}
    y = _run(x, offs, E, N, K, experts)
    ref, _, valid = oracle.ref_grouped_gemm(x, offs, lambda e: experts[e], N, E, 128, cols=cols)
    got = y if cols is None else y[:, cols]
    check_float(got[valid], ref[valid], f"grouped R={R}")
    assert (y[~valid] == NAN_BF16).all(), "rows outside every range must not be written"
    return y


@pytest.mark.parametrize("R,E,N,K,counts", [
    (100, 4, 256, 512, [30, 0, 50, 20]),                       # 32-row blocks, an empty expert
    (1000, 8, 512, 1024, [400, 10, 0, 250, 1, 200, 39, 100]),   # 64-row blocks, skewed
    (7, 16, 128, 256, [0, 2, 0, 0, 1, 0, 0, 0, 3, 0, 0, 0, 0, 0, 1, 0]),   # 16-row blocks, sparse
    (333, 5, 384, 640, [70, 70, 70, 70, 53]),                 # N not a multiple of 256, 5 groups
    (256, 1, 256, 256, [256]),                                 # one expert: the dense GEMM
])
def test_grouped_gemm(R, E, N, K, counts):
    assert sum(counts) == R
    _case(R, E, N, K, counts, 40 + R)


def test_grouped_gemm_random_shapes():
    """Eight seeded random problems: up to 64 experts with Zipf-like row counts (empty experts
    included, so the block size the library picks varies), rows before the first and after the
    last range, N a multiple of 16 up to 768, K a multiple of 128 up to 1536."""
    g = np.random.default_rng(41)
    done = 0
    while done < 8:
        E = int(g.integers(1, 65))
        N = int(16 * g.integers(1, 49))
        K = int(128 * g.integers(1, 13))
        counts = np.floor(g.pareto(1.2, E) * g.choice([1, 8, 40])).astype(np.int64)
        counts[g.random(E) < 0.2] = 0
        R_used = int(counts.sum())
        lead, tail = int(g.integers(0, 5)), int(g.integers(0, 5))
        R = R_used + lead + tail
        if R == 0 or R * N * K > 3e8:
            continue
        y = _case(R, E, N, K, counts.tolist(), 900 + done, lead=lead, random_codes=True)
        assert (y[:lead] == NAN_BF16).all() and (y[lead + R_used:] == NAN_BF16).all()
        done += 1


def test_grouped_gemm_rows_outside_the_ranges():
    """offsets[0] > 0 and offsets[E] < R: the leading and trailing rows are left untouched."""
    R, E, N, K = 120, 6, 256, 384
    counts = [10, 30, 0, 25, 40, 5]            # 110 rows from row 4 on: rows 0-3 and 114-119 idle
    y = _case(R, E, N, K, counts, 77, lead=4)
    assert (y[:4] == NAN_BF16).all() and (y[114:] == NAN_BF16).all()


def test_grouped_gemm_full_size_sampled():
    """DeepSeek-V3 gate_up shape, 256 experts with the skewed routing's row counts (T = 512,
    top-8: 4096 rows), sampled output columns."""
    E, N, K, T = 256, 4096, 7168, 512
    ids = synth.make_moe_inputs(5, T, K, E, 8)["topk_ids"]
    counts = np.bincount(ids.reshape(-1), minlength=E)
    cols = np.unique(np.concatenate([[0, N - 1], synth.rng(9).integers(0, N, 96)]))
    _case(int(counts.sum()), E, N, K, counts, 5, random_codes=True, cols=cols)


def test_grouped_gemm_argument_errors():
    R, E, N, K = 32, 2, 256, 256
    buf = torch.zeros(R * K, dtype=torch.int16, device=DEV)
    offs = to_dev(np.array([0, 16, 32], np.int32))
    w = torch.zeros(hq.hq_prepacked_bytes(DESC, E, N, K), dtype=torch.uint8, device=DEV)
    wsb = hq.hq_grouped_gemm_workspace_bytes(DESC, R, E, N, K)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    y = torch.empty(R * N, dtype=torch.int16, device=DEV)
    with pytest.raises(hq.HQError):
        hq.hq_grouped_gemm(DESC, R, E, N, K, buf, None, w, offs, y, ws, wsb - 256)
    with pytest.raises(hq.HQError):
        hq.hq_grouped_gemm(DESC, R, E, N, K, buf, torch.ones(R, device=DEV), w, offs, y, ws, wsb)
    with pytest.raises(hq.HQError):
        hq.hq_grouped_gemm(DESC, R, 0, N, K, buf, None, w, offs, y, ws, wsb)
    hq.hq_grouped_gemm(DESC, 0, E, N, K, buf, None, w, offs, y, ws, wsb)   # empty: no-op
    torch.cuda.synchronize()
