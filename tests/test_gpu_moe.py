"""GPU parity of the MoE token sort (exact) and the grouped WNA16 GEMM (oracle tolerance)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_prepacked_amd as hq
import synth

from gpu_harness import DEV, check_float, moe_random_shapes, prepack, say, to_dev

pytestmark = pytest.mark.gpu

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))


def align(ids: np.ndarray, E: int, bm: int):
    T, topk = ids.shape
    cap = hq.hq_moe_align_capacity(T, topk, E, bm)
    sorted_ids = torch.full((max(cap, 1),), -7, dtype=torch.int32, device=DEV)
    block_expert = torch.full((max(cap // bm, 1),), -7, dtype=torch.int32, device=DEV)
    offs = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    npad = torch.empty(1, dtype=torch.int32, device=DEV)
    hq.hq_moe_align(to_dev(ids.astype(np.int32)), T, topk, E, bm, sorted_ids, block_expert, offs, npad)
    torch.cuda.synchronize()
    n = int(npad.item())
    be = block_expert.cpu().numpy()
    # blocks past the sorted rows, up to the capacity, are marked as having no expert (-1), so a
    # grouped GEMM launched over the capacity skips them
    assert (be[n // bm: cap // bm] == -1).all()
    return {
        "num_padded": n, "expert_offsets": offs.cpu().numpy(),
        "sorted_ids": sorted_ids.cpu().numpy()[:n], "block_expert": be[:n // bm],
        "dev": (sorted_ids, block_expert, npad),
    }


def _check_align(ids, E, bm):
    got = align(ids, E, bm)
    ref = oracle.ref_moe_align(ids, E, bm)
    assert got["num_padded"] == ref["num_padded"]
    assert np.array_equal(got["expert_offsets"], ref["expert_offsets"])
    assert np.array_equal(got["sorted_ids"], ref["sorted_ids"])
    assert np.array_equal(got["block_expert"], ref["block_expert"])
    return got


def test_moe_align_hand_case():
    """The hand case's routing at the smallest block the library takes (16 rows): expert 0 gets
    flat ids 1, 4; expert 2 gets 0, 2, 5; expert 3 gets 3; sentinel T*topk = 6."""
    c = GOLD["H5_moe_align"]
    say("[moe_align] hand case, block_m 16")
    got = _check_align(np.array(c["topk_ids"], np.int32), c["E"], 16)
    s = got["sorted_ids"].tolist()
    assert got["num_padded"] == 48 and got["expert_offsets"].tolist() == [0, 16, 16, 32, 48]
    assert s[:2] == [1, 4] and s[16:19] == [0, 2, 5] and s[32] == 3
    assert all(v == 6 for v in s[2:16] + s[19:32] + s[33:48])
    assert got["block_expert"].tolist() == [0, 2, 3]


@pytest.mark.parametrize("T", [1, 3, 32, 512, 1100, 4096, 20000])
@pytest.mark.parametrize("bm", [16, 64])
def test_moe_align_skewed_routing(T, bm):
    # 1100 x 8 = 8800 entries: nine workgroups, the last with a ragged tile; 4096 x 8: 32
    # workgroups of one tile; 20000 x 8 = 160000 entries: 79 workgroups of two tiles, each range
    # starting inside an 8192-entry chunk of the histogram pass, the last one ragged
    say(f"[moe_align] T={T} bm={bm}")
    ids = synth.make_moe_inputs(5, T, 64)["topk_ids"]
    _check_align(ids, 256, bm)


@pytest.mark.parametrize("T,topk", [(5, 8), (2600, 4)])
def test_moe_align_512_experts(T, topk):
    # the largest expert count the sort takes; 2600 x 4 = 10400 entries span two chunks
    ids = np.random.default_rng(T).integers(0, 512, (T, topk)).astype(np.int32)
    say(f"[moe_align] E=512 T={T} topk={topk}")
    _check_align(ids, 512, 16)


@pytest.mark.parametrize("T,topk", [(700, 4), (10, 4), (16, 4)])
def test_moe_align_out_of_range_ids_and_small_E(T, topk):
    # 2800 entries over three workgroups; 40 and 64 entries on the one-wave form
    ids = np.random.default_rng(3).integers(-2, 9, (T, topk)).astype(np.int32)
    say(f"[moe_align] invalid ids T={T} topk={topk}")
    _check_align(ids, 7, 32)


@pytest.mark.parametrize("T,topk,E,bm", [(1, 8, 256, 16), (8, 8, 512, 16), (16, 4, 3, 64), (65, 1, 64, 32),
                                         (2, 8, 1, 128)])
def test_moe_align_few_entries(T, topk, E, bm):
    """The one-wave form (at most 64 entries) and the first size past it, against the oracle."""
    ids = np.random.default_rng(T * 100 + E).integers(0, E, (T, topk)).astype(np.int32)
    say(f"[moe_align] few entries T={T} topk={topk} E={E} bm={bm}")
    _check_align(ids, E, bm)


def test_moe_align_and_grouped_gemm_with_no_tokens():
    """T = 0: the sort writes zero offsets and num_padded = 0 and nothing else (the capacity is 0);
    the grouped GEMM returns without a launch and leaves its output as it was."""
    E, bm, N, K = 16, 16, 256, 256
    assert hq.hq_moe_align_capacity(0, 8, E, bm) == 0
    ids = torch.zeros(8, dtype=torch.int32, device=DEV)
    so = torch.full((16,), -7, dtype=torch.int32, device=DEV)
    be = torch.full((16,), -7, dtype=torch.int32, device=DEV)
    offs = torch.full((E + 1,), -7, dtype=torch.int32, device=DEV)
    npad = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    hq.hq_moe_align(ids, 0, 8, E, bm, so, be, offs, npad)
    torch.cuda.synchronize()
    assert int(npad.item()) == 0 and (offs.cpu().numpy() == 0).all()
    assert (so.cpu().numpy() == -7).all() and (be.cpu().numpy() == -7).all()
    desc = hq.DESC_W4A16_SYM
    w = torch.zeros(hq.hq_prepacked_bytes(desc, E, N, K), dtype=torch.uint8, device=DEV)
    x = torch.zeros((1, K), dtype=torch.int16, device=DEV)
    y = torch.full((8, N), 0x7FC0, dtype=torch.int16, device=DEV)
    hq.hq_moe_grouped_gemm(desc, 0, 8, E, N, K, x, None, w, so, be, npad, bm, None, y)
    torch.cuda.synchronize()
    assert (y.cpu().numpy() == 0x7FC0).all()


def _moe_case(T, topk, E, N, K, bm, with_weights, seed, random_codes=False):
    inp = synth.make_moe_inputs(seed, T, K, E, topk)
    ids = inp["topk_ids"]
    active = np.unique(ids)
    if random_codes:   # uniformly random INT4 codes: fast to draw for hundreds of full-size experts
        experts = {int(e): synth.random_int4_sym_expert(synth.rng(seed, 7, int(e)), N, K) for e in active}
    else:
        experts = {int(e): synth.make_moe_weights_expert(seed, int(e), N, K) for e in active}
    desc = hq.DESC_W4A16_SYM
    stride = hq.hq_prepacked_bytes(desc, 1, N, K)
    w = torch.zeros(stride * E, dtype=torch.uint8, device=DEV)
    for e, wd in experts.items():
        w[e * stride:(e + 1) * stride] = prepack(desc, 1, N, K, wd["wq"], wd["scales"])
    al = _check_align(ids, E, bm)
    sorted_ids, block_expert, npad = al["dev"]
    y = torch.full((T * topk, N), 0x7FC0, dtype=torch.int16, device=DEV)
    tw = to_dev(inp["topk_weights"].reshape(-1)) if with_weights else None
    say(f"[moe gemm] T={T} topk={topk} E={E} N={N} K={K} bm={bm} weights={with_weights}")
    wsb = hq.hq_moe_gemm_workspace_bytes(desc, T, topk, E, N, K, bm)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=DEV)
    hq.hq_moe_grouped_gemm(desc, T, topk, E, N, K, to_dev(inp["x"]), None, w, sorted_ids,
                           block_expert, npad, bm, tw, y, ws, wsb)
    torch.cuda.synchronize()
    return inp, experts, y.cpu().numpy()


@pytest.mark.parametrize("T,topk,E,N,K,bm,tw", [
    (5, 2, 4, 64, 256, 16, False),
    (64, 8, 16, 512, 1024, 16, True),
    (300, 4, 8, 256, 512, 32, False),
    (200, 8, 32, 272, 384, 64, True),     # odd channel tiles
    (512, 8, 16, 256, 512, 64, True),     # 64-row blocks on the LDS-tiled kernel
    (700, 8, 64, 384, 1024, 64, False),   # skewed, ragged expert counts, tiled kernel
    (300, 8, 16, 256, 640, 64, True),     # K/128 = 5 groups (not a multiple of 4)
    (400, 8, 16, 1024, 768, 64, True),    # ping-pong 64 x 512 tiles
    (150, 8, 8, 512, 384, 32, True),      # ping-pong 32 x 256 tiles
    (90, 8, 24, 768, 1152, 32, False),    # 32 x 256 tiles, 9 groups, sparse experts
    (600, 8, 16, 512, 512, 128, True),    # 128-row blocks: ping-pong 128 x 256
    (300, 8, 64, 384, 640, 128, False),   # 128 x 128 tiles, 5 groups, every count of live row blocks
])
def test_moe_gemm_small(T, topk, E, N, K, bm, tw):
    inp, experts, y = _moe_case(T, topk, E, N, K, bm, tw, 500 + T)
    ref, _, valid = oracle.ref_moe_gemm(inp["x"], inp["topk_ids"], lambda e: experts[e], N, E, 128,
                                        topk_weights=inp["topk_weights"] if tw else None)
    assert valid.all()
    check_float(y, ref, "moe gemm")


def test_moe_gemm_random_shapes():
    """INT4 experts on eight seeded random problems (T up to 700, top-k 1..8, E up to 64, every
    block size; `moe_random_shapes`), the sort and the grouped GEMM against the oracle."""
    for i, (T, topk, E, N, K, bm, tw) in enumerate(moe_random_shapes(31, 8)):
        inp, experts, y = _moe_case(T, topk, E, N, K, bm, tw, 1500 + i)
        ref, _, valid = oracle.ref_moe_gemm(inp["x"], inp["topk_ids"], lambda e: experts[e], N, E, 128,
                                            topk_weights=inp["topk_weights"] if tw else None)
        assert valid.all()
        check_float(y, ref, f"moe gemm random {i}")


@pytest.mark.parametrize("T", [1, 8, 32, 512, 2048, 4096])
def test_moe_gemm_full_size_sampled(T):
    """DeepSeek-V3-shaped layer: 256 experts, top-8, K=7168, fused gate_up N=4096, at every token
    count of the MoE workload (1, 32, 512, 4096) and two between them; skewed routing, so at
    T=4096 one expert takes nearly every token and many take a handful."""
    E, topk, N, K = 256, 8, 4096, 7168
    bm = hq.hq_moe_block_m(hq.DESC_W4A16_SYM, T, topk, E, N, K)
    inp, experts, y = _moe_case(T, topk, E, N, K, bm, False, 5, random_codes=T > 8)
    cols = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(T).integers(0, N, 128)]))
    ref, _, _ = oracle.ref_moe_gemm(inp["x"], inp["topk_ids"], lambda e: experts[e], N, E, 128, cols=cols)
    check_float(y[:, cols], ref, f"moe full T={T}")
