"""GPU parity of the MoE layer built from the library's calls: token sort -> gate_up grouped GEMM
-> SiLU-gated activation -> Down grouped GEMM (router weights in its epilogue) -> top-k combine.

Each stage is checked on its own against the oracle applied to the GPU's own input of that
stage (so an error is pinned to the stage that made it), then the layer's output against the
oracle's whole layer. The two elementwise stages compute in fp32 and round once to bf16; their
bound is half a bf16 ulp of the result plus the fp32 error before rounding."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_prepacked_amd as hq
import synth

from gpu_harness import DEV, bf16_to_f64, check_float, prepack, say, to_dev

pytestmark = pytest.mark.gpu

DESC = hq.DESC_W4A16_SYM
U24 = 2.0 ** -24


def _ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (normal range; 2^-133 below it)."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax >= 2.0 ** -126, 2.0 ** (e - 7), 2.0 ** -133)


def _check_rounded(got_bits, ref64, delta, what):
    """|bf16 result - exact| <= ulp/2 at (|exact| + delta) + delta, delta = fp32 error bound."""
    got = bf16_to_f64(got_bits.view(np.uint16))
    bound = 0.5 * _ulp_bf16(np.abs(ref64) + delta) + delta
    err = np.abs(got - ref64)
    bad = ~(err <= bound)
    say(f"  {what}: {int(bad.sum())} of {got.size} outside the bound, "
        f"{float(np.mean(got_bits.view(np.uint16) == oracle.round_to_bf16(ref64))):.5f} bit-equal")
    assert not bad.any(), f"{what}: first bad at {np.argwhere(bad)[0]}"


def _silu_bound(gu_bits):
    I = gu_bits.shape[1] // 2
    gu = bf16_to_f64(gu_bits.view(np.uint16))
    act, _ = oracle.ref_silu_mul(gu_bits.view(np.uint16))
    # expf, the sigmoid's division and two products: a few fp32 roundings, plus the absolute
    # error of a subnormal exp(-|g|) (at most 2^-149) carried by |g * u|
    delta = 8 * U24 * np.abs(act) + 2.0 ** -149 * np.abs(gu[:, :I] * gu[:, I:]) * 2
    return act, delta


def _combine_bound(y_bits, ids, E):
    T, topk = ids.shape
    y = bf16_to_f64(y_bits.view(np.uint16)).reshape(T, topk, -1)
    valid = ((ids >= 0) & (ids < E))[:, :, None]
    out, _ = oracle.ref_moe_combine(y_bits.view(np.uint16), ids, E)
    # topk - 1 fp32 additions, each rounding at most 2^-24 of the running sum <= sum |y|
    delta = topk * U24 * np.where(valid, np.abs(y), 0.0).sum(axis=1)
    return out, delta


class Layer:
    """Prepacked gate_up [E, 2I, H] and Down [E, H, I] weights plus the device buffers of one
    layer call; weights exist only for the experts the routing touches."""

    def __init__(self, seed, T, topk, E, H, I, bm=None, invalid_frac=0.0):
        inp = synth.make_moe_inputs(seed, T, H, E, topk)
        ids = inp["topk_ids"].copy()
        if invalid_frac:
            g = synth.rng(seed, 99)
            ids[g.random(ids.shape) < invalid_frac] = -1
        self.T, self.topk, self.E, self.H, self.I = T, topk, E, H, I
        self.x, self.ids, self.tw = inp["x"], ids, inp["topk_weights"]
        active = [int(e) for e in np.unique(ids) if 0 <= e < E]
        self.gu_w = {e: synth.make_moe_weights_expert(seed, e, 2 * I, H) for e in active}
        self.dn_w = {e: synth.make_moe_weights_expert(seed + 1, e, H, I) for e in active}
        self.w_gu = self._pack(self.gu_w, 2 * I, H)
        self.w_dn = self._pack(self.dn_w, H, I)
        self.bm = bm or hq.hq_moe_block_m(DESC, T, topk, E, 2 * I, H)

    def _pack(self, ws, N, K):
        stride = hq.hq_prepacked_bytes(DESC, 1, N, K)
        w = torch.zeros(stride * self.E, dtype=torch.uint8, device=DEV)
        for e, wd in ws.items():
            w[e * stride:(e + 1) * stride] = prepack(DESC, 1, N, K, wd["wq"], wd["scales"])
        return w

    def run(self):
        T, topk, E, H, I, bm = self.T, self.topk, self.E, self.H, self.I, self.bm
        R = T * topk
        cap = hq.hq_moe_align_capacity(T, topk, E, bm)
        sorted_ids = torch.empty(max(cap, 1), dtype=torch.int32, device=DEV)
        block_expert = torch.empty(max(cap // bm, 1), dtype=torch.int32, device=DEV)
        offs = torch.empty(E + 1, dtype=torch.int32, device=DEV)
        npad = torch.empty(1, dtype=torch.int32, device=DEV)
        ids_d = to_dev(self.ids.astype(np.int32))
        hq.hq_moe_align(ids_d, T, topk, E, bm, sorted_ids, block_expert, offs, npad)
        # rows no GEMM writes hold NaN: the later stages must never read them into a result
        gu = torch.full((R, 2 * I), 0x7FC0, dtype=torch.int16, device=DEV)
        act = torch.full((R, I), 0x7FC0, dtype=torch.int16, device=DEV)
        dn = torch.full((R, H), 0x7FC0, dtype=torch.int16, device=DEV)
        out = torch.full((T, H), 0x7FC0, dtype=torch.int16, device=DEV)
        ws1 = hq.hq_moe_gemm_workspace_bytes(DESC, T, topk, E, 2 * I, H, bm)
        ws2 = hq.hq_moe_gemm_workspace_bytes(DESC, R, 1, E, H, I, bm)
        ws = torch.empty(max(ws1, ws2, 16), dtype=torch.uint8, device=DEV)
        hq.hq_moe_grouped_gemm(DESC, T, topk, E, 2 * I, H, to_dev(self.x), None, self.w_gu, sorted_ids,
                               block_expert, npad, bm, None, gu, ws, ws1)
        hq.hq_moe_silu_mul(R, I, gu, act)
        hq.hq_moe_grouped_gemm(DESC, R, 1, E, H, I, act, None, self.w_dn, sorted_ids, block_expert,
                               npad, bm, to_dev(self.tw.reshape(-1).astype(np.float32)), dn, ws, ws2)
        hq.hq_moe_combine(T, topk, E, H, ids_d, dn, out)
        torch.cuda.synchronize()
        return {k: v.cpu().numpy().view(np.uint16) for k, v in
                (("gate_up", gu), ("act", act), ("down", dn), ("out", out))}


def _check_layer(L: Layer, stages=True):
    say(f"[moe layer] T={L.T} topk={L.topk} E={L.E} H={L.H} I={L.I} bm={L.bm}")
    got = L.run()
    valid = ((L.ids >= 0) & (L.ids < L.E)).reshape(-1)
    if stages:
        ref_gu, _, v = oracle.ref_moe_gemm(L.x, L.ids, lambda e: L.gu_w[e], 2 * L.I, L.E, 128)
        assert np.array_equal(v, valid)
        check_float(got["gate_up"][valid], ref_gu[valid], "gate_up")
        act64, delta = _silu_bound(got["gate_up"][valid])
        _check_rounded(got["act"][valid], act64, delta, "silu_mul")
        ref_dn, _, _ = oracle.ref_moe_gemm(got["act"], L.ids.reshape(-1, 1), lambda e: L.dn_w[e], L.H, L.E,
                                           128, topk_weights=L.tw.reshape(-1, 1))
        check_float(got["down"][valid], ref_dn[valid], "down")
        dn = np.where(valid[:, None], got["down"], np.uint16(0))
        out64, delta = _combine_bound(dn, L.ids, L.E)
        _check_rounded(got["out"], out64, delta, "combine")
    # End to end, against the layer with no rounding between stages. The GPU rounds to bf16 at
    # the same four boundaries as the oracle's layer, so both sit at about the same distance from
    # the exact chain -- the rounding noise -- and only that: the kernels' own fp32 error is far
    # smaller. Measured, the two distances agree to 1 % (ratio 1.000-1.010 over every case here).
    # The bar is 1.1x the oracle's own distance (plus the usual max-abs bar): an extra error of
    # its own in the GPU chain, independent of the rounding noise, then passes only below
    # sqrt(1.1^2 - 1) = 0.46 of that distance (~1.7e-3 relative L2), under the float bar.
    args = (L.x, L.ids, L.tw, lambda e: L.gu_w[e], lambda e: L.dn_w[e], L.I, L.H, L.E, 128)
    ref = bf16_to_f64(oracle.ref_moe_layer(*args)["out"])
    exact = oracle.ref_moe_layer(*args, exact=True)["out"]
    out = bf16_to_f64(got["out"])
    assert np.isfinite(out).all()
    norm = np.linalg.norm(exact)
    e_round = np.linalg.norm(ref - exact) / norm
    e_gpu = np.linalg.norm(out - exact) / norm
    mx = np.abs(out - exact).max() / np.abs(exact).max()
    say(f"  layer out: rel_l2 to the exact chain {e_gpu:.3e} (oracle's bf16 chain {e_round:.3e}), "
        f"max_abs/max_ref={mx:.3e}, rel_l2 to the oracle's chain {np.linalg.norm(out - ref) / norm:.3e}")
    # (The GPU chain is not held to the float bar against the oracle's bf16 chain itself: the
    # gated activation is within a bound of its exact value, not correctly rounded, so many of its
    # bf16 values sit one ulp from the oracle's, and the two chains measured up to 2.8e-3 apart --
    # as far apart as each is from the exact chain. Every stage is held to its own bar above.)
    assert e_gpu <= 1.1 * e_round, f"layer out: {e_gpu:.3e} > 1.1 x {e_round:.3e}"
    assert mx <= 2e-2
    return got


@pytest.mark.parametrize("T,topk,E,H,I,bm", [
    (1, 8, 16, 256, 128, 16),
    (5, 2, 4, 256, 256, 16),
    (64, 8, 16, 512, 256, 16),
    (300, 4, 8, 384, 512, 32),       # K = I = 512 on Down, ragged token count
    (256, 8, 32, 640, 384, 64),      # Down K/128 = 3 groups, gate_up N = 768
])
def test_moe_layer_stages(T, topk, E, H, I, bm):
    _check_layer(Layer(900 + T, T, topk, E, H, I, bm))


def test_moe_layer_unrouted_entries():
    """A fifth of the top-k entries route nowhere (expert -1): their rows of every intermediate
    tensor stay unwritten (NaN here) and the combine leaves them out; a token may lose all."""
    L = Layer(31, 120, 4, 8, 256, 256, 16, invalid_frac=0.2)
    L.ids[7, :] = -1
    got = _check_layer(L)
    assert (got["out"][7] == 0).all()


def test_moe_layer_full_size_one_token():
    """DeepSeek-V3 expert shapes: H = 7168, I = 2048 (gate_up N = 4096), 256 experts, top-8; every
    stage against the oracle on the GPU's own input of that stage, then the layer end to end."""
    _check_layer(Layer(7, 1, 8, 256, 7168, 2048))


def test_silu_mul_edge_values():
    """Gates across the whole range, including where exp(-g) overflows fp32 and where the result
    is subnormal in bf16; zero and signed-zero inputs; a ragged row count."""
    g = np.array([0.0, -0.0, 1e-30, -1e-30, 0.5, -0.5, 8.0, -8.0, 20.0, -20.0, 80.0, -80.0, 88.5, -88.5,
                  89.0, -89.0, 95.0, -95.0, 100.0, -100.0, 150.0, -150.0, 1e30, -1e30, 3e38, -3e38,
                  2.0, -3.0, 0.25, -0.25, 1e-3, -1e-3], dtype=np.float32)
    R, I = 37, 32
    gate = np.resize(g, (R, I)) * synth.rng(3).choice([1.0, 1.01, 0.99], (R, I)).astype(np.float32)
    up = synth.rng(4).standard_normal((R, I)).astype(np.float32)
    up[0, :4] = [0.0, -0.0, 1e30, -2.0]
    gu_bits = synth.bf16_bits(np.concatenate([gate, up], axis=1).astype(np.float32))
    act = torch.full((R, I), 0x7FC0, dtype=torch.int16, device=DEV)
    say(f"[silu_mul] edge values R={R} I={I}")
    hq.hq_moe_silu_mul(R, I, to_dev(gu_bits.view(np.int16)), act)
    torch.cuda.synchronize()
    got = act.cpu().numpy().view(np.uint16)
    with np.errstate(over="ignore", invalid="ignore"):
        ref64, delta = _silu_bound(gu_bits)
    # bf16's largest finite value is 3.3895e38; exact results past 3.3962e38 round to infinity
    fin = np.abs(ref64) < 3.389e38
    ovf = np.abs(ref64) > 3.397e38
    assert fin.sum() > 1000 and ovf.any()
    _check_rounded(got[fin], ref64[fin], delta[fin], "silu_mul edges")
    gotf = bf16_to_f64(got)
    assert (np.isinf(gotf[ovf]) & (np.sign(gotf[ovf]) == np.sign(ref64[ovf]))).all()


@pytest.mark.parametrize("T,topk,N", [(1, 1, 8), (3, 8, 7168), (1000, 6, 264)])
def test_combine_against_oracle(T, topk, N):
    E = 16
    g = synth.rng(T, topk, N)
    ids = g.integers(-1, E + 1, (T, topk)).astype(np.int32)
    y = synth.normal_bf16(g, (T * topk, N), std=4.0)
    out = torch.full((T, N), 0x7FC0, dtype=torch.int16, device=DEV)
    say(f"[combine] T={T} topk={topk} N={N}")
    hq.hq_moe_combine(T, topk, E, N, to_dev(ids), to_dev(y.view(np.int16)), out)
    torch.cuda.synchronize()
    out64, delta = _combine_bound(y, ids, E)
    _check_rounded(out.cpu().numpy().view(np.uint16), out64, delta, "combine")


def test_layer_stage_calls_reject_bad_shapes_and_accept_empty():
    buf = torch.zeros(64, dtype=torch.int16, device=DEV)
    hq.hq_moe_silu_mul(0, 8, buf, buf)
    hq.hq_moe_combine(0, 8, 4, 8, buf, buf, buf)
    with pytest.raises(hq.HQError):
        hq.hq_moe_silu_mul(2, 12, buf, buf)
    with pytest.raises(hq.HQError):
        hq.hq_moe_combine(2, 2, 4, 12, buf, buf, buf)
    with pytest.raises(hq.HQError):
        hq.hq_moe_combine(2, 0, 4, 8, buf, buf, buf)


class LayerW4A8:
    """The layer with MXFP4 experts and tokenwise FP8 activations: per-token e4m3 quantization of
    the tokens and of the SiLU output (hq_quantize_activations) before each grouped GEMM."""

    def __init__(self, seed, T, topk, E, H, I):
        inp = synth.make_moe_inputs(seed, T, H, E, topk)
        self.T, self.topk, self.E, self.H, self.I = T, topk, E, H, I
        self.x, self.ids, self.tw = inp["x"], inp["topk_ids"], inp["topk_weights"]
        active = [int(e) for e in np.unique(self.ids)]
        self.gu_w = {e: synth.make_moe_weights_expert_mx(seed, e, 2 * I, H) for e in active}
        self.dn_w = {e: synth.make_moe_weights_expert_mx(seed + 1, e, H, I) for e in active}
        self.desc = hq.DESC_W4A8_MXFP4
        self.w_gu = self._pack(self.gu_w, 2 * I, H)
        self.w_dn = self._pack(self.dn_w, H, I)
        self.bm = hq.hq_moe_block_m(self.desc, T, topk, E, 2 * I, H)

    def _pack(self, ws, N, K):
        stride = hq.hq_prepacked_bytes(self.desc, 1, N, K)
        w = torch.zeros(stride * self.E, dtype=torch.uint8, device=DEV)
        for e, wd in ws.items():
            w[e * stride:(e + 1) * stride] = prepack(self.desc, 1, N, K, wd["wq"], wd["scales"])
        return w

    def run(self):
        T, topk, E, H, I, bm, D = self.T, self.topk, self.E, self.H, self.I, self.bm, self.desc
        R = T * topk
        cap = hq.hq_moe_align_capacity(T, topk, E, bm)
        sorted_ids = torch.empty(cap, dtype=torch.int32, device=DEV)
        block_expert = torch.empty(max(cap // bm, 1), dtype=torch.int32, device=DEV)
        offs = torch.empty(E + 1, dtype=torch.int32, device=DEV)
        npad = torch.empty(1, dtype=torch.int32, device=DEV)
        ids_d = to_dev(self.ids.astype(np.int32))
        hq.hq_moe_align(ids_d, T, topk, E, bm, sorted_ids, block_expert, offs, npad)
        xq = torch.empty((T, H), dtype=torch.uint8, device=DEV)
        xs = torch.empty(T, dtype=torch.float32, device=DEV)
        gu = torch.full((R, 2 * I), 0x7FC0, dtype=torch.int16, device=DEV)
        act = torch.full((R, I), 0x7FC0, dtype=torch.int16, device=DEV)
        aq = torch.empty((R, I), dtype=torch.uint8, device=DEV)
        as_ = torch.empty(R, dtype=torch.float32, device=DEV)
        dn = torch.full((R, H), 0x7FC0, dtype=torch.int16, device=DEV)
        out = torch.full((T, H), 0x7FC0, dtype=torch.int16, device=DEV)
        ws1 = hq.hq_moe_gemm_workspace_bytes(D, T, topk, E, 2 * I, H, bm)
        ws2 = hq.hq_moe_gemm_workspace_bytes(D, R, 1, E, H, I, bm)
        ws = torch.empty(max(ws1, ws2, 16), dtype=torch.uint8, device=DEV)
        hq.hq_quantize_activations(hq.HQ_ACT_FP8E4M3_PER_TOKEN, T, H, to_dev(self.x), xq, xs)
        hq.hq_moe_grouped_gemm(D, T, topk, E, 2 * I, H, xq, xs, self.w_gu, sorted_ids, block_expert, npad, bm,
                               None, gu, ws, ws1)
        hq.hq_moe_silu_mul(R, I, gu, act)
        hq.hq_quantize_activations(hq.HQ_ACT_FP8E4M3_PER_TOKEN, R, I, act, aq, as_)
        hq.hq_moe_grouped_gemm(D, R, 1, E, H, I, aq, as_, self.w_dn, sorted_ids, block_expert, npad, bm,
                               to_dev(self.tw.reshape(-1).astype(np.float32)), dn, ws, ws2)
        hq.hq_moe_combine(T, topk, E, H, ids_d, dn, out)
        torch.cuda.synchronize()
        res = {k: v.cpu().numpy().view(np.uint16) for k, v in
               (("gate_up", gu), ("act", act), ("down", dn), ("out", out))}
        res.update(xq=xq.cpu().numpy(), xs=xs.cpu().numpy(), aq=aq.cpu().numpy(), as_=as_.cpu().numpy())
        return res


@pytest.mark.parametrize("T,topk,E,H,I", [(7, 4, 8, 512, 256), (300, 8, 32, 1024, 256)])
def test_moe_layer_w4a8(T, topk, E, H, I):
    """Every stage against the oracle on the GPU's own input of that stage (the quantizations bit
    for bit), then the layer's output against the oracle's layer: both chains quantize the same
    way, so they differ only where a GEMM's last-bit difference moves an activation code, and the
    float bar applies between them."""
    L = LayerW4A8(60 + T, T, topk, E, H, I)
    say(f"[moe layer w4a8] T={T} topk={topk} E={E} H={H} I={I} bm={L.bm}")
    got = L.run()
    xq, xs = oracle.quantize_per_token(L.x, "e4m3")
    assert np.array_equal(got["xq"], xq) and np.array_equal(got["xs"], xs)
    ref_gu, _, valid = oracle.ref_moe_gemm_q(xq, xs, L.ids, lambda e: L.gu_w[e], 2 * I, E, "e4m3")
    assert valid.all()
    check_float(got["gate_up"], ref_gu, "gate_up w4a8")
    act64, delta = _silu_bound(got["gate_up"])
    _check_rounded(got["act"], act64, delta, "silu_mul")
    aq, as_ = oracle.quantize_per_token(got["act"], "e4m3")
    assert np.array_equal(got["aq"], aq) and np.array_equal(got["as_"], as_)
    ref_dn, _, _ = oracle.ref_moe_gemm_q(aq, as_, L.ids.reshape(-1, 1), lambda e: L.dn_w[e], H, E, "e4m3",
                                         topk_weights=L.tw.reshape(-1, 1))
    check_float(got["down"], ref_dn, "down w4a8")
    out64, delta = _combine_bound(got["down"], L.ids, E)
    _check_rounded(got["out"], out64, delta, "combine")
    ref = oracle.ref_moe_layer_w4a8(L.x, L.ids, L.tw, lambda e: L.gu_w[e], lambda e: L.dn_w[e], I, H, E)
    check_float(got["out"], bf16_to_f64(ref["out"]), "layer out w4a8 vs the oracle's layer")


@pytest.mark.parametrize("R,I", [(37, 256), (5, 2048), (300, 1024)])
@pytest.mark.parametrize("act_fmt", [hq.HQ_ACT_FP8E4M3_PER_TOKEN, hq.HQ_ACT_INT8_PER_TOKEN])
def test_silu_mul_quantize_is_the_two_calls(R, I, act_fmt):
    """The fused gated activation + per-row quantization equals hq_moe_silu_mul followed by
    hq_quantize_activations bit for bit (codes and scales), and its codes are the oracle's
    quantizer applied to that gated activation. Gates include large magnitudes of both signs and a
    zero row."""
    g = synth.rng(70 + R, I)
    gu32 = g.standard_normal((R, 2 * I)).astype(np.float32) * np.float32(3.0)
    gu32[0, :8] = [-100.0, -30.0, 30.0, 100.0, 0.0, -0.0, 1e-30, -1e-30]
    gu32[R - 1] = 0.0                                           # an all-zero row: scale 1, codes 0
    gu = to_dev(synth.bf16_bits(gu32))
    act = torch.empty((R, I), dtype=torch.int16, device=DEV)
    q2 = torch.empty((R, I), dtype=torch.uint8, device=DEV)
    s2 = torch.empty(R, dtype=torch.float32, device=DEV)
    q1 = torch.full((R, I), 0xAB, dtype=torch.uint8, device=DEV)
    s1 = torch.full((R,), -1.0, dtype=torch.float32, device=DEV)
    say(f"[silu_mul_quantize] R={R} I={I} act_fmt={act_fmt}")
    hq.hq_moe_silu_mul(R, I, gu, act)
    hq.hq_quantize_activations(act_fmt, R, I, act, q2, s2)
    hq.hq_moe_silu_mul_quantize(act_fmt, R, I, gu, q1, s1)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(s1, s2)
    kind = "e4m3" if act_fmt == hq.HQ_ACT_FP8E4M3_PER_TOKEN else "int8"
    qo, so = oracle.quantize_per_token(act.cpu().numpy().view(np.uint16), kind)
    assert np.array_equal(q1.cpu().numpy(), qo.view(np.uint8)) and np.array_equal(s1.cpu().numpy(), so)


def test_silu_mul_quantize_rejections():
    with pytest.raises(hq.HQError):
        hq.hq_moe_silu_mul_quantize(hq.HQ_ACT_MXFP4, 4, 64, 16, 16, 16)        # per-token formats only
    with pytest.raises(hq.HQError):
        hq.hq_moe_silu_mul_quantize(hq.HQ_ACT_FP8E4M3_PER_TOKEN, 4, 60, 16, 16, 16)   # I % 8
    hq.hq_moe_silu_mul_quantize(hq.HQ_ACT_FP8E4M3_PER_TOKEN, 0, 64, 0, 0, 0)   # R = 0: no-op
