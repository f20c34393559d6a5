"""Invariants of the seeded standard-format inputs, checked with the oracle's decoders:
codes in range, reconstruction error within half a quantization step, the MX shared-exponent
rule, round-half-even tie cases of the e2m1 encoder, and seed reproducibility."""
import numpy as np

import oracle
import synth


def test_int4_sym_invariants():
    w = synth.rng(1, 0).standard_normal((64, 512), dtype=np.float32) * np.float32(0.02)
    d = synth.quantize_int4_sym(w, 128)
    deq = oracle.dequant_wna16(d["wq"], d["scales"], None, 128)
    s = oracle.decode_bf16(d["scales"])
    assert np.all(np.abs(w - deq) <= s.repeat(128, axis=1) / 2 * (1 + 1e-6) + 1e-12)
    q = oracle.decode_int4_sym(oracle.unpack_nibbles(d["wq"]))
    assert q.min() >= -8 and q.max() <= 7


def test_uint4_asym_invariants():
    w = synth.rng(2, 0).standard_normal((64, 512), dtype=np.float32) * np.float32(0.02)
    d = synth.quantize_uint4_asym(w, 128)
    deq = oracle.dequant_wna16(d["wq"], d["scales"], d["zeros"], 128)
    s = oracle.decode_bf16(d["scales"]).repeat(128, axis=1)
    # zero-point rounding can push the clipped range by up to one step
    assert np.all(np.abs(w - deq) <= s * 1.0 + 1e-12)
    assert np.mean(np.abs(w - deq) <= s / 2 + 1e-12) > 0.97
    assert d["zeros"].max() <= 15


def test_int8_rows_invariants():
    x = synth.rng(3, 0).standard_normal((16, 300), dtype=np.float32)
    q, s = synth.quantize_int8_rows(x)
    assert q.min() >= -127 and q.max() <= 127
    assert np.all(np.abs(x - q * s[:, None]) <= s[:, None] / 2 * (1 + 1e-6))
    assert np.all(np.abs(q).max(axis=1) == 127)


def test_mxfp4_shared_exponent_rule():
    # amax = 0.05: floor(log2 0.05) = -5, minus emax 2 -> -7 -> e8m0 byte 120; 0.05/2^-7 = 6.4
    # saturates to the largest code 0x7 (= 6).
    w = np.zeros((1, 32), np.float32)
    w[0, 3] = 0.05
    d = synth.quantize_mxfp4(w)
    assert d["scales"][0, 0] == 120
    assert oracle.unpack_nibbles(d["wq"])[0, 3] == 0x7
    z = synth.quantize_mxfp4(np.zeros((1, 32), np.float32))
    assert z["scales"][0, 0] == 0 and not z["wq"].any()


def test_e2m1_encoder_ties_to_even():
    vals = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, -0.75, 0.3])
    codes = synth._encode_e2m1(vals)
    assert oracle.decode_e2m1(codes).tolist() == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, -1.0, 0.5]


def test_mxfp4_reconstruction_error():
    w = synth.rng(4, 0).standard_normal((32, 1024), dtype=np.float32) * np.float32(0.02)
    d = synth.quantize_mxfp4(w)
    deq = oracle.dequant_mxfp4(d["wq"], d["scales"])
    x = oracle.decode_e8m0(d["scales"]).repeat(32, axis=1)
    # in units of the block scale: e2m1 spacing is at most 2 (between 4 and 6), so unsaturated
    # elements are within 1; the OCP rule leaves amax/2^e in [4, 8), so saturation at 6 costs
    # less than 2
    err = np.abs(w - deq)
    unsat = np.abs(w) <= 6 * x
    assert np.all(err[unsat] <= x[unsat] + 1e-12)
    assert np.all(err < 2 * x)


def test_fp8_rows_invariants():
    x = synth.rng(5, 0).standard_normal((8, 700), dtype=np.float32)
    q, s = synth.quantize_fp8_rows(x)
    v = oracle.decode_e4m3(q)
    assert not np.isnan(v).any() and np.abs(v).max() <= 448
    rel = np.abs(x - v * s[:, None]) / np.maximum(np.abs(x), 1e-30)
    big = np.abs(x) > s[:, None] * 2 ** -6 * 8     # normal range of e4m3
    assert rel[big].max() <= 2 ** -4 + 1e-7


def test_seeds_reproducible():
    a = synth.make_wna16(2, 4, 64, 256, asym=True)
    b = synth.make_wna16(2, 4, 64, 256, asym=True)
    for k in a:
        assert np.array_equal(a[k], b[k])
    c = synth.make_wna16(2, 5, 64, 256, asym=True)
    assert np.array_equal(a["wq"], c["wq"]) and not np.array_equal(a["x"][:4], c["x"][:4])


def test_moe_routing_skewed_and_valid():
    ids, w = synth.moe_routing(synth.rng(5, 512), 512, 256, 8, bias_rng=synth.rng(5, 1 << 20))
    assert ids.shape == (512, 8) and ids.min() >= 0 and ids.max() < 256
    assert all(len(set(r)) == 8 for r in ids.tolist())
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6) and np.all(np.diff(w, axis=1) <= 1e-7)
    hist = np.bincount(ids.reshape(-1), minlength=256)
    assert hist.max() > 4 * hist.mean()                 # skewed load
