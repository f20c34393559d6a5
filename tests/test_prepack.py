"""Host prepack: an independent unpacker, written from the layout documented in
quantized_gemm_prepacked_amd/csrc/layout.h, must give back the standard-format tensors bit for
bit (the repack is a bijection), for every format and for stacked experts."""
import numpy as np
import pytest

import quantized_gemm_prepacked_amd as hq
import synth


def _a256(x):
    return (x + 255) // 256 * 256


def _regions(fam, asym, N, K):
    ku = 64 if fam == "w8a8" else 128
    units = (N // 16) * (K // ku)
    codes = units * 1024
    s_off = _a256(codes)
    s_bytes = {"wna16": units * 32, "w8a8": N * 4, "w4a8": units * 64}[fam]
    z_off = _a256(s_off + s_bytes)
    z_bytes = units * 8 if (fam == "wna16" and asym) else 0
    return ku, s_off, z_off, _a256(z_off + z_bytes)


def unpack_wna16(buf, N, K, asym):
    ku, s_off, z_off, _ = _regions("wna16", asym, N, K)
    nt_n, kt_n = N // 16, K // 128
    codes = np.zeros((N, K), np.uint8)
    units = buf[:nt_n * kt_n * 1024].reshape(nt_n, kt_n, 64, 4, 4)  # lane, dword, byte
    words = units.view(np.uint32).reshape(nt_n, kt_n, 64, 4)
    for p in range(8):                           # nibble slot p holds j = 2*(p&3) + (p>>2)
        j = 2 * (p & 3) + (p >> 2)
        nib = ((words >> (4 * p)) & 0xF).astype(np.uint8)      # [nt, kt, lane, d]
        for lane in range(64):
            n = np.arange(nt_n)[:, None] * 16 + (lane & 15)
            for d in range(4):
                k = np.arange(kt_n)[None, :] * 128 + 32 * (lane >> 4) + 8 * d + j
                codes[n, k] = nib[:, :, lane, d]
    if not asym:
        codes ^= 0x8
    wq = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    s = buf[s_off:s_off + nt_n * kt_n * 32].view(np.uint16).reshape(nt_n, kt_n, 16)
    scales = s.transpose(0, 2, 1).reshape(N, kt_n)
    zeros = None
    if asym:
        zb = buf[z_off:z_off + nt_n * kt_n * 8].reshape(nt_n, kt_n, 8)
        z = np.stack([zb & 0xF, zb >> 4], axis=-1).reshape(nt_n, kt_n, 16)
        zeros = z.transpose(0, 2, 1).reshape(N, kt_n).astype(np.uint8)
    return wq, scales, zeros


def unpack_w8a8(buf, N, K):
    ku, s_off, _, _ = _regions("w8a8", False, N, K)
    nt_n, kt_n = N // 16, K // 64
    u = buf[:nt_n * kt_n * 1024].reshape(nt_n, kt_n, 4, 16, 16)   # [nt, kt, l>>4, l&15, byte]
    wq = u.transpose(0, 3, 1, 2, 4).reshape(N, K).view(np.int8)
    s = buf[s_off:s_off + N * 4].view(np.float32)
    return wq, s


def unpack_w4a8(buf, N, K):
    ku, s_off, _, _ = _regions("w4a8", False, N, K)
    nt_n, kt_n = N // 16, K // 128
    u = buf[:nt_n * kt_n * 1024].reshape(nt_n, kt_n, 4, 16, 16)   # 16 bytes = one 32-block
    wq = u.transpose(0, 3, 1, 2, 4).reshape(N, K // 2)
    s = buf[s_off:s_off + nt_n * kt_n * 64].reshape(nt_n, kt_n, 4, 16)
    scales = s.transpose(0, 3, 1, 2).reshape(N, K // 32)
    return wq, scales


@pytest.mark.parametrize("asym", [False, True])
def test_wna16_roundtrip(asym):
    N, K = 48, 384
    d = synth.make_wna16(910 + asym, 2, N, K, asym=asym)
    desc = hq.DESC_W4A16_ASYM if asym else hq.DESC_W4A16_SYM
    out = np.zeros(hq.hq_prepacked_bytes(desc, 1, N, K), np.uint8)
    hq.hq_prepack_weights(desc, 1, N, K, d["wq"], d["scales"], d.get("zeros"), out)
    assert out.size == _regions("wna16", asym, N, K)[3]
    wq, s, z = unpack_wna16(out, N, K, asym)
    assert np.array_equal(wq, d["wq"]) and np.array_equal(s, d["scales"])
    if asym:
        assert np.array_equal(z, d["zeros"])


def test_w8a8_roundtrip():
    N, K = 32, 320
    d = synth.make_w8a8(911, 2, N, K)
    out = np.zeros(hq.hq_prepacked_bytes(hq.DESC_W8A8, 1, N, K), np.uint8)
    hq.hq_prepack_weights(hq.DESC_W8A8, 1, N, K, d["wq"], d["s_ch"], None, out)
    wq, s = unpack_w8a8(out, N, K)
    assert np.array_equal(wq, d["wq"]) and np.array_equal(s, d["s_ch"])


def test_w4a8_roundtrip():
    N, K = 32, 384
    d = synth.make_w4a8(912, 2, N, K)
    out = np.zeros(hq.hq_prepacked_bytes(hq.DESC_W4A8_MXFP4, 1, N, K), np.uint8)
    hq.hq_prepack_weights(hq.DESC_W4A8_MXFP4, 1, N, K, d["wq"], d["scales"], None, out)
    wq, s = unpack_w4a8(out, N, K)
    assert np.array_equal(wq, d["wq"]) and np.array_equal(s, d["scales"])


def test_stacked_experts_roundtrip():
    E, N, K = 3, 32, 256
    ws = [synth.make_moe_weights_expert(913, e, N, K) for e in range(E)]
    wq = np.stack([w["wq"] for w in ws])
    sc = np.stack([w["scales"] for w in ws])
    desc = hq.DESC_W4A16_SYM
    out = np.zeros(hq.hq_prepacked_bytes(desc, E, N, K), np.uint8)
    stride = out.size // E
    assert stride == hq.hq_prepacked_bytes(desc, 1, N, K) and stride % 256 == 0
    hq.hq_prepack_weights(desc, E, N, K, wq, sc, None, out)
    for e in range(E):
        w2, s2, _ = unpack_wna16(out[e * stride:(e + 1) * stride], N, K, False)
        assert np.array_equal(w2, ws[e]["wq"]) and np.array_equal(s2, ws[e]["scales"])


def test_prepacked_sizes_match_nominal_bytes():
    # codes + scales (+ 4-bit zeros) exactly, up to 256-byte region alignment
    N, K = 14336, 4096
    b = hq.hq_prepacked_bytes(hq.DESC_W4A16_ASYM, 1, N, K)
    nominal = N * K // 2 + N * (K // 128) * 2 + N * (K // 128) // 2
    assert nominal <= b < nominal + 3 * 256


def test_fp8_block_roundtrip():
    """Block-scaled FP8: codes in W8A8's 64-k units, then per (16-channel tile, 128-k step) the
    128 x 128 block's fp32 scale four times."""
    N, K = 256, 384
    d = synth.make_w8a8_fp8_block(914, 2, N, K)
    desc = hq.DESC_W8A8_FP8_BLOCK
    out = np.zeros(hq.hq_prepacked_bytes(desc, 1, N, K), np.uint8)
    hq.hq_prepack_weights(desc, 1, N, K, d["wq"], d["ws"], None, out)
    nt_n, G = N // 16, K // 128
    codes = nt_n * (K // 64) * 1024
    u = out[:codes].reshape(nt_n, K // 64, 4, 16, 16)
    assert np.array_equal(u.transpose(0, 3, 1, 2, 4).reshape(N, K), d["wq"])
    s_off = _a256(codes)
    s = out[s_off:s_off + nt_n * G * 16].view(np.float32).reshape(nt_n, G, 4)
    assert (s == s[:, :, :1]).all()
    assert np.array_equal(s[:, :, 0], d["ws"][np.arange(nt_n) * 16 // 128])
    assert out.size == _a256(s_off + nt_n * G * 16)


def test_mxfp4_weight_layout_is_shared_by_its_activation_formats():
    """W4A8, W4A4, MXFP8-activation W4A8 and bf16-activation W4A16 take the same MXFP4 weights."""
    N, K = 32, 256
    d = synth.make_w4a8(915, 1, N, K)
    outs = []
    for desc in (hq.DESC_W4A8_MXFP4, hq.DESC_W4A4_MXFP4, hq.DESC_W4A8_MXFP8, hq.DESC_W4A16_MXFP4):
        out = np.zeros(hq.hq_prepacked_bytes(desc, 1, N, K), np.uint8)
        hq.hq_prepack_weights(desc, 1, N, K, d["wq"], d["scales"], None, out)
        outs.append(out)
    assert all(np.array_equal(o, outs[0]) for o in outs)


def unpack_w8a16(buf, N, K):
    """8-bit codes for the bf16 MFMA: in 128-k step kt, 64-k unit j (0, 1), lane l, byte b holds
    k = 128 kt + 32 (l >> 4) + 16 j + b of channel 16 nt + (l & 15); fp32 scales [N] follow."""
    nt_n, u_n = N // 16, K // 64
    units = buf[:nt_n * u_n * 1024].reshape(nt_n, K // 128, 2, 4, 16, 16)   # nt, kt, j, g, c, b
    # -> [nt, c, kt, g, j, b] = channel 16 nt + c, k = 128 kt + 32 g + 16 j + b
    wq = units.transpose(0, 4, 1, 3, 2, 5).reshape(N, K)
    s_off = _a256(nt_n * u_n * 1024)
    return wq, buf[s_off:s_off + 4 * N].view(np.float32)


@pytest.mark.parametrize("fp8", [False, True])
def test_w8a16_roundtrip(fp8):
    N, K = 48, 384
    d = synth.make_w8a16(913, 2, N, K, fp8=fp8)
    desc = hq.DESC_W8A16_FP8 if fp8 else hq.DESC_W8A16_INT8
    out = np.zeros(hq.hq_prepacked_bytes(desc, 1, N, K), np.uint8)
    hq.hq_prepack_weights(desc, 1, N, K, d["wq"], d["s_ch"], None, out)
    wq, s = unpack_w8a16(out, N, K)
    assert np.array_equal(wq, d["wq"].view(np.uint8)) and np.array_equal(s, d["s_ch"])
    assert out.size == _a256(_a256((N // 16) * (K // 64) * 1024) + 4 * N)


def unpack_wna2(buf, N, K):
    """2-bit units of 16 channels x 128 k in 512 bytes: lane l holds two dwords, dword h holds
    k = 128 kt + 32 (l >> 4) + 16 h + c, code c = 2 s + e in bits 16 e + 2 s; then WNA16's scale
    and zero regions."""
    nt_n, kt_n = N // 16, K // 128
    d = buf[:nt_n * kt_n * 512].view(np.uint32).reshape(nt_n, kt_n, 4, 16, 2)   # nt, kt, g, ch, h
    codes = np.zeros((N, K), np.uint8)
    for c in range(16):
        s, e = c >> 1, c & 1
        v = ((d >> np.uint32(16 * e + 2 * s)) & np.uint32(3)).astype(np.uint8)     # nt, kt, g, ch, h
        # k = 128 kt + 32 g + 16 h + c of channel 16 nt + ch
        codes.reshape(nt_n, 16, kt_n, 4, 2, 16)[..., c] = v.transpose(0, 3, 1, 2, 4)
    wq = (codes[:, 0::4] | (codes[:, 1::4] << 2) | (codes[:, 2::4] << 4) | (codes[:, 3::4] << 6)).astype(np.uint8)
    s_off = _a256(nt_n * kt_n * 512)
    sc = buf[s_off:s_off + nt_n * kt_n * 32].view(np.uint16).reshape(nt_n, kt_n, 16)
    scales = sc.transpose(0, 2, 1).reshape(N, kt_n)
    z_off = _a256(s_off + nt_n * kt_n * 32)
    zb = buf[z_off:z_off + nt_n * kt_n * 8].reshape(nt_n, kt_n, 8)
    z = np.stack([zb & 0xF, zb >> 4], axis=-1).reshape(nt_n, kt_n, 16).transpose(0, 2, 1).reshape(N, kt_n)
    return wq, scales, z


def test_wna2_roundtrip():
    N, K = 48, 384
    d = synth.make_wna2(914, 2, N, K)
    out = np.zeros(hq.hq_prepacked_bytes(hq.DESC_W2A16_ASYM, 1, N, K), np.uint8)
    hq.hq_prepack_weights(hq.DESC_W2A16_ASYM, 1, N, K, d["wq"], d["scales"], d["zeros"], out)
    wq, s, z = unpack_wna2(out, N, K)
    assert np.array_equal(wq, d["wq"]) and np.array_equal(s, d["scales"]) and np.array_equal(z, d["zeros"])


def unpack_wna3(buf, N, K):
    """3-bit units of 16 channels x 128 k in 768 bytes: the low two bits as 2-bit codes (512
    bytes), then lane l's dword at 512 + 4 l holds the high bit of code c = 2s + e of dword h in
    bit 16 e + 8 h + s; WNA16's scale and zero regions follow."""
    nt_n, kt_n = N // 16, K // 128
    units = buf[:nt_n * kt_n * 768].reshape(nt_n, kt_n, 768)
    lo = np.ascontiguousarray(units[:, :, :512]).view(np.uint32).reshape(nt_n, kt_n, 4, 16, 2)   # nt, kt, g, ch, h
    hi = np.ascontiguousarray(units[:, :, 512:]).view(np.uint32).reshape(nt_n, kt_n, 4, 16)
    codes = np.zeros((N, K), np.uint8)
    for h in range(2):
        for c in range(16):
            s, e = c >> 1, c & 1
            v = ((lo[..., h] >> np.uint32(16 * e + 2 * s)) & np.uint32(3)) | \
                (((hi >> np.uint32(16 * e + 8 * h + s)) & np.uint32(1)) << np.uint32(2))
            codes.reshape(nt_n, 16, kt_n, 4, 2, 16)[:, :, :, :, h, c] = v.astype(np.uint8).transpose(0, 3, 1, 2)
    s_off = _a256(nt_n * kt_n * 768)
    sc = buf[s_off:s_off + nt_n * kt_n * 32].view(np.uint16).reshape(nt_n, kt_n, 16)
    scales = sc.transpose(0, 2, 1).reshape(N, kt_n)
    z_off = _a256(s_off + nt_n * kt_n * 32)
    zb = buf[z_off:z_off + nt_n * kt_n * 8].reshape(nt_n, kt_n, 8)
    z = np.stack([zb & 0xF, zb >> 4], axis=-1).reshape(nt_n, kt_n, 16).transpose(0, 2, 1).reshape(N, kt_n)
    return synth._pack_triplets(codes), scales, z


def test_wna3_roundtrip():
    N, K = 48, 384
    d = synth.make_wna3(915, 2, N, K)
    out = np.zeros(hq.hq_prepacked_bytes(hq.DESC_W3A16_ASYM, 1, N, K), np.uint8)
    hq.hq_prepack_weights(hq.DESC_W3A16_ASYM, 1, N, K, d["wq"], d["scales"], d["zeros"], out)
    wq, s, z = unpack_wna3(out, N, K)
    assert np.array_equal(wq, d["wq"]) and np.array_equal(s, d["scales"]) and np.array_equal(z, d["zeros"])
