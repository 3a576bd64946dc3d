"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each check is independent of the oracle's own code path:
  * block sizes and packed totals against figures printed on the pages
    (tests/golden/page_figures.txt);
  * dequantization against exact rational arithmetic (fractions.Fraction) on
    blocks built by encoders written here in the opposite direction (field ->
    byte position), with number formats decoded by numpy / torch;
  * the product against numpy's fp64 matmul, brute-force exact sums, one-hot
    activations and integer closed forms;
  * the routing generator against the closed form for expected distinct experts;
  * the MoE block's bf16 rounding against exact rational rounding and torch's
    fp32 -> bf16 conversion, the whole block against a pure-Python brute force
    on a tiny integer case, and its invariants (linearity in the routing
    weights, merged duplicate experts, order of a token's experts, E = 1
    reducing to two pinned products, invalid ids).
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.txt")


def page_figures():
    figs = {}
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = line.split()
            figs[k] = float(v) if "." in v else int(v)
    return figs


# ---------------------------------------------------------------- encoders (field -> bytes)

def f16_bits(v):
    return int(np.array(v, dtype=np.float16).view(np.uint16))


def f16_value(bits):
    return Fraction(float(np.array(bits, dtype=np.uint16).view(np.float16)))


def e4m3_value(byte):
    t = torch.tensor([byte], dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float32)
    v = float(t[0])
    return v if math.isnan(v) else Fraction(v)


E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]  # the format's eight magnitudes


def e2m1_value(c):
    v = Fraction(E2M1[c & 7])
    return -v if c & 8 else v


def rn32(fr):
    """Round an exact rational once to fp32 (it must be exact in fp64 first)."""
    d = float(fr)
    assert Fraction(d) == fr, "value not exact in fp64"
    return np.float32(d)


def enc_q8_0(d_bits, q):
    b = bytearray(34)
    b[0:2] = d_bits.to_bytes(2, "little")
    for i in range(32):
        b[2 + i] = q[i] & 0xFF
    return bytes(b)


def enc_q4_k(d_bits, dmin_bits, sc, mn, q):
    """sc, mn: 8 six-bit values; q: 256 nibbles in value order."""
    b = bytearray(144)
    b[0:2] = d_bits.to_bytes(2, "little")
    b[2:4] = dmin_bits.to_bytes(2, "little")
    S = [0] * 12
    for j in range(4):
        S[j] |= sc[j] & 63
        S[j + 4] |= mn[j] & 63
    for j in range(4, 8):
        S[j + 4] |= (sc[j] & 15) | ((mn[j] & 15) << 4)
        S[j - 4] |= (sc[j] >> 4) << 6
        S[j] |= (mn[j] >> 4) << 6
    b[4:16] = bytes(S)
    for g in range(4):
        for l in range(32):
            b[16 + 32 * g + l] = (q[64 * g + l] & 15) | ((q[64 * g + 32 + l] & 15) << 4)
    return bytes(b)


def enc_q5_k(d_bits, dmin_bits, sc, mn, q):
    """sc, mn: 8 six-bit values; q: 256 five-bit codes in value order.  The low
    four bits go where Q4_K keeps its nibbles (28 bytes further on); bit 4 of
    the code of sub-block j, position l is bit j of byte 16 + l."""
    b = bytearray(enc_q4_k(d_bits, dmin_bits, sc, mn, [v & 15 for v in q]))
    nib = bytes(b[16:144])
    b = bytearray(176)
    b[0:16] = enc_q4_k(d_bits, dmin_bits, sc, mn, [0] * 256)[0:16]
    b[48:176] = nib
    for j in range(8):
        for l in range(32):
            b[16 + l] |= ((q[32 * j + l] >> 4) & 1) << j
    return bytes(b)


def enc_q6_k(d_bits, s, q):
    """s: 16 int8 sub-scales; q: 256 six-bit codes in value order."""
    b = bytearray(210)
    for h in range(2):
        for l in range(32):
            v0, v1, v2, v3 = (q[128 * h + 32 * t + l] for t in range(4))
            b[64 * h + l] = (v0 & 15) | ((v2 & 15) << 4)
            b[64 * h + 32 + l] = (v1 & 15) | ((v3 & 15) << 4)
            b[128 + 32 * h + l] = (v0 >> 4) | ((v1 >> 4) << 2) | ((v2 >> 4) << 4) | ((v3 >> 4) << 6)
    for i in range(16):
        b[192 + i] = s[i] & 0xFF
    b[208:210] = d_bits.to_bytes(2, "little")
    return bytes(b)


def enc_nvfp4(codes, scales, gvals):
    """codes: [R][K] nibbles; scales: [R][K/16] bytes; gvals: E fp32 values."""
    R, K = len(codes), len(codes[0])
    cb = bytearray(R * K // 2)
    for r in range(R):
        for k in range(0, K, 2):
            cb[r * K // 2 + k // 2] = (codes[r][k] & 15) | ((codes[r][k + 1] & 15) << 4)
    sb = bytes(s for row in scales for s in row)
    gb = np.array(gvals, dtype=np.float32).tobytes()
    return np.frombuffer(bytes(cb) + sb + gb, dtype=np.uint8)


def as_u8(bs):
    return np.frombuffer(bs, dtype=np.uint8)


def same_values(got, exp):
    """Equal as real numbers (+0 == -0, the exact rational has no signed zero); nonzero signs agree."""
    got, exp = np.asarray(got, np.float32), np.asarray(exp, np.float32)
    return got.shape == exp.shape and bool(np.all(got == exp))


# ---------------------------------------------------------------- sizes against the pages

def test_block_sizes_match_pages():
    f = page_figures()
    assert oracle.block_bytes(oracle.Q8_0) == f["q8_0_block_bytes"]
    assert oracle.block_bytes(oracle.Q6_K) == f["q6_k_block_bytes"]
    assert -(-oracle.block_bytes(oracle.Q8_0) // 4) == f["q8_0_block_words"]
    assert -(-oracle.block_bytes(oracle.Q6_K) // 4) == f["q6_k_block_words"]
    # Q4_K: 2 + 2 + 12 + 128 bytes; Q5_K adds one bit per value (32 bytes);
    # NVFP4: 8 code bytes + 1 scale byte per 16 values
    assert oracle.block_bytes(oracle.Q4_K) == 2 + 2 + 12 + 256 // 2
    assert oracle.block_bytes(oracle.Q5_K) == 2 + 2 + 12 + 256 // 8 + 256 // 2
    assert oracle.block_bytes(oracle.NVFP4) == 16 // 2 + 1
    assert [oracle.block_values(t) for t in (1, 2, 3, 4, 5)] == [32, 256, 256, 16, 256]


def test_packed_totals_match_pages():
    f = page_figures()
    K, N = f["output_head_k"], f["output_head_n"]
    head = oracle.packed_bytes(oracle.Q6_K, 1, N, K)
    assert head == 1_042_944_000
    assert round(head / 2**30, 2) == f["output_head_q6_k_gib_2dp"]
    assert round(2 * N * K / 2**30, 2) == f["output_head_bf16_gib_2dp"]
    # the routed-expert parameter count of the 288-expert model
    params = f["glm_sparse_layers"] * f["glm_experts"] * f["glm_expert_matrices"] * \
        f["glm_expert_rows"] * f["glm_expert_cols"]
    assert params == f["glm_routed_expert_params"]
    # one such layer in Q4_K, stacked as weight[E*N, K]: gate and up [288*2048, 4096], down [288*4096, 2048]
    E = f["glm_experts"]
    layer = 2 * oracle.packed_bytes(oracle.Q4_K, E, 2048, 4096) + oracle.packed_bytes(oracle.Q4_K, E, 4096, 2048)
    assert layer == E * 3 * 4096 * 2048 * 144 // 256 == 4_076_863_488
    # NVFP4 at the MLP shape: codes + scales + one fp32 tensor scale
    assert oracle.packed_bytes(oracle.NVFP4, 1, f["qwen27b_mlp"], f["qwen27b_hidden"]) == \
        17408 * 5120 // 2 + 17408 * 5120 // 16 + 4 == 50_135_044
    assert oracle.packed_bytes(oracle.Q4_K, 1, 2 * 17408, 5120) == 100_270_080


def test_packed_bytes_rejects():
    assert oracle.packed_bytes(oracle.Q4_K, 1, 4, 100) == 0
    assert oracle.packed_bytes(9, 1, 4, 256) == 0
    assert oracle.packed_bytes(oracle.NVFP4, 1, 4, 24) == 0
    assert oracle.packed_bytes(oracle.Q8_0, 1, 0, 64) == 0
    assert oracle.packed_bytes(oracle.FP8, 1, 4, 96) == 0  # K not a multiple of 64
    # FP8: one byte per value plus one fp32 scale per row
    assert oracle.packed_bytes(oracle.FP8, 3, 5, 128) == 15 * 128 + 15 * 4


# ---------------------------------------------------------------- number formats

def test_fp16_decode_all_codes():
    """Every finite fp16 pattern as a Q8_0 scale with q = 1 gives w = d, against numpy's decode."""
    codes = [c for c in range(65536) if (c >> 10) & 31 != 31]
    blocks = b"".join(enc_q8_0(c, [1] + [0] * 31) for c in codes)
    w = oracle.dequant_rows(oracle.Q8_0, as_u8(blocks), 1, len(codes), 32)
    ref = np.array(codes, dtype=np.uint16).view(np.float16).astype(np.float32)
    assert np.array_equal(w[:, 0].view(np.uint32), ref.view(np.uint32))  # also -0.0
    assert not w[:, 1:].any()


def test_e4m3_and_e2m1_decode_all_codes():
    """NVFP4 with g = 1: code 2 (1.0) exposes the block scale; scale 0x38 (1.0) exposes the code."""
    K = 16
    rows_s = list(range(256))
    codes = [[2] * K for _ in rows_s]
    scales = [[s] for s in rows_s]
    w = oracle.dequant_rows(oracle.NVFP4, enc_nvfp4(codes, scales, [1.0]), 1, 256, K)
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(w[:, 0]), nan) and nan.sum() == 2
    assert np.array_equal(w[~nan, 0].view(np.uint32), ref[~nan].view(np.uint32))
    assert float(w[0x7E, 0]) == 448.0 and float(w[1, 0]) == 2.0 ** -9
    w2 = oracle.dequant_rows(oracle.NVFP4, enc_nvfp4([list(range(16))], [[0x38]], [1.0]), 1, 1, K)
    expect = np.array([-E2M1[c & 7] if c & 8 else E2M1[c & 7] for c in range(16)], dtype=np.float32)
    assert np.array_equal(w2[0].view(np.uint32), expect.view(np.uint32))  # code 8 is -0.0
    assert np.signbit(w2[0, 8])


# ---------------------------------------------------------------- dequantization, exact

def _rand_f16_bits(g, special):
    if special == "zero":
        return 0
    if special == "sub":
        return int(g.integers(1, 1024))
    if special == "max":
        return 0x7BFF  # 65504
    if special == "neg":
        return f16_bits(-abs(g.standard_normal()) * 0.01)
    return f16_bits(abs(g.standard_normal()) * 0.01 + 1e-4)


SPECIALS = [None, None, None, "zero", "sub", "max", "neg"]


def test_q8_0_exact():
    g = np.random.default_rng(11)
    blocks, expect = [], []
    for i in range(40):
        db = _rand_f16_bits(g, SPECIALS[i % len(SPECIALS)])
        q = [int(v) for v in g.integers(-128, 128, 32)]
        blocks.append(enc_q8_0(db, q))
        d = f16_value(db)
        expect.extend(rn32(d * qi) for qi in q)
    w = oracle.dequant_rows(oracle.Q8_0, as_u8(b"".join(blocks)), 1, 40, 32)
    assert same_values(w.reshape(-1), np.array(expect, np.float32))


def test_q4_k_exact():
    g = np.random.default_rng(12)
    nb = 28
    blocks, expect = [], []
    for i in range(nb):
        db = _rand_f16_bits(g, SPECIALS[i % len(SPECIALS)])
        mb = _rand_f16_bits(g, SPECIALS[(i // 2) % len(SPECIALS)])
        sc = [int(v) for v in g.integers(0, 64, 8)]
        mn = [int(v) for v in g.integers(0, 64, 8)]
        if i == 1:
            sc, mn = [63] * 8, [63] * 8
        q = [int(v) for v in g.integers(0, 16, 256)]
        blocks.append(enc_q4_k(db, mb, sc, mn, q))
        d, dmin = f16_value(db), f16_value(mb)
        for v in range(256):
            j = v // 32
            expect.append(rn32(d * sc[j] * q[v] - dmin * mn[j]))
    w = oracle.dequant_rows(oracle.Q4_K, as_u8(b"".join(blocks)), 1, nb, 256)
    assert same_values(w.reshape(-1), np.array(expect, np.float32))


def test_q4_k_scale_layout_every_code():
    """All 64x64 (scale, min) pairs through every sub-block position."""
    blocks, expect = [], []
    one = f16_bits(1.0)
    q = [(v * 7) % 16 for v in range(256)]
    for a in range(64):
        for j0 in range(0, 64, 8):
            sc = [(a + 5 * j) % 64 for j in range(8)]
            mn = [(j0 + j * 9 + a) % 64 for j in range(8)]
            blocks.append(enc_q4_k(one, one, sc, mn, q))
            expect.extend(float(sc[v // 32] * q[v] - mn[v // 32]) for v in range(256))
    w = oracle.dequant_rows(oracle.Q4_K, as_u8(b"".join(blocks)), 1, len(blocks), 256)
    assert np.array_equal(w.reshape(-1), np.array(expect, np.float32))


def test_q5_k_exact():
    g = np.random.default_rng(15)
    nb = 28
    blocks, expect = [], []
    for i in range(nb):
        db = _rand_f16_bits(g, SPECIALS[i % len(SPECIALS)])
        mb = _rand_f16_bits(g, SPECIALS[(i // 2) % len(SPECIALS)])
        sc = [int(v) for v in g.integers(0, 64, 8)]
        mn = [int(v) for v in g.integers(0, 64, 8)]
        if i == 1:
            sc, mn = [63] * 8, [63] * 8
        q = [int(v) for v in g.integers(0, 32, 256)]
        if i == 2:
            q = [31, 16] * 128
        blocks.append(enc_q5_k(db, mb, sc, mn, q))
        d, dmin = f16_value(db), f16_value(mb)
        for v in range(256):
            j = v // 32
            expect.append(rn32(d * sc[j] * q[v] - dmin * mn[j]))
    w = oracle.dequant_rows(oracle.Q5_K, as_u8(b"".join(blocks)), 1, nb, 256)
    assert same_values(w.reshape(-1), np.array(expect, np.float32))


def test_q5_k_fifth_bit_every_position():
    """A code of 16 (only the fifth bit set) at each of the 256 positions in turn,
    with d = sc = 1 and no min: the dequantized block is 16 at that position only."""
    one = f16_bits(1.0)
    blocks = []
    for v in range(256):
        q = [0] * 256
        q[v] = 16
        blocks.append(enc_q5_k(one, one, [1] * 8, [0] * 8, q))
    w = oracle.dequant_rows(oracle.Q5_K, as_u8(b"".join(blocks)), 1, 256, 256)
    assert np.array_equal(w, 16.0 * np.eye(256, dtype=np.float32))


def test_q6_k_exact():
    g = np.random.default_rng(13)
    nb = 21
    blocks, expect = [], []
    for i in range(nb):
        db = _rand_f16_bits(g, SPECIALS[i % len(SPECIALS)])
        s = [int(v) for v in g.integers(-128, 128, 16)]
        if i == 2:
            s = [-128] * 16
        q = [int(v) for v in g.integers(0, 64, 256)]
        if i == 3:
            q = [0, 63] * 128
        blocks.append(enc_q6_k(db, s, q))
        d = f16_value(db)
        expect.extend(rn32(d * s[v // 16] * (q[v] - 32)) for v in range(256))
    w = oracle.dequant_rows(oracle.Q6_K, as_u8(b"".join(blocks)), 1, nb, 256)
    assert same_values(w.reshape(-1), np.array(expect, np.float32))


def test_nvfp4_exact_and_order():
    """w = RN32(e2m1 * e4m3 * g) rounded once; the order c * RN32(s * g) is not equivalent."""
    g = np.random.default_rng(14)
    E, N, K = 2, 5, 64
    R = E * N
    codes = [[int(v) for v in g.integers(0, 16, K)] for _ in range(R)]
    scales = [[int(v) for v in g.integers(0, 0x7F, K // 16)] for _ in range(R)]
    scales[0] = [0x01, 0x07, 0x7E, 0x00]  # subnormals, max 448, zero
    gvals = [float(np.float32(0.01 * (1 + g.random()))) for _ in range(E)]
    w = oracle.dequant_rows(oracle.NVFP4, enc_nvfp4(codes, scales, gvals), E, N, K)
    differ = 0
    for r in range(R):
        gv = Fraction(gvals[r // N])
        for k in range(K):
            c = e2m1_value(codes[r][k])
            s = e4m3_value(scales[r][k // 16])
            exact = rn32(c * s * gv)
            assert same_values(w[r, k:k + 1], np.array([exact], np.float32)), (r, k)
            alt = np.float32(float(c)) * np.float32(float(s) * gvals[r // N])
            differ += alt != exact
    assert differ > 0


def enc_fp8(codes, scales):
    """Planes [codes R x K][R fp32 row scales], written field by field."""
    b = bytearray()
    for row in codes:
        b += bytes(row)
    for sc in scales:
        b += np.float32(sc).tobytes()
    return as_u8(bytes(b))


def test_fp8_exact_every_code():
    """w = RN32(e4m3(c) * s), one rounding; all 256 codes (NaN codes give NaN)
    under several scales, including subnormal, negative and zero scales."""
    K = 256
    scale_list = [1.0, 0.0123456789, -3.5e-3, 1.4e-45, 2.0**-130, 0.0, 3.3e38]
    codes = [list(range(256)) for _ in scale_list]
    w = oracle.dequant_rows(oracle.FP8, enc_fp8(codes, scale_list), 1, len(scale_list), K)
    for r, sc in enumerate(scale_list):
        sv = Fraction(float(np.float32(sc)))
        for c in range(256):
            v = e4m3_value(c)
            if isinstance(v, float):  # NaN
                assert np.isnan(w[r, c]), (r, c)
                continue
            exact = v * sv
            big = abs(exact) >= Fraction(2) ** 128
            exp32 = np.float32(np.inf if exact > 0 else -np.inf) if big else rn32(exact)
            assert same_values(w[r, c:c + 1], np.array([exp32], np.float32)), (r, c, sc)
    # stacked rows take their own scales
    wr = oracle.dequant_rows(oracle.FP8, enc_fp8([[0x38] * 64, [0x38] * 64], [2.0, -0.5]), 1, 2, 64)
    assert (wr[0] == 2.0).all() and (wr[1] == -0.5).all()  # 0x38 = 1.0


def test_generator_fields_in_range():
    g = synth.rng(1, 0)
    w = synth.weights(synth.Q8_0, g, 64, 1024).reshape(-1, 34)
    q = w[:, 2:].view(np.int8)
    assert q.min() >= -127 and q.max() <= 127
    d = w[:, 0:2].copy().view(np.float16).astype(np.float64)
    assert (d >= 0).all() and 0.004 < d.mean() < 0.012
    w4 = synth.weights(synth.Q4_K, synth.rng(2, 0), 16, 512).reshape(-1, 144)
    d4 = w4[:, 0:2].copy().view(np.float16).astype(np.float64)
    assert (d4 >= 0.005 - 1e-6).all() and (d4 <= 0.015 + 1e-5).all()
    w5 = synth.weights(synth.Q5_K, synth.rng(6, 0), 16, 512)
    assert w5.size == oracle.packed_bytes(oracle.Q5_K, 1, 16, 512)
    d5 = w5.reshape(-1, 176)[:, 0:4].copy().view(np.float16).astype(np.float64)
    assert (d5 >= 0.005 - 1e-6).all() and (d5 <= 0.015 + 1e-5).all()
    nv = synth.weights(synth.NVFP4, synth.rng(4, 0), 32, 256)
    assert nv.size == oracle.packed_bytes(oracle.NVFP4, 1, 32, 256)
    gsc = nv[-4:].view(np.float32)[0]
    assert 0.01 <= gsc <= 0.02
    f8 = synth.weights(synth.FP8, synth.rng(7, 0), 40, 512)
    assert f8.size == oracle.packed_bytes(oracle.FP8, 1, 40, 512)
    codes = f8[:40 * 512]
    assert not ((codes & 0x7F) == 0x7F).any() and len(np.unique(codes)) == 254
    rs = f8[40 * 512:].view(np.float32)
    assert (rs > 0.005 / 448 - 1e-9).all() and (rs < 0.015 / 448 + 1e-9).all()


# ---------------------------------------------------------------- the product

def _bf16_to_f64(xb):
    return (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("fmt,K", [(1, 1024), (2, 1024), (3, 768), (4, 512), (5, 768), (6, 512)])
def test_gemm_matches_numpy_fp64(fmt, K):
    N, M = 67, 3
    w = synth.weights(fmt, synth.rng(5, 0), N, K)
    x = synth.x_bf16(synth.rng(5, 1), M, K)
    y, b = oracle.gemm(fmt, w, N, K, x)
    W = oracle.dequant_rows(fmt, w, 1, N, K).astype(np.float64)
    X = _bf16_to_f64(x)
    yn = X @ W.T
    bn = np.abs(X) @ np.abs(W).T
    assert np.all(np.abs(y - yn) <= 1e-12 * bn)
    assert np.allclose(b, bn, rtol=1e-12, atol=0)
    assert np.all(np.abs(y) <= b)


def test_gemm_brute_force_exact_tiny():
    fmt, N, K, M = oracle.Q4_K, 3, 256, 2
    w = synth.weights(fmt, synth.rng(6, 0), N, K)
    x = synth.x_bf16(synth.rng(6, 1), M, K)
    y, b = oracle.gemm(fmt, w, N, K, x)
    W = oracle.dequant_rows(fmt, w, 1, N, K)
    X = _bf16_to_f64(x)
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(float(W[n, k])) * Fraction(float(X[m, k])) for k in range(K))
            absum = sum(abs(Fraction(float(W[n, k])) * Fraction(float(X[m, k]))) for k in range(K))
            assert abs(Fraction(y[m, n]) - exact) <= Fraction(K, 2**53) * absum
            assert abs(Fraction(b[m, n]) - absum) <= Fraction(K, 2**53) * absum


def test_gemm_one_hot_and_integer_sums():
    # one-hot x picks one dequantized column bit for bit
    fmt, N, K = oracle.Q6_K, 9, 512
    w = synth.weights(fmt, synth.rng(7, 0), N, K)
    W = oracle.dequant_rows(fmt, w, 1, N, K)
    for k in (0, 1, 255, 256, 511):
        x = np.zeros((1, K), np.uint16)
        x[0, k] = 0x3F80  # bf16 1.0
        y, _ = oracle.gemm(fmt, w, N, K, x)
        assert np.array_equal(y[0].astype(np.float32), W[:, k])
    # Q8_0 with d = 1 and x = 1: y is the integer sum of the codes
    g = np.random.default_rng(3)
    qs = [[int(v) for v in g.integers(-128, 128, 32)] for _ in range(8)]
    one = f16_bits(1.0)
    wq = as_u8(b"".join(enc_q8_0(one, q) for q in qs))
    y, _ = oracle.gemm(oracle.Q8_0, wq, 2, 128, np.full((1, 128), 0x3F80, np.uint16))
    assert y[0, 0] == sum(map(sum, qs[:4])) and y[0, 1] == sum(map(sum, qs[4:]))
    # Q4_K with d = dmin = sc = 1, m = 0, x = 1: y = sum of the nibbles
    q = [int(v) for v in g.integers(0, 16, 256)]
    w4 = as_u8(enc_q4_k(one, one, [1] * 8, [0] * 8, q))
    y, b = oracle.gemm(oracle.Q4_K, w4, 1, 256, np.full((1, 256), 0x3F80, np.uint16))
    assert y[0, 0] == sum(q) == b[0, 0]
    # Q5_K likewise: y = sum of the five-bit codes
    q5 = [int(v) for v in g.integers(0, 32, 256)]
    w5 = as_u8(enc_q5_k(one, one, [1] * 8, [0] * 8, q5))
    y, b = oracle.gemm(oracle.Q5_K, w5, 1, 256, np.full((1, 256), 0x3F80, np.uint16))
    assert y[0, 0] == sum(q5) == b[0, 0]
    # x = 0: y = 0 and bound = 0
    y, b = oracle.gemm(oracle.Q4_K, w4, 1, 256, np.zeros((1, 256), np.uint16))
    assert y[0, 0] == 0 and b[0, 0] == 0


def test_grouped_equals_per_expert_dense():
    fmt, E, N, K = oracle.Q4_K, 4, 6, 512
    w = synth.weights(fmt, synth.rng(8, 0), E * N, K)
    x = synth.x_bf16(synth.rng(8, 1), 5, K)
    ids = np.array([3, 0, 3, 1, 7], np.int32)  # 7 is out of range
    y, b = oracle.gemm(fmt, w, N, K, x, E=E, ids=ids)
    ebytes = oracle.packed_bytes(fmt, 1, N, K)
    for m, e in enumerate(ids):
        if e >= E:
            assert np.isnan(y[m]).all() and np.isnan(b[m]).all()
            continue
        yd, bd = oracle.gemm(fmt, w[e * ebytes:(e + 1) * ebytes], N, K, x[m:m + 1])
        assert np.array_equal(y[m], yd[0]) and np.array_equal(b[m], bd[0])
    # E = 1 with ids = None is the dense product; selected columns agree with the full result
    yd, _ = oracle.gemm(fmt, w[:ebytes], N, K, x)
    y1, _ = oracle.gemm(fmt, w[:ebytes], N, K, x, E=1, ids=np.zeros(5, np.int32))
    ys, _ = oracle.gemm(fmt, w[:ebytes], N, K, x, cols=[5, 0, 2])
    assert np.array_equal(yd, y1) and np.array_equal(ys, yd[:, [5, 0, 2]])


def test_grouped_nvfp4_uses_each_experts_tensor_scale():
    E, N, K = 3, 4, 32
    w = synth.weights(oracle.NVFP4, synth.rng(9, 0), E * N, K, E=E)
    W = oracle.dequant_rows(oracle.NVFP4, w, E, N, K)
    gs = w[-4 * E:].view(np.float32)
    # zero the per-tensor scale of expert 1 only: its rows vanish, the others stay
    w2 = w.copy()
    w2[-4 * E + 4:-4 * E + 8] = 0
    W2 = oracle.dequant_rows(oracle.NVFP4, w2, E, N, K)
    assert not W2[N:2 * N].any() and np.array_equal(W2[:N], W[:N]) and np.array_equal(W2[2 * N:], W[2 * N:])
    assert gs.shape == (3,)


# ---------------------------------------------------------------- the routing generator

def test_routing_distinct_experts_closed_form():
    f = page_figures()
    E, k = f["glm_experts"], f["distinct_topk"]

    def expected(T):
        return E * (1 - (1 - k / E) ** T)

    assert round(expected(f["distinct_tokens"]), 1) == f["distinct_experts_expected_1dp"]
    assert f["distinct_tokens"] * k == f["distinct_pairs"]
    for T, trials in ((3, 3000), (16, 1500)):
        counts = []
        for s in range(trials):
            ids = synth.routing(synth.rng(1000 + s, 2), T, k, E)
            assert ids.min() >= 0 and ids.max() < E
            per = ids.reshape(T, k)
            assert all(len(set(r)) == k for r in per)
            counts.append(len(set(ids.tolist())))
        mean = float(np.mean(counts))
        sem = float(np.std(counts)) / math.sqrt(trials)
        assert abs(mean - expected(T)) < 4 * sem + 0.02, (T, mean, expected(T))
    assert abs(expected(16) - 104.50) < 0.01


# ---------------------------------------------------------------- the MoE block

def _rne_bf16_exact(fr):
    """bf16 bits of an exact rational, rounded to nearest even (normal range only)."""
    if fr == 0:
        return 0
    sign = 0x8000 if fr < 0 else 0
    a = abs(fr)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    # a in [1, 2): 7 fraction bits
    scaled = a * 128
    q = int(scaled)
    rem = scaled - q
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and q % 2 == 1):
        q += 1
    if q == 256:
        q = 128
        e += 1
    return sign | ((e + 127) << 7) | (q - 128)


def test_round_bf16_exact_rational_and_torch():
    g = np.random.default_rng(11)
    # fp64 values that are not fp32 values: one rounding from fp64, checked exactly
    v = g.standard_normal(4000) * np.exp2(g.integers(-20, 20, 4000))
    v = np.concatenate([v, [1 + 2.0**-8 + 2.0**-40, 1 + 2.0**-8, 1 + 3 * 2.0**-8, -(1 + 2.0**-8 + 2.0**-40),
                            255.5, 256.5, 0.1, -0.1]])
    got = oracle.round_bf16(v)
    exp = np.array([_rne_bf16_exact(Fraction(float(t))) for t in v], np.uint16)
    assert np.array_equal(got, exp)
    assert got[-8] == 0x3F81 and got[-7] == 0x3F80 and got[-6] == 0x3F82  # above a tie; ties to even
    # fp32 values (exact in fp64): torch's fp32 -> bf16 conversion, specials included
    f = (g.standard_normal(20000) * np.exp2(g.integers(-140, 127, 20000))).astype(np.float32)
    ties = ((g.integers(0, 1 << 15, 2000).astype(np.uint32) << 16) | 0x8000).astype(np.uint32).view(np.float32)
    f = np.concatenate([f, ties[np.isfinite(ties)], np.float32([0.0, -0.0, np.inf, -np.inf, 3.4e38, -3.39e38,
                                                               1e-40, -1e-45, 1.17e-38])])
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.round_bf16(f.astype(np.float64)), ref)
    assert oracle.round_bf16(np.array([np.nan]))[0] == 0x7FC0


def test_moe_block_brute_force_tiny():
    """Q8_0 experts with d = 1 and small integer codes, small integer activations:
    the block computed by hand (Python integers, exact rational rounding)."""
    E, D, F, T, topk = 3, 64, 32, 2, 2
    g = np.random.default_rng(12)
    one = f16_bits(1.0)
    qgu = g.integers(-3, 4, (E * 2 * F, D))
    qdn = g.integers(-3, 4, (E * D, F))
    w_gu = as_u8(b"".join(enc_q8_0(one, [int(v) for v in row[b * 32:(b + 1) * 32]])
                          for row in qgu for b in range(D // 32)))
    w_dn = as_u8(b"".join(enc_q8_0(one, [int(v) for v in row[b * 32:(b + 1) * 32]])
                          for row in qdn for b in range(F // 32)))
    xi = g.integers(-2, 3, (T, D))
    x = np.array([[f16_to_bf16_bits(float(v)) for v in r] for r in xi], np.uint16)
    idx = np.array([[2, 0], [1, 1]], np.int32)
    wts = np.array([[0.75, 0.25], [0.5, -1.5]], np.float32)
    y, b, h = oracle.moe_block(oracle.Q8_0, w_gu, oracle.Q8_0, w_dn, E, D, F, x, idx, wts, want_h=True)
    for t in range(T):
        acc = Fraction(0)
        hs = []
        for j in range(topk):
            e = int(idx[t, j])
            gv = [int(sum(int(qgu[e * 2 * F + f, k]) * int(xi[t, k]) for k in range(D))) for f in range(F)]
            uv = [int(sum(int(qgu[e * 2 * F + F + f, k]) * int(xi[t, k]) for k in range(D))) for f in range(F)]
            vs = [gg / (1.0 + math.exp(-gg)) * uu for gg, uu in zip(gv, uv)]
            # (IEEE sign of zero: a negative silu times u = 0 is -0)
            hb = [(0x8000 if math.copysign(1.0, v) < 0 else 0) if v == 0 else _rne_bf16_exact(Fraction(v))
                  for v in vs]
            assert list(h[t * topk + j]) == hb
            hs.append(hb)
        for d in range(D):
            s = Fraction(0)
            for j in range(topk):
                e = int(idx[t, j])
                hv = [Fraction(float(np.uint32(v << 16).view(np.float32))) for v in hs[j]]
                s += Fraction(float(wts[t, j])) * sum(int(qdn[e * D + d, f]) * hv[f] for f in range(F))
            assert abs(Fraction(y[t, d]) - s) <= Fraction(1, 2**40) * (abs(s) + 1), (t, d)
    assert np.all(np.abs(y) <= b)


def f16_to_bf16_bits(v):
    return int(np.float32(v).view(np.uint32) >> 16)


def _moe_case(fmt_gu, fmt_dn, E, D, F, T, topk, seed):
    w_gu = synth.weights(fmt_gu, synth.rng(seed, 0), E * 2 * F, D, E=E)
    w_dn = synth.weights(fmt_dn, synth.rng(seed, 1), E * D, F, E=E)
    x = synth.x_bf16(synth.rng(seed, 2), T, D)
    idx = synth.routing(synth.rng(seed, 3), T, topk, E).reshape(T, topk)
    wts = synth.routing_weights(synth.rng(seed, 4), T, topk)
    return w_gu, w_dn, x, idx, wts


def test_moe_block_invariants():
    fg, fd, E, D, F, T, topk = oracle.Q4_K, oracle.Q6_K, 5, 256, 512, 4, 3
    w_gu, w_dn, x, idx, wts = _moe_case(fg, fd, E, D, F, T, topk, 13)
    y, b, h = oracle.moe_block(fg, w_gu, fd, w_dn, E, D, F, x, idx, wts, want_h=True)
    # linear in the routing weights (doubling is exact in fp64)
    y2, b2 = oracle.moe_block(fg, w_gu, fd, w_dn, E, D, F, x, idx, 2 * wts)
    assert np.array_equal(y2, 2 * y) and np.array_equal(b2, 2 * b)
    # the order of a token's experts does not matter (up to fp64 rounding)
    yr, _ = oracle.moe_block(fg, w_gu, fd, w_dn, E, D, F, x, idx[:, ::-1], wts[:, ::-1])
    assert np.all(np.abs(yr - y) <= 1e-12 * b)
    # a duplicated expert equals one expert with the summed weight
    idx_d = np.stack([idx[:, 0], idx[:, 0]], 1)
    wts_d = (np.round(wts[:, :2] * 64) / 64).astype(np.float32)  # multiples of 1/64: sums are exact
    yd, bd = oracle.moe_block(fg, w_gu, fd, w_dn, E, D, F, x, idx_d, wts_d)
    ys, _ = oracle.moe_block(fg, w_gu, fd, w_dn, E, D, F, x, idx[:, :1], wts_d.sum(axis=1, keepdims=True))
    assert np.all(np.abs(yd - ys) <= 1e-12 * bd)
    # each pair's intermediate and down product are the two pinned products
    for t in range(T):
        for j in range(topk):
            e = int(idx[t, j])
            gu, _ = oracle.gemm(fg, w_gu, 2 * F, D, x[t:t + 1], E=E, ids=np.array([e], np.int32))
            gg, uu = gu[0, :F], gu[0, F:]
            with np.errstate(over="ignore"):
                v = gg / (1.0 + np.exp(-gg)) * uu
            hb = oracle.round_bf16(v)
            # numpy's exp may differ from libm's in the last bit: allow a different
            # rounding only where v sits within 1e-12 of a bf16 midpoint
            mid = np.abs(v) * 2.0**-8
            near = np.abs(np.abs(v) / mid - np.round(np.abs(v) / mid)) < 1e-9
            diff = hb != h[t * topk + j]
            assert not np.any(diff & ~near)
    hx = h[: topk].copy()  # token 0's intermediates as activations of the down product
    for j in range(topk):
        e = int(idx[0, j])
        yd_j, bd_j = oracle.gemm(fd, w_dn, D, F, hx[j:j + 1], E=E, ids=np.array([e], np.int32))
        if j == 0:
            acc = wts[0, j].astype(np.float64) * yd_j[0]
            accb = abs(wts[0, j].astype(np.float64)) * bd_j[0]
        else:
            acc = acc + wts[0, j].astype(np.float64) * yd_j[0]
            accb = accb + abs(wts[0, j].astype(np.float64)) * bd_j[0]
    assert np.all(np.abs(acc - y[0]) <= 1e-12 * b[0]) and np.allclose(accb, b[0], rtol=1e-12, atol=0)
    # an id outside [0, E) makes that token's row NaN, and only that row
    idx_bad = idx.copy()
    idx_bad[2, 1] = E
    yb, bb = oracle.moe_block(fg, w_gu, fd, w_dn, E, D, F, x, idx_bad, wts)
    assert np.isnan(yb[2]).all() and np.isnan(bb[2]).all()
    assert np.array_equal(np.delete(yb, 2, 0), np.delete(y, 2, 0))
    # selected columns equal the full result
    yc, bc = oracle.moe_block(fg, w_gu, fd, w_dn, E, D, F, x, idx, wts, cols=[255, 0, 17])
    assert np.array_equal(yc, y[:, [255, 0, 17]]) and np.array_equal(bc, b[:, [255, 0, 17]])


def test_routing_weights_generator():
    w = synth.routing_weights(synth.rng(3, 4), 16, 8)
    assert w.shape == (16, 8) and w.dtype == np.float32
    assert np.all(w > 0) and np.allclose(w.sum(axis=1), 1.0, atol=1e-6)
