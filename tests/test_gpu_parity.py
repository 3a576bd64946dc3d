"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

* dequantization: bit-exact fp32 (NaN matches NaN);
* products: |y - y_ref| <= 2e-3 * sum_k |w x| for every output element;
* invariants: row m of an M-row call equals the M = 1 call bit for bit, runs
  repeat bit for bit.
Shapes span several row tiles, ragged N, K of one block, K-segmented rows and
every row-pass width.
"""
import numpy as np
import pytest

import gemm_block_quant_amd as qg
import oracle
import synth
from helpers import assert_band, dev_bytes, dev_x, make_case, same_bits

pytestmark = pytest.mark.gpu

DEQ_SHAPES = [
    (qg.Q8_0, 37, 96), (qg.Q8_0, 5, 1024),
    (qg.Q4_K, 13, 512), (qg.Q4_K, 3, 5120),
    (qg.Q5_K, 7, 512), (qg.Q5_K, 3, 5120),
    (qg.Q6_K, 11, 768), (qg.Q6_K, 2, 17408),
    (qg.NVFP4, 9, 48), (qg.NVFP4, 17, 5120),
    (qg.FP8, 5, 64), (qg.FP8, 9, 5120),
]


def _put_f16(buf, off, value_bits):
    buf[off] = value_bits & 0xFF
    buf[off + 1] = value_bits >> 8


def _with_specials(fmt, w, N, K):
    """Overwrite a few blocks with edge values: zero / subnormal / max / negative fp16
    scales, int8 sub-scale -128, E4M3 subnormal, max, zero, -0 and NaN scales."""
    w = w.copy()
    if fmt == qg.NVFP4:
        R = N
        sc0 = R * K // 2
        specials = [0x00, 0x01, 0x07, 0x7E, 0x7F, 0x80, 0xFE, 0x08]
        for i, s in enumerate(specials[: R * K // 16]):
            w[sc0 + i] = s
        w[0] = 0x08  # codes -0 and +0
        return w
    if fmt == qg.FP8:
        codes = [0x00, 0x80, 0x01, 0x81, 0x07, 0x08, 0x7E, 0xFE, 0x7F, 0xFF, 0x38, 0xB8]
        w[:len(codes)] = codes  # zeros, subnormals, smallest normal, max, NaN, +-1
        rs = w[N * K:].view(np.float32)
        for i, v in enumerate([0.0, 1.4e-45, -2.5e-3, 3.0e38]):
            if i < N:
                rs[i] = v
        return w
    bb = {qg.Q8_0: 34, qg.Q4_K: 144, qg.Q5_K: 176, qg.Q6_K: 210}[fmt]
    doff = {qg.Q8_0: 0, qg.Q4_K: 0, qg.Q5_K: 0, qg.Q6_K: 208}[fmt]
    nblk = w.size // bb
    for i, bits in enumerate([0x0000, 0x0001, 0x03FF, 0x7BFF, 0x8000 | 0x2E66, 0x0400]):
        if i < nblk:
            _put_f16(w, i * bb + doff, bits)
    if fmt in (qg.Q4_K, qg.Q5_K) and nblk > 2:
        _put_f16(w, 2 * bb + 2, 0x0001)  # subnormal dmin
    if fmt == qg.Q6_K and nblk > 1:
        w[bb + 192: bb + 208] = 0x80  # sub-scales -128
    return w


@pytest.mark.parametrize("fmt,N,K", DEQ_SHAPES)
def test_dequant_bit_exact(fmt, N, K):
    w, _ = make_case(fmt, N, K, 1, seed=100 + fmt)
    w = _with_specials(fmt, w, N, K)
    ref = oracle.dequant_rows(fmt, w, 1, N, K)
    got = qg.quant_dequantize(dev_bytes(w), fmt, N, K).cpu().numpy()
    assert same_bits(got, ref)


def test_dequant_stacked_nvfp4_scales():
    E, N, K = 3, 5, 64
    w, _ = make_case(qg.NVFP4, N, K, 1, seed=7, E=E)
    ref = oracle.dequant_rows(qg.NVFP4, w, E, N, K)
    got = qg.quant_dequantize_stacked(dev_bytes(w), qg.NVFP4, E, N, K).cpu().numpy()
    assert same_bits(got, ref)


PRODUCT_CASES = [
    # (fmt, N, K, M)
    # odd row counts: 7 and 15 (partial groups of 4 and 8 activation rows), 31 (a 16-row pass and a 15-row one)
    (qg.Q4_K, 300, 5120, 7), (qg.Q4_K, 300, 5120, 15), (qg.Q4_K, 300, 5120, 31), (qg.Q6_K, 300, 17408, 7),
    (qg.Q6_K, 300, 5120, 15), (qg.Q6_K, 300, 5120, 31), (qg.NVFP4, 300, 5120, 7), (qg.NVFP4, 300, 17408, 15),
    (qg.NVFP4, 300, 5120, 31), (qg.Q5_K, 300, 5120, 7), (qg.Q5_K, 130, 5120, 31), (qg.FP8, 300, 5120, 15),
    (qg.FP8, 300, 5120, 31), (qg.Q8_0, 300, 1024, 7), (qg.Q8_0, 300, 1024, 15), (qg.Q8_0, 300, 1024, 31),
    (qg.Q8_0, 1, 32, 1), (qg.Q8_0, 300, 1024, 1), (qg.Q8_0, 1000, 2048, 3), (qg.Q8_0, 129, 4192, 8),
    (qg.Q4_K, 1, 256, 1), (qg.Q4_K, 5, 512, 2), (qg.Q4_K, 1000, 5120, 1), (qg.Q4_K, 777, 5120, 8),
    (qg.Q4_K, 257, 1792, 16), (qg.Q4_K, 130, 17408, 1), (qg.Q4_K, 64, 17408, 17),
    (qg.Q5_K, 1, 256, 1), (qg.Q5_K, 5, 512, 2), (qg.Q5_K, 1000, 5120, 1), (qg.Q5_K, 777, 5120, 8),
    (qg.Q5_K, 257, 1792, 16), (qg.Q5_K, 130, 17408, 1), (qg.Q5_K, 64, 17408, 17), (qg.Q5_K, 33, 4096, 3),
    (qg.Q6_K, 1, 256, 1), (qg.Q6_K, 3, 768, 4), (qg.Q6_K, 1000, 5120, 1), (qg.Q6_K, 150, 17408, 1),
    (qg.Q6_K, 99, 17408, 8), (qg.Q6_K, 333, 5120, 33),
    (qg.NVFP4, 1, 16, 1), (qg.NVFP4, 3, 48, 2), (qg.NVFP4, 1000, 5120, 1), (qg.NVFP4, 100, 17408, 1),
    (qg.NVFP4, 77, 592, 8), (qg.NVFP4, 200, 5120, 16), (qg.NVFP4, 51, 17408, 8),
    (qg.NVFP4, 70, 96, 3), (qg.NVFP4, 33, 1056, 8),  # K % 64 == 32: row-buffer path
    # matrix-core path (NVFP4, M >= 32): ragged M and N tiles, K % 32 == 16 (half step)
    (qg.NVFP4, 200, 5120, 37), (qg.NVFP4, 130, 48, 33), (qg.NVFP4, 300, 1040, 130), (qg.NVFP4, 1000, 512, 64),
    (qg.NVFP4, 64, 16, 32),
    # matrix-core path (Q4_K, Q5_K, M >= 32): ragged tiles, K of one super-block,
    # 64 x 64 and 128 x 64 tiles (the latter once the tile count covers the CUs)
    (qg.Q4_K, 200, 5120, 37), (qg.Q4_K, 130, 256, 33), (qg.Q4_K, 300, 1280, 130), (qg.Q4_K, 1000, 512, 64),
    (qg.Q4_K, 4100, 768, 450),
    (qg.Q5_K, 200, 5120, 37), (qg.Q5_K, 64, 256, 32), (qg.Q5_K, 300, 1792, 130), (qg.Q5_K, 4100, 768, 450),
    (qg.Q6_K, 200, 5120, 37), (qg.Q6_K, 130, 256, 33), (qg.Q6_K, 300, 1792, 130), (qg.Q6_K, 4100, 768, 450),
    (qg.Q8_0, 200, 1024, 37), (qg.Q8_0, 130, 64, 33), (qg.Q8_0, 300, 1088, 130), (qg.Q8_0, 4100, 768, 450),
    # Q8_0 with K % 64 == 32 keeps the 16-row passes
    (qg.Q8_0, 100, 1056, 40),
    # row-scaled FP8: decode, skinny, tall and matrix-core shapes
    (qg.FP8, 1, 64, 1), (qg.FP8, 7, 192, 2), (qg.FP8, 1000, 5120, 1), (qg.FP8, 777, 5120, 8),
    (qg.FP8, 257, 1792, 16), (qg.FP8, 130, 17408, 1), (qg.FP8, 64, 17408, 17), (qg.FP8, 33, 4096, 3),
    (qg.FP8, 200, 5120, 37), (qg.FP8, 130, 64, 33), (qg.FP8, 300, 1088, 130), (qg.FP8, 4100, 768, 450),
]


@pytest.mark.parametrize("fmt,N,K,M", PRODUCT_CASES)
def test_product_band(fmt, N, K, M):
    w, x = make_case(fmt, N, K, M, seed=1000 + N + K + M)
    y_ref, bound = oracle.gemm(fmt, w, N, K, x)
    wd, xd = dev_bytes(w), dev_x(x)
    if M == 1:
        y = qg.quant_gemv(wd, fmt, N, K, xd).cpu().numpy().reshape(1, N)
    else:
        y = qg.quant_gemm(wd, fmt, N, K, M, xd).cpu().numpy()
    assert_band(y, y_ref, bound, "fmt %d N %d K %d M %d" % (fmt, N, K, M))


@pytest.mark.parametrize("fmt,N,K", [(qg.Q8_0, 300, 1024), (qg.Q4_K, 300, 5120), (qg.Q6_K, 300, 17408),
                                     (qg.NVFP4, 300, 5120), (qg.Q5_K, 300, 5120), (qg.FP8, 300, 5120),
                                     # tall: up to 8 rows take the whole-row-group kernel, 16 the direct one
                                     (qg.Q4_K, 16385, 5120), (qg.NVFP4, 16387, 5120),
                                     # rows in K segments whose 8 and 16 activation rows are staged in
                                     # K phases (sums carried across phases)
                                     (qg.Q6_K, 5120, 17408), (qg.NVFP4, 5120, 17408)])
def test_rows_match_decode_bitwise_and_repeat(fmt, N, K):
    """Row m of M = 8 (and M = 16) equals the M = 1 result bit for bit; runs repeat."""
    M = 16
    w, x = make_case(fmt, N, K, M, seed=55)
    wd, xd = dev_bytes(w), dev_x(x)
    y16 = qg.quant_gemm(wd, fmt, N, K, M, xd).cpu().numpy()
    y8 = qg.quant_gemm(wd, fmt, N, K, 8, xd[:8].contiguous()).cpu().numpy()
    for m in range(M):
        y1 = qg.quant_gemv(wd, fmt, N, K, xd[m].contiguous()).cpu().numpy()
        assert same_bits(y16[m], y1), m
        if m < 8:
            assert same_bits(y8[m], y1), m
    again = qg.quant_gemm(wd, fmt, N, K, M, xd).cpu().numpy()
    assert same_bits(again, y16)


def test_read_probe_runs_and_writes_nothing():
    """The streaming-read reference reads every granule (odd sizes included) and
    leaves the sink alone for data whose per-thread xor cannot be the sentinel."""
    import torch
    for nbytes in (16, 4096 + 16, (1 << 20) + 48):
        buf = torch.full((nbytes // 4,), 1.0, dtype=torch.float32, device="cuda")
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        qg.quant_read_probe(buf, sink)
        torch.cuda.synchronize()
        assert int(sink.item()) == 0


def test_zero_activations_and_zero_weights():
    fmt, N, K = qg.Q4_K, 64, 512
    w, x = make_case(fmt, N, K, 1, seed=3)
    y = qg.quant_gemv(dev_bytes(w), fmt, N, K, dev_x(np.zeros_like(x))).cpu().numpy()
    assert not y.any()
    wz = w.copy().reshape(-1, 144)
    wz[:, 0:4] = 0  # d = dmin = 0
    y = qg.quant_gemv(dev_bytes(wz.reshape(-1)), fmt, N, K, dev_x(x)).cpu().numpy()
    assert not y.any()


FULL = [
    # the workload shapes: Q8_0 1024x1024; Q4_K fused gate+up; Q6_K down and LM head; NVFP4 both MLP shapes
    (qg.Q8_0, 1024, 1024, 1),
    (qg.Q4_K, 2 * 17408, 5120, 1), (qg.Q4_K, 2 * 17408, 5120, 8),
    # tall with a ragged last row group (whole-row-group kernel)
    (qg.Q4_K, 16385, 5120, 3), (qg.NVFP4, 16387, 5120, 5),
    # Q5_K at the fused gate+up shape
    (qg.Q5_K, 2 * 17408, 5120, 1), (qg.Q5_K, 2 * 17408, 5120, 8),
    (qg.Q6_K, 5120, 17408, 1), (qg.Q6_K, 5120, 17408, 8),
    (qg.Q6_K, 248320, 5120, 1), (qg.Q6_K, 248320, 5120, 8),
    (qg.NVFP4, 17408, 5120, 1), (qg.NVFP4, 17408, 5120, 8),
    (qg.NVFP4, 5120, 17408, 1), (qg.NVFP4, 5120, 17408, 8),
    (qg.NVFP4, 17408, 5120, 512), (qg.NVFP4, 5120, 17408, 512),
    (qg.Q4_K, 2 * 17408, 5120, 512), (qg.Q5_K, 2 * 17408, 5120, 512), (qg.Q6_K, 5120, 17408, 512),
    (qg.Q8_0, 1024, 1024, 512),
    # row-scaled FP8: the output head and the fused gate+up shape
    (qg.FP8, 248320, 5120, 1), (qg.FP8, 248320, 5120, 8),
    (qg.FP8, 2 * 17408, 5120, 1), (qg.FP8, 2 * 17408, 5120, 8), (qg.FP8, 2 * 17408, 5120, 512),
]


@pytest.mark.parametrize("fmt,N,K,M", FULL)
def test_full_size(fmt, N, K, M):
    """The workload shapes, in the launch configuration the bench times.  Every
    output is compared for M <= 16; for M = 512 every output of 48 rows drawn
    from the first, a middle and the last 128-row tile."""
    seed = {qg.Q8_0: 1, qg.Q4_K: 2, qg.Q6_K: 3, qg.NVFP4: 4, qg.Q5_K: 6, qg.FP8: 7}[fmt]
    w = synth.weights(fmt, synth.rng(seed, 0), N, K)
    x = synth.x_bf16(synth.rng(seed, 1), M, K)
    wd, xd = dev_bytes(w), dev_x(x)
    y = (qg.quant_gemv(wd, fmt, N, K, xd).reshape(1, N) if M == 1 else qg.quant_gemm(wd, fmt, N, K, M, xd))
    y = y.cpu().numpy()
    rows = np.arange(M)
    if M > 16:
        rows = np.unique(np.concatenate([np.arange(16), M // 2 - 8 + np.arange(16), M - 16 + np.arange(16)]))
        rows = rows[rows < M]
    y_ref, bound = oracle.gemm(fmt, w, N, K, x[rows])
    assert_band(y[rows], y_ref, bound, "full fmt %d N %d K %d M %d" % (fmt, N, K, M))


@pytest.mark.parametrize("fmt,N,K", [(qg.NVFP4, 1000, 1040), (qg.Q4_K, 4100, 768), (qg.Q5_K, 4100, 768),
                                     (qg.Q6_K, 4100, 768), (qg.Q8_0, 4100, 768), (qg.FP8, 4100, 768),
                                     (qg.NVFP4, 4100, 768)])
def test_mfma_rows_independent_of_tiling_and_repeat(fmt, N, K):
    """M >= 32 on the matrix cores: each output is one fixed fp32 accumulation
    over K, so the rows of a 37-row call equal those rows of a 512-row call
    (other tile shapes and grid) bit for bit, and runs repeat."""
    w, x = make_case(fmt, N, K, 512, seed=77)
    wd, xd = dev_bytes(w), dev_x(x)
    y512 = qg.quant_gemm(wd, fmt, N, K, 512, xd).cpu().numpy()
    y37 = qg.quant_gemm(wd, fmt, N, K, 37, xd[:37].contiguous()).cpu().numpy()
    assert same_bits(y37, y512[:37])
    again = qg.quant_gemm(wd, fmt, N, K, 512, xd).cpu().numpy()
    assert same_bits(again, y512)


def test_mfma_rows_past_the_grid_row_limit():
    """More activation rows than one launch's row tiles can hold (2^21 per
    launch): rows on both sides of the chunk boundary equal the same rows of a
    small call bit for bit."""
    import torch
    fmt, N, K = qg.FP8, 64, 64
    M = (1 << 21) + 40
    w, _ = make_case(fmt, N, K, 1, seed=91)
    g = torch.Generator().manual_seed(91)
    xd = torch.randn((M, K), generator=g).to(torch.bfloat16).cuda()
    wd = dev_bytes(w)
    y = qg.quant_gemm(wd, fmt, N, K, M, xd)
    for r0 in (0, (1 << 21) - 20, M - 40):
        ys = qg.quant_gemm(wd, fmt, N, K, 40, xd[r0:r0 + 40].contiguous())
        assert same_bits(y[r0:r0 + 40].cpu().numpy(), ys.cpu().numpy()), r0
    # and against the oracle on the rows around the boundary
    xs = xd[(1 << 21) - 4:(1 << 21) + 4].cpu().view(torch.int16).numpy().view(np.uint16)
    y_ref, bound = oracle.gemm(fmt, w, N, K, xs)
    assert_band(y[(1 << 21) - 4:(1 << 21) + 4].cpu().numpy(), y_ref, bound, "rows past the grid limit")
    del y, xd
    torch.cuda.empty_cache()
