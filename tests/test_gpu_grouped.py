"""GPU parity of the grouped-expert product over stacked weight[E*N, K]."""
import numpy as np
import pytest

import gemm_block_quant_amd as qg
import oracle
import synth
from helpers import assert_band, dev_bytes, dev_x, same_bits

pytestmark = pytest.mark.gpu


def _ids_dev(ids):
    import torch
    return torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda()


@pytest.mark.parametrize("fmt,E,N,K,M", [
    (qg.Q4_K, 5, 100, 512, 12), (qg.Q6_K, 4, 77, 768, 9), (qg.Q8_0, 6, 50, 1024, 20),
    (qg.NVFP4, 3, 64, 592, 7), (qg.Q4_K, 40, 130, 2048, 37), (qg.Q5_K, 6, 90, 1024, 15),
    (qg.FP8, 5, 100, 1024, 13),
])
def test_grouped_band_and_invalid_rows(fmt, E, N, K, M):
    w = synth.weights(fmt, synth.rng(21, 0), E * N, K, E=E)
    x = synth.x_bf16(synth.rng(21, 1), M, K)
    g = np.random.default_rng(E + M)
    ids = g.integers(0, E, M).astype(np.int32)
    ids[1] = -1
    ids[M // 2] = E  # out of range
    ids[2:5] = ids[0]  # repeats
    y = qg.quant_grouped_gemm(dev_bytes(w), fmt, E, N, K, M, dev_x(x), _ids_dev(ids)).cpu().numpy()
    y_ref, bound = oracle.gemm(fmt, w, N, K, x, E=E, ids=ids)
    bad = (ids < 0) | (ids >= E)
    assert np.isnan(y[bad]).all()
    assert_band(y[~bad], y_ref[~bad], bound[~bad], "grouped fmt %d" % fmt)


@pytest.mark.parametrize("fmt,K", [(qg.Q4_K, 4096), (qg.NVFP4, 5120), (qg.Q6_K, 2048), (qg.Q5_K, 2048),
                                   (qg.FP8, 2048)])
def test_grouped_e1_is_dense_bitwise(fmt, K):
    """E = 1 is the dense product bit for bit.  With E > 1 rows are never cut
    into K segments, so a row equals its expert's decode GEMV bit for bit
    wherever that dense shape is not cut either (here 16384-row experts), and
    permuting the rows of a call permutes its outputs bit for bit."""
    N, M = 257, 11
    w = synth.weights(fmt, synth.rng(22, 0), N, K)
    x = synth.x_bf16(synth.rng(22, 1), M, K)
    wd, xd = dev_bytes(w), dev_x(x)
    yd = qg.quant_gemm(wd, fmt, N, K, M, xd).cpu().numpy()
    yg = qg.quant_grouped_gemm(wd, fmt, 1, N, K, M, xd, None).cpu().numpy()
    assert same_bits(yg, yd)
    # each row of a grouped call equals the decode GEMV of its own expert
    E, N = 3, 16384
    ws = synth.weights(fmt, synth.rng(23, 0), E * N, K, E=E)
    ids = np.array([2, 0, 2, 1, 2, 0, 1, 1, 2, 0, 2], np.int32)
    wsd = dev_bytes(ws)
    yg = qg.quant_grouped_gemm(wsd, fmt, E, N, K, M, xd, _ids_dev(ids)).cpu().numpy()
    for i, e in enumerate(ids):
        if fmt == qg.NVFP4:
            R = E * N
            codes = ws[e * N * K // 2:(e + 1) * N * K // 2]
            sc = ws[R * K // 2 + e * N * K // 16: R * K // 2 + (e + 1) * N * K // 16]
            gs = ws[R * K // 2 + R * K // 16 + 4 * e: R * K // 2 + R * K // 16 + 4 * e + 4]
            we = np.concatenate([codes, sc, gs])
        elif fmt == qg.FP8:  # planes: codes [E*N][K], then E*N fp32 row scales
            R = E * N
            codes = ws[e * N * K:(e + 1) * N * K]
            sc = ws[R * K + 4 * e * N: R * K + 4 * (e + 1) * N]
            we = np.concatenate([codes, sc])
        else:
            eb = oracle.packed_bytes(fmt, 1, N, K)
            we = ws[e * eb:(e + 1) * eb]
        y1 = qg.quant_gemv(dev_bytes(we), fmt, N, K, xd[i].contiguous()).cpu().numpy()
        assert same_bits(yg[i], y1), i
    perm = np.random.default_rng(24).permutation(M)
    yp = qg.quant_grouped_gemm(wsd, fmt, E, N, K, M, dev_x(x[perm]), _ids_dev(ids[perm])).cpu().numpy()
    assert same_bits(yp, yg[perm])


@pytest.mark.parametrize("N,K", [(2048, 4096), (4096, 2048)])
def test_grouped_moe_layer(N, K):
    """288 stacked Q4_K experts, 16 tokens each routed to 8 distinct experts: every output."""
    E, T, topk = 288, 16, 8
    w = synth.weights(qg.Q4_K, synth.rng(5, 0 if K == 4096 else 4), E * N, K, E=E)
    x = synth.x_bf16(synth.rng(5, 1 if K == 4096 else 3), T * topk, K)
    ids = synth.routing(synth.rng(5, 2), T, topk, E)
    y = qg.quant_grouped_gemm(dev_bytes(w), qg.Q4_K, E, N, K, T * topk, dev_x(x), _ids_dev(ids)).cpu().numpy()
    y_ref, bound = oracle.gemm(qg.Q4_K, w, N, K, x, E=E, ids=ids)
    assert_band(y, y_ref, bound, "moe N %d K %d" % (N, K))


@pytest.mark.parametrize("fmt", [qg.Q4_K, qg.Q5_K, qg.Q6_K, qg.NVFP4, qg.FP8])
def test_grouped_decode_batch_rows_bitwise(fmt):
    """A decode-like batch (fewer rows than experts, a few experts with 3 to 5
    rows, streamed in passes of up to 4 rows): every row equals the same row
    computed alone (a one-row grouped call) bit for bit, and the band."""
    E, N, K = 40, 256, 1024
    sizes = [5, 4, 4, 3, 3, 2, 2, 2] + [1] * 15
    ids = np.concatenate([np.full(c, e * 3 % E, np.int32) for e, c in enumerate(sizes)])
    ids = ids[np.random.default_rng(31).permutation(len(ids))]
    M = len(ids)
    w = synth.weights(fmt, synth.rng(30, 0), E * N, K, E=E)
    x = synth.x_bf16(synth.rng(30, 1), M, K)
    wd, xd = dev_bytes(w), dev_x(x)
    y = qg.quant_grouped_gemm(wd, fmt, E, N, K, M, xd, _ids_dev(ids)).cpu().numpy()
    for i in range(M):
        y1 = qg.quant_grouped_gemm(wd, fmt, E, N, K, 1, xd[i:i + 1].contiguous(), _ids_dev(ids[i:i + 1]))
        assert same_bits(y[i], y1.cpu().numpy()[0]), i
    y_ref, bound = oracle.gemm(fmt, w, N, K, x, E=E, ids=ids)
    assert_band(y, y_ref, bound, "decode batch fmt %d" % fmt)


def _slot_ids(sizes, E, seed, invalid=2):
    """ids giving expert e sizes[e] rows (shuffled), plus `invalid` rows with bad ids."""
    ids = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(sizes)] +
                         [np.array([-1, E] * (invalid // 2), np.int32)])
    return ids[np.random.default_rng(seed).permutation(len(ids))]


def _expert_weights(fmt, w, E, N, K, e):
    """Packed bytes of expert e alone (the planes of a stacked tensor cut out)."""
    R = E * N
    if fmt == qg.NVFP4:
        codes = w[e * N * K // 2:(e + 1) * N * K // 2]
        sc = w[R * K // 2 + e * N * K // 16: R * K // 2 + (e + 1) * N * K // 16]
        gs = w[R * K // 2 + R * K // 16 + 4 * e: R * K // 2 + R * K // 16 + 4 * e + 4]
        return np.concatenate([codes, sc, gs])
    if fmt == qg.FP8:
        return np.concatenate([w[e * N * K:(e + 1) * N * K], w[R * K + 4 * e * N: R * K + 4 * (e + 1) * N]])
    eb = oracle.packed_bytes(fmt, 1, N, K)
    return w[e * eb:(e + 1) * eb]


# slot sizes around the tile threshold (32) and the tile heights (64, 128):
# the mean rows per expert picks 64-row tiles in the first shape, 128 in the second
@pytest.mark.parametrize("sizes", [(32, 31, 64, 65, 129, 1, 0), (300, 140, 40, 7)])
@pytest.mark.parametrize("fmt,K", [(qg.Q4_K, 512), (qg.Q6_K, 512), (qg.Q8_0, 512), (qg.NVFP4, 512), (qg.FP8, 512),
                                   (qg.Q5_K, 512), (qg.NVFP4, 528), (qg.Q8_0, 544)])
def test_grouped_large_experts_on_tiles(fmt, K, sizes):
    """Experts with 32 or more rows run on the matrix-core tiles (each expert's
    weights read once per tile of rows), the others stream; every output
    against the oracle, and the tiled experts' rows bit for bit equal to the
    dense product over that expert's rows.  (NVFP4 with K % 64 = 16 and Q8_0
    with K % 64 = 32 have no grouped tile path: all their experts stream; the
    dense Q8_0 product then streams too, the dense NVFP4 one has a tile kernel
    of its own.)"""
    import torch
    E, N = len(sizes), 96
    w = synth.weights(fmt, synth.rng(25, fmt), E * N, K, E=E)
    ids = _slot_ids(sizes, E, 26 + fmt)
    M = len(ids)
    x = synth.x_bf16(synth.rng(25, 10 + fmt), M, K)
    wd, xd = dev_bytes(w), dev_x(x)
    y = qg.quant_grouped_gemm(wd, fmt, E, N, K, M, xd, _ids_dev(ids)).cpu().numpy()
    bad = (ids < 0) | (ids >= E)
    assert np.isnan(y[bad]).all()
    y_ref, bound = oracle.gemm(fmt, w, N, K, x, E=E, ids=ids)
    assert_band(y[~bad], y_ref[~bad], bound[~bad], "grouped tiles fmt %d K %d" % (fmt, K))
    if fmt == qg.NVFP4 and K % 64:
        return  # the dense product has its own NVFP4 tile kernel for such K: equal in band only
    for e, c in enumerate(sizes):
        if c < 32:
            continue
        rows = np.nonzero(ids == e)[0]
        we = dev_bytes(_expert_weights(fmt, w, E, N, K, e))
        yd = qg.quant_gemm(we, fmt, N, K, c, xd[torch.from_numpy(rows).cuda()].contiguous()).cpu().numpy()
        assert same_bits(y[rows], yd), (fmt, K, e, c)


@pytest.mark.parametrize("fmt,K", [(qg.Q4_K, 1024), (qg.Q6_K, 512), (qg.NVFP4, 512), (qg.Q8_0, 512)])
def test_grouped_e1_is_dense_bitwise_on_tiles(fmt, K):
    """E = 1 with ids = NULL and M >= 32 is the dense matrix-core product bit
    for bit (both take the tiles), at tile heights 64 and 128."""
    N = 200
    w = synth.weights(fmt, synth.rng(27, fmt), N, K)
    for M in (45, 300):
        x = synth.x_bf16(synth.rng(27, M), M, K)
        wd, xd = dev_bytes(w), dev_x(x)
        yd = qg.quant_gemm(wd, fmt, N, K, M, xd).cpu().numpy()
        yg = qg.quant_grouped_gemm(wd, fmt, 1, N, K, M, xd, None).cpu().numpy()
        assert same_bits(yg, yd), (fmt, K, M)


@pytest.mark.parametrize("E,M,mode", [(20000, 300, "random"), (5000, 200, "random"), (7, 200, "invalid"),
                                      (1, 129, "null"), (64, 129, "one"), (3, 4096, "random"),
                                      # small calls: counting sort, and the one-wave bitonic sort (E > 16384)
                                      (288, 128, "random"), (4, 31, "invalid"), (9, 1, "random"),
                                      (20000, 100, "random")])
def test_grouped_bucketing_paths(E, M, mode):
    """Calls bucket by counting sort (E <= 16384) or by a bitonic sort of
    (id, row) keys (larger E): every output against the
    oracle for many experts, all ids invalid, ids = NULL, one expert, and a
    large call over few experts."""
    fmt, N, K = qg.Q4_K, 8, 256
    w = synth.weights(fmt, synth.rng(28, E % 97), E * N, K, E=E)
    x = synth.x_bf16(synth.rng(28, M), M, K)
    g = np.random.default_rng(E + M)
    if mode == "random":
        ids = g.integers(0, E, M).astype(np.int32)
        ids[::17] = E + 3  # some invalid
    elif mode == "invalid":
        ids = np.full(M, -1, np.int32)
    elif mode == "one":
        ids = np.full(M, E - 1, np.int32)
    else:
        ids = None
    y = qg.quant_grouped_gemm(dev_bytes(w), fmt, E, N, K, M, dev_x(x), None if ids is None else _ids_dev(ids))
    y = y.cpu().numpy()
    ids_ref = np.zeros(M, np.int32) if ids is None else ids
    bad = (ids_ref < 0) | (ids_ref >= E)
    assert np.isnan(y[bad]).all()
    if (~bad).any():
        y_ref, bound = oracle.gemm(fmt, w, N, K, x, E=E, ids=ids_ref)
        assert_band(y[~bad], y_ref[~bad], bound[~bad], "bucketing E %d M %d %s" % (E, M, mode))
