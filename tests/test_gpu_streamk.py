"""The stream-K tile schedule (quant_gemm_streamk) against the CPU oracle,
through the C ABI.

The shapes have a tile count of at least half the resident workgroups (two
per compute unit) but fewer than them: the schedule then deals (tile, K step)
iterations evenly and splits tiles between two or three workgroups, whose
partial sums the last part to arrive adds.  Covered:
every format, ragged rows and columns, K short enough that one workgroup
covers less than a tile, the workload shapes at M = 512, repeats bit for bit
(with the workspace overwritten in between), and graph capture.
"""
import numpy as np
import pytest

import gemm_block_quant_amd as qg
import oracle
import synth
from helpers import assert_band, dev_bytes, dev_x, make_case, same_bits

pytestmark = pytest.mark.gpu

SPLIT_CASES = [
    # (fmt, N, K, M): 260 tiles of 128 x 128 (row-scaled formats) or 128 x 64,
    # 16 K steps each, about 8 steps per workgroup: tiles in two and three parts
    (qg.NVFP4, 8320, 1024, 512), (qg.FP8, 8320, 1024, 512),
    (qg.Q4_K, 4160, 1024, 512), (qg.Q5_K, 4160, 1024, 512), (qg.Q6_K, 4160, 1024, 512),
    (qg.Q8_0, 4160, 1024, 512),
    # ragged rows (300) and columns (N % 64 != 0), 12 K steps: 330 and 258 tiles
    (qg.Q4_K, 7000, 768, 300), (qg.NVFP4, 11000, 768, 300),
    # one K step per tile (fewer iterations than workgroups: empty ranges, no
    # tile split) and two (splits of two parts only)
    (qg.FP8, 8320, 64, 512), (qg.Q8_0, 4160, 64, 512), (qg.NVFP4, 8320, 128, 512),
]


def _streamk(wd, fmt, N, K, M, xd, workspace=None, stream=None):
    return qg.quant_gemm_streamk(wd, fmt, N, K, M, xd, workspace=workspace, stream=stream)


@pytest.mark.parametrize("fmt,N,K,M", SPLIT_CASES)
def test_streamk_band_every_output(fmt, N, K, M):
    wsb = qg.quant_gemm_streamk_workspace_bytes(fmt, N, K, M)
    assert wsb > 0, "shape does not take the stream-K schedule on this device"
    w, x = make_case(fmt, N, K, M, seed=400 + fmt)
    wd, xd = dev_bytes(w), dev_x(x)
    y = _streamk(wd, fmt, N, K, M, xd).cpu().numpy()
    y_ref, bound = oracle.gemm(fmt, w, N, K, x)
    assert_band(y, y_ref, bound, "stream-K fmt %d N %d K %d M %d" % (fmt, N, K, M))


@pytest.mark.parametrize("fmt,N,K,M", SPLIT_CASES[:3])
def test_streamk_repeats_bitwise_with_dirty_workspace(fmt, N, K, M):
    """One rounding order per shape: two calls agree bit for bit, also when
    the workspace is overwritten between them (its counters are cleared by
    every call), and agree with the plain schedule within the band."""
    import torch
    w, x = make_case(fmt, N, K, M, seed=500 + fmt)
    wd, xd = dev_bytes(w), dev_x(x)
    ws = torch.empty(qg.quant_gemm_streamk_workspace_bytes(fmt, N, K, M), dtype=torch.uint8, device="cuda")
    y1 = _streamk(wd, fmt, N, K, M, xd, workspace=ws).cpu().numpy()
    ws.fill_(0xFF)
    y2 = _streamk(wd, fmt, N, K, M, xd, workspace=ws).cpu().numpy()
    assert same_bits(y1, y2)
    ws.fill_(0x01)
    y3 = _streamk(wd, fmt, N, K, M, xd, workspace=ws).cpu().numpy()
    assert same_bits(y1, y3)
    yp = qg.quant_gemm(wd, fmt, N, K, M, xd).cpu().numpy()
    _, bound = oracle.gemm(fmt, w, N, K, x[:64])
    assert_band(y1[:64], yp[:64].astype(np.float64), bound, "stream-K vs plain")


# the 5120-row down projections take the stream-K schedule (320 tiles); the
# others have more tiles than slots and run quant_gemm's
FULL_512 = [(qg.NVFP4, 5120, 17408, 512), (qg.Q6_K, 5120, 17408, 512), (qg.NVFP4, 17408, 5120, 512),
            (qg.Q4_K, 2 * 17408, 5120, 512)]


@pytest.mark.parametrize("fmt,N,K,M", FULL_512)
def test_streamk_full_size(fmt, N, K, M):
    """The prefill workload shapes in the configuration the bench times: every
    output of 48 rows drawn from the first, a middle and the last row tile."""
    seed = {qg.Q4_K: 2, qg.Q6_K: 3, qg.NVFP4: 4, qg.Q5_K: 6, qg.FP8: 7}[fmt]
    w = synth.weights(fmt, synth.rng(seed, 0), N, K)
    x = synth.x_bf16(synth.rng(seed, 1), M, K)
    wd, xd = dev_bytes(w), dev_x(x)
    y = _streamk(wd, fmt, N, K, M, xd).cpu().numpy()
    rows = np.unique(np.concatenate([np.arange(16), M // 2 - 8 + np.arange(16), M - 16 + np.arange(16)]))
    y_ref, bound = oracle.gemm(fmt, w, N, K, x[rows])
    assert_band(y[rows], y_ref, bound, "stream-K full fmt %d N %d K %d M %d" % (fmt, N, K, M))


def test_streamk_without_split_is_quant_gemm():
    """Where the plain schedule is as balanced (or the call is not on the
    tiles) no workspace is needed and the result is quant_gemm's bit for bit."""
    for fmt, N, K, M in [(qg.Q4_K, 200, 512, 300), (qg.NVFP4, 520, 1024, 8), (qg.Q6_K, 64, 256, 40),
                         (qg.NVFP4, 17408, 1024, 512)]:
        assert qg.quant_gemm_streamk_workspace_bytes(fmt, N, K, M) == 0
        w, x = make_case(fmt, N, K, M, seed=600 + N)
        wd, xd = dev_bytes(w), dev_x(x)
        y = qg.quant_gemm_streamk(wd, fmt, N, K, M, xd).cpu().numpy()
        assert same_bits(y, qg.quant_gemm(wd, fmt, N, K, M, xd).cpu().numpy()), (fmt, N, K, M)


def test_streamk_graph_replays_match_eager():
    """Captured into a HIP graph (counter clearing by a kernel, no memset) and
    replayed three times with eager work between: every replay equals the
    eager result bit for bit."""
    import torch
    fmt, N, K, M = qg.NVFP4, 8320, 1024, 512
    w, x = make_case(fmt, N, K, M, seed=650)
    wd, xd = dev_bytes(w), dev_x(x)
    ws = torch.empty(qg.quant_gemm_streamk_workspace_bytes(fmt, N, K, M), dtype=torch.uint8, device="cuda")
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    _streamk(wd, fmt, N, K, M, xd, workspace=ws)
    torch.cuda.synchronize()
    eager = qg.quant_gemm_streamk(wd, fmt, N, K, M, xd, y=y, workspace=ws).cpu().numpy().copy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        qg.quant_gemm_streamk(wd, fmt, N, K, M, xd, y=y, workspace=ws, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qg.quant_gemm_streamk(wd, fmt, N, K, M, xd, y=y, workspace=ws, stream=torch.cuda.current_stream())
    for rep in range(3):
        y.fill_(-1.0)
        ws.fill_(0x7F)  # eager work between replays, the counters dirtied
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert same_bits(y.cpu().numpy(), eager), rep
