"""quant_gemm_streamk at up to 16 rows on the K-phased shapes, through the C ABI.

Where the plain direct launch would stage the activations of 5..8 rows in
several K phases (the 5120-row down projections at K = 17,408), the workspace
entry gives each workgroup one K segment and adds the segments' sums through
the workspace, in segment order.  Every output keeps the arithmetic of the
single-workgroup path, so each row equals the M = 1 result bit for bit.
"""
import numpy as np
import pytest

import gemm_block_quant_amd as qg
import oracle
import synth
from helpers import assert_band, dev_bytes, dev_x, make_case, same_bits

pytestmark = pytest.mark.gpu

DOWN = [(qg.Q6_K, 5120, 17408), (qg.NVFP4, 5120, 17408)]


@pytest.mark.parametrize("fmt,N,K", DOWN)
def test_xseg_rows_equal_decode_bitwise(fmt, N, K):
    """Rows of 5..16-row calls (16 and 9: passes of 8 rows, the last of 8 and of
    1) equal the M = 1 result and quant_gemm's bit for bit."""
    M = 16
    w, x = make_case(fmt, N, K, M, seed=700 + fmt)
    wd, xd = dev_bytes(w), dev_x(x)
    y1 = [qg.quant_gemv(wd, fmt, N, K, xd[m].contiguous()).cpu().numpy() for m in range(M)]
    for m_rows in (8, 7, 5, 16, 11, 9):
        assert qg.quant_gemm_streamk_workspace_bytes(fmt, N, K, m_rows) > 0, m_rows
        xs = xd[:m_rows].contiguous()
        y = qg.quant_gemm_streamk(wd, fmt, N, K, m_rows, xs).cpu().numpy()
        yp = qg.quant_gemm(wd, fmt, N, K, m_rows, xs).cpu().numpy()
        assert same_bits(y, yp), m_rows
        for m in range(m_rows):
            assert same_bits(y[m], y1[m]), (m_rows, m)


@pytest.mark.parametrize("fmt", [qg.Q4_K, qg.Q5_K, qg.Q6_K, qg.NVFP4, qg.FP8])
def test_xseg_band_every_output(fmt):
    N, K, M = 5120, 17408, 8
    assert qg.quant_gemm_streamk_workspace_bytes(fmt, N, K, M) > 0
    w, x = make_case(fmt, N, K, M, seed=720 + fmt)
    y = qg.quant_gemm_streamk(dev_bytes(w), fmt, N, K, M, dev_x(x)).cpu().numpy()
    y_ref, bound = oracle.gemm(fmt, w, N, K, x)
    assert_band(y, y_ref, bound, "segment-per-workgroup fmt %d" % fmt)


def test_xseg_ragged_rows_and_dirty_workspace():
    """N not a multiple of the row group (rows past N are never written), two
    calls with the workspace overwritten in between agree bit for bit."""
    import torch
    fmt, N, K, M = qg.Q6_K, 5122, 17408, 6
    wsb = qg.quant_gemm_streamk_workspace_bytes(fmt, N, K, M)
    assert wsb > 0
    w, x = make_case(fmt, N, K, M, seed=740)
    wd, xd = dev_bytes(w), dev_x(x)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    y = torch.full((M + 1, N), 7.0, dtype=torch.float32, device="cuda")
    qg.quant_gemm_streamk(wd, fmt, N, K, M, xd, y=y[:M], workspace=ws)
    first = y.cpu().numpy().copy()
    assert (first[M] == 7.0).all()  # nothing past the output
    ws.fill_(0xFF)
    qg.quant_gemm_streamk(wd, fmt, N, K, M, xd, y=y[:M], workspace=ws)
    assert same_bits(y.cpu().numpy(), first)
    y_ref, bound = oracle.gemm(fmt, w, N, K, x)
    assert_band(first[:M], y_ref, bound, "ragged")


def test_xseg_graph_replays_match_eager():
    import torch
    fmt, N, K, M = qg.NVFP4, 5120, 17408, 8
    w, x = make_case(fmt, N, K, M, seed=760)
    wd, xd = dev_bytes(w), dev_x(x)
    ws = torch.empty(qg.quant_gemm_streamk_workspace_bytes(fmt, N, K, M), dtype=torch.uint8, device="cuda")
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
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
        ws.fill_(0x7F)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert same_bits(y.cpu().numpy(), eager), rep
