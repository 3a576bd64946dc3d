"""GPU cases at the edges of the entry points: the largest grouped and MoE
calls, one-row weights on the matrix-core path, launches on a side stream,
and products captured in a HIP graph and replayed."""
import numpy as np
import pytest

import gemm_block_quant_amd as qg
import oracle
import synth
from helpers import assert_band, dev_bytes, dev_x, make_case, same_bits

pytestmark = pytest.mark.gpu


def _dev(a, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=dtype)).cuda()


def test_grouped_at_the_row_limit():
    """M = 16384 rows over 8 experts (about 2,048 rows each: many passes per expert)."""
    fmt, E, N, K, M = qg.Q4_K, 8, 96, 512, 16384
    w = synth.weights(fmt, synth.rng(61, 0), E * N, K, E=E)
    x = synth.x_bf16(synth.rng(61, 1), M, K)
    ids = np.random.default_rng(61).integers(0, E, M).astype(np.int32)
    y = qg.quant_grouped_gemm(dev_bytes(w), fmt, E, N, K, M, dev_x(x), _dev(ids, np.int32)).cpu().numpy()
    y_ref, bound = oracle.gemm(fmt, w, N, K, x, E=E, ids=ids)
    assert_band(y, y_ref, bound, "grouped M=16384")


def test_moe_block_at_the_pair_limit():
    """T * topk = 16384 pairs (2,048 tokens x top-8 over 64 experts)."""
    fg = fd = qg.Q4_K
    E, D, F, T, topk = 64, 256, 256, 2048, 8
    w_gu = synth.weights(fg, synth.rng(63, 0), E * 2 * F, D, E=E)
    w_dn = synth.weights(fd, synth.rng(63, 1), E * D, F, E=E)
    x = synth.x_bf16(synth.rng(63, 2), T, D)
    idx = synth.routing(synth.rng(63, 3), T, topk, E).reshape(T, topk)
    wts = synth.routing_weights(synth.rng(63, 4), T, topk)
    y = qg.quant_moe_block(dev_bytes(w_gu), fg, dev_bytes(w_dn), fd, E, D, F, dev_x(x), _dev(idx, np.int32),
                           _dev(wts, np.float32)).cpu().numpy()
    toks = np.unique(np.concatenate([[0, 1, T - 1], np.random.default_rng(64).integers(0, T, 40)]))
    y_ref, bound = oracle.moe_block(fg, w_gu, fd, w_dn, E, D, F, x[toks], idx[toks], wts[toks])
    assert_band(y[toks], y_ref, bound, "moe 16384 pairs")


@pytest.mark.parametrize("fmt,N,K,M", [(qg.Q4_K, 1, 256, 40), (qg.Q8_0, 3, 64, 35), (qg.Q6_K, 2, 256, 64),
                                       (qg.Q5_K, 1, 512, 33), (qg.FP8, 1, 128, 32), (qg.NVFP4, 1, 32, 100)])
def test_matrix_core_path_tiny_n(fmt, N, K, M):
    w, x = make_case(fmt, N, K, M, seed=70 + fmt)
    y = qg.quant_gemm(dev_bytes(w), fmt, N, K, M, dev_x(x)).cpu().numpy()
    y_ref, bound = oracle.gemm(fmt, w, N, K, x)
    assert_band(y, y_ref, bound, "tiny N fmt %d" % fmt)


def test_side_stream():
    """Launches on a non-default stream give the default stream's results."""
    import torch
    fmt, N, K = qg.Q6_K, 300, 2048
    w, x = make_case(fmt, N, K, 40, seed=80)
    wd, xd = dev_bytes(w), dev_x(x)
    ref1 = qg.quant_gemv(wd, fmt, N, K, xd[0].contiguous())
    ref40 = qg.quant_gemm(wd, fmt, N, K, 40, xd)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        y1 = qg.quant_gemv(wd, fmt, N, K, xd[0].contiguous(), stream=s)
        y40 = qg.quant_gemm(wd, fmt, N, K, 40, xd, stream=s)
    s.synchronize()
    assert same_bits(y1.cpu().numpy(), ref1.cpu().numpy())
    assert same_bits(y40.cpu().numpy(), ref40.cpu().numpy())


def test_graph_capture_replays_match_eager():
    """Decode, prefill, grouped and MoE-block calls captured in one HIP graph
    (torch's CUDAGraph) and replayed three times, with eager work between
    replays: every replay equals the eager results bit for bit."""
    import torch
    fmt, N, K = qg.Q4_K, 520, 1024
    w, x = make_case(fmt, N, K, 40, seed=81)
    wd, xd = dev_bytes(w), dev_x(x)
    E, M = 4, 24
    wg = synth.weights(qg.Q4_K, synth.rng(82, 0), E * N, K, E=E)
    wgd = dev_bytes(wg)
    xg = dev_x(synth.x_bf16(synth.rng(82, 1), M, K))
    ids = _dev(np.random.default_rng(82).integers(0, E, M), np.int32)
    ws = torch.empty(qg.quant_grouped_workspace_bytes(E, M), dtype=torch.uint8, device="cuda")
    Em, D, F, T, topk = 6, 256, 512, 5, 3
    w_gu = dev_bytes(synth.weights(qg.Q4_K, synth.rng(83, 0), Em * 2 * F, D, E=Em))
    w_dn = dev_bytes(synth.weights(qg.Q6_K, synth.rng(83, 1), Em * D, F, E=Em))
    xm = dev_x(synth.x_bf16(synth.rng(83, 2), T, D))
    idx = _dev(synth.routing(synth.rng(83, 3), T, topk, Em).reshape(T, topk), np.int32)
    wts = _dev(synth.routing_weights(synth.rng(83, 4), T, topk), np.float32)
    wsm = torch.empty(qg.quant_moe_workspace_bytes(qg.Q4_K, qg.Q6_K, Em, D, F, T, topk), dtype=torch.uint8,
                      device="cuda")
    outs = [torch.empty(N, dtype=torch.float32, device="cuda"), torch.empty((40, N), dtype=torch.float32, device="cuda"),
            torch.empty((M, N), dtype=torch.float32, device="cuda"), torch.empty((T, D), dtype=torch.float32, device="cuda")]

    def run(stream):
        qg.quant_gemv(wd, fmt, N, K, xd[0].contiguous(), y=outs[0], stream=stream)
        qg.quant_gemm(wd, fmt, N, K, 40, xd, y=outs[1], stream=stream)
        qg.quant_grouped_gemm(wgd, qg.Q4_K, E, N, K, M, xg, ids, y=outs[2], workspace=ws, stream=stream)
        qg.quant_moe_block(w_gu, qg.Q4_K, w_dn, qg.Q6_K, Em, D, F, xm, idx, wts, y=outs[3], workspace=wsm,
                           stream=stream)

    xd0 = xd[0].contiguous()  # allocated before capture
    run(None)
    torch.cuda.synchronize()
    eager = [o.cpu().numpy().copy() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(side)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = torch.cuda.current_stream()
        qg.quant_gemv(wd, fmt, N, K, xd0, y=outs[0], stream=st)
        qg.quant_gemm(wd, fmt, N, K, 40, xd, y=outs[1], stream=st)
        qg.quant_grouped_gemm(wgd, qg.Q4_K, E, N, K, M, xg, ids, y=outs[2], workspace=ws, stream=st)
        qg.quant_moe_block(w_gu, qg.Q4_K, w_dn, qg.Q6_K, Em, D, F, xm, idx, wts, y=outs[3], workspace=wsm,
                           stream=st)
    for rep in range(3):
        for o in outs:
            o.fill_(-1.0)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            assert same_bits(o.cpu().numpy(), eager[i]), (rep, i)
