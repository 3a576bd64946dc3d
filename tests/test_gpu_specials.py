"""Edge values through every product kernel, compared with the oracle.

The dequantization export is bit-exact on special values (test_gpu_parity);
here the same kind of values go through the decoders the products use: the
register-direct streaming kernels (M = 1, 7, 8, 15, 16; K segments and K
phases), the row-buffer kernels (Q8_0; NVFP4 with K % 64 = 32), 16-row passes
(M = 17..31), the matrix-core tiles (M >= 32), the workspace entry's
segment-per-workgroup and stream-K schedules, the grouped product and the MoE
block.  Each case also carries zero-point rows (every code at the format's
zero point, scales non-zero): their weights are exactly zero, so the band
asks for y = 0 exactly there.  The pattern is the pages' kernel-versus-
dequantize-then-matvec check ("A 320B MoE on a free Kaggle TPU", section
"What I actually ran").
"""
import numpy as np
import pytest

import gemm_block_quant_amd as qg
import oracle
from helpers import assert_band, dev_bytes, dev_x
from specials import special_case

pytestmark = pytest.mark.gpu


def _check(y, w, fmt, N, K, x, zrows, what, E=1, ids=None):
    y = np.asarray(y, np.float64).reshape(x.shape[0], N)
    y_ref, bound = oracle.gemm(fmt, w, N, K, x, E=E, ids=ids)
    assert np.isfinite(y_ref).all() and np.isfinite(bound).all(), what
    if ids is None and zrows:
        assert (bound[:, zrows] == 0).all(), what
        nz = y[:, zrows] != 0
        assert not nz.any(), "%s: %d zero-point outputs are not exactly 0 (e.g. %r)" % (
            what, int(nz.sum()), y[:, zrows][nz][:4])
    assert_band(y, y_ref, bound, what)


CASES = [
    # register-direct streaming: decode, skinny, odd M, K segments (few rows) and K phases
    (qg.Q4_K, 300, 5120, 1), (qg.Q4_K, 300, 5120, 7), (qg.Q4_K, 1000, 5120, 16), (qg.Q4_K, 300, 17408, 8),
    (qg.Q5_K, 300, 5120, 1), (qg.Q5_K, 300, 5120, 15), (qg.Q5_K, 300, 17408, 8),
    (qg.Q6_K, 300, 5120, 1), (qg.Q6_K, 300, 5120, 7), (qg.Q6_K, 300, 17408, 1), (qg.Q6_K, 300, 17408, 8),
    (qg.Q6_K, 1000, 5120, 16),
    (qg.NVFP4, 300, 5120, 1), (qg.NVFP4, 300, 5120, 15), (qg.NVFP4, 300, 17408, 8),
    (qg.FP8, 300, 5120, 1), (qg.FP8, 300, 5120, 7), (qg.FP8, 300, 17408, 16),
    # LDS row-buffer kernels
    (qg.Q8_0, 300, 1024, 1), (qg.Q8_0, 300, 2048, 7), (qg.Q8_0, 130, 4192, 16),
    (qg.NVFP4, 130, 1056, 1), (qg.NVFP4, 130, 1056, 8),
    # 16-row passes (17 <= M <= 31) and Q8_0 with K % 64 = 32 at M >= 32
    (qg.Q4_K, 130, 1024, 31), (qg.Q6_K, 130, 1024, 17), (qg.FP8, 130, 1024, 31), (qg.Q8_0, 100, 1056, 40),
    # matrix-core tiles
    (qg.Q4_K, 200, 1024, 37), (qg.Q4_K, 4100, 512, 130), (qg.Q5_K, 200, 1024, 37),
    (qg.Q6_K, 200, 1024, 37), (qg.Q6_K, 4100, 512, 130), (qg.Q8_0, 200, 1024, 37),
    (qg.NVFP4, 200, 1024, 37), (qg.NVFP4, 130, 1040, 33), (qg.FP8, 200, 1024, 37), (qg.FP8, 4100, 512, 130),
]


@pytest.mark.parametrize("fmt,N,K,M", CASES)
def test_specials_and_zero_point_rows(fmt, N, K, M):
    w, x, zrows = special_case(fmt, N, K, M, seed=500 + fmt + M)
    wd, xd = dev_bytes(w), dev_x(x)
    if M == 1:
        y = qg.quant_gemv(wd, fmt, N, K, xd).cpu().numpy()
    else:
        y = qg.quant_gemm(wd, fmt, N, K, M, xd).cpu().numpy()
    _check(y, w, fmt, N, K, x, zrows, "specials fmt %d N %d K %d M %d" % (fmt, N, K, M))


WORKSPACE_CASES = [
    # one K segment per workgroup (quant_gemm_streamk, 5..16 rows on K-phased
    # shapes): N = 300 cuts each row into 16 segments, N = 5120 into 3
    (qg.Q6_K, 300, 17408, 8), (qg.NVFP4, 300, 17408, 8), (qg.Q4_K, 300, 17408, 16), (qg.FP8, 300, 17408, 8),
    (qg.Q5_K, 300, 17408, 8), (qg.Q6_K, 5120, 17408, 8),
    # stream-K tiles (260 tiles for 512 resident workgroups, 4 or 8 K steps)
    (qg.Q4_K, 4160, 256, 512), (qg.Q6_K, 4160, 512, 512), (qg.NVFP4, 8320, 256, 512), (qg.FP8, 8320, 512, 512),
]


@pytest.mark.parametrize("fmt,N,K,M", WORKSPACE_CASES)
def test_workspace_schedules_specials_and_zero_point_rows(fmt, N, K, M):
    """The workspace entry's two schedules on the same edge values."""
    assert qg.quant_gemm_streamk_workspace_bytes(fmt, N, K, M) > 0, "not on a workspace schedule"
    w, x, zrows = special_case(fmt, N, K, M, seed=800 + fmt + M)
    y = qg.quant_gemm_streamk(dev_bytes(w), fmt, N, K, M, dev_x(x)).cpu().numpy()
    _check(y, w, fmt, N, K, x, zrows, "workspace specials fmt %d N %d K %d M %d" % (fmt, N, K, M))


@pytest.mark.parametrize("fmt,K", [(qg.Q4_K, 1024), (qg.Q5_K, 1024), (qg.Q6_K, 1024), (qg.Q8_0, 1024),
                                   (qg.NVFP4, 1024), (qg.NVFP4, 1056), (qg.FP8, 1024)])
def test_grouped_specials_and_zero_point_rows(fmt, K):
    E, N, M = 5, 70, 24
    w, x, zrows = special_case(fmt, N, K, M, seed=600 + fmt, E=E)
    ids = np.random.default_rng(fmt).integers(0, E, M).astype(np.int32)
    import torch
    y = qg.quant_grouped_gemm(dev_bytes(w), fmt, E, N, K, M, dev_x(x), torch.from_numpy(ids).cuda())
    y = y.cpu().numpy().astype(np.float64)
    y_ref, bound = oracle.gemm(fmt, w, N, K, x, E=E, ids=ids)
    assert np.isfinite(y_ref).all()
    # zero-point rows of the stacked tensor, as (expert, row) -> outputs of the rows routed there
    for r in zrows:
        e, n = divmod(r, N)
        sel = ids == e
        if sel.any():
            assert (bound[sel, n] == 0).all()
            assert (y[sel, n] == 0).all(), (e, n, y[sel, n])
    assert_band(y, y_ref, bound, "grouped specials fmt %d" % fmt)


@pytest.mark.parametrize("fg,fd", [(qg.Q4_K, qg.Q6_K), (qg.Q5_K, qg.Q8_0), (qg.FP8, qg.NVFP4)])
def test_moe_block_specials(fg, fd):
    import torch

    import synth
    from specials import with_specials
    E, D, F, T, topk = 5, 512, 256, 6, 2
    w_gu = with_specials(fg, synth.weights(fg, synth.rng(71, 0), E * 2 * F, D, E=E), E, 2 * F, D, seed=71)
    w_dn = with_specials(fd, synth.weights(fd, synth.rng(71, 1), E * D, F, E=E), E, D, F, seed=72)
    x = synth.x_bf16(synth.rng(71, 2), T, D)
    idx = synth.routing(synth.rng(71, 3), T, topk, E).reshape(T, topk)
    wts = synth.routing_weights(synth.rng(71, 4), T, topk)
    y = qg.quant_moe_block(dev_bytes(w_gu), fg, dev_bytes(w_dn), fd, E, D, F, dev_x(x),
                           torch.from_numpy(idx).cuda(), torch.from_numpy(wts).cuda()).cpu().numpy()
    y_ref, bound = oracle.moe_block(fg, w_gu, fd, w_dn, E, D, F, x, idx, wts)
    assert np.isfinite(y_ref).all()
    assert_band(y, y_ref, bound, "moe specials %d/%d" % (fg, fd))
