"""The edge-value weight builders of tests/specials.py, checked on the CPU with
the (separately pinned) oracle: special blocks dequantize to finite values that
include the intended extremes, and zero-point rows dequantize to exactly zero
although their scales are non-zero."""
import numpy as np
import pytest

import oracle
from specials import FP8, NVFP4, Q4_K, Q5_K, Q6_K, Q8_0, special_case, with_specials, zero_point_rows

FMTS = [(Q8_0, 1024), (Q4_K, 1024), (Q5_K, 1024), (Q6_K, 1024), (NVFP4, 1024), (NVFP4, 1056), (FP8, 1024)]


@pytest.mark.parametrize("fmt,K", FMTS)
def test_special_weights_finite_zero_rows_zero(fmt, K):
    E, N = 2, 37
    w, x, zrows = special_case(fmt, N, K, 3, seed=11, E=E)
    deq = oracle.dequant_rows(fmt, w, E, N, K)
    assert np.isfinite(deq).all()
    assert zrows and (deq[zrows] == 0).all()
    others = np.setdiff1d(np.arange(E * N), zrows)
    assert (np.abs(deq[others]).sum(axis=1) > 0).all()


def test_zero_point_rows_keep_nonzero_scales():
    """The zero rows are zero because of their codes, not their scales."""
    N, K = 4, 512
    for fmt, bb, d_off in ((Q4_K, 144, 0), (Q5_K, 176, 0), (Q6_K, 210, 208), (Q8_0, 34, 0)):
        w, _, _ = special_case(fmt, N, K, 1, seed=3, zero_rows=False)
        z = zero_point_rows(fmt, w, 1, N, K, [1])
        row = z.reshape(N, -1)[1].reshape(-1, bb)
        d = row[:, d_off].astype(np.uint16) | (row[:, d_off + 1].astype(np.uint16) << 8)
        assert (d & 0x7FFF).all()
        if fmt in (Q4_K, Q5_K):
            assert row[:, 4:8].any()  # sub-block scales are non-zero
        if fmt == Q6_K:
            assert (row[:, 192:208] != 0).all()


@pytest.mark.parametrize("fmt,K", FMTS)
def test_specials_reach_the_extremes(fmt, K):
    N = 64
    from synth import rng, weights
    w0 = weights(fmt, rng(5, 0), N, K)
    w = with_specials(fmt, w0, 1, N, K, seed=5)
    deq = oracle.dequant_rows(fmt, w, 1, N, K)
    assert np.isfinite(deq).all()
    a = np.abs(deq)
    nz = a[a > 0]
    if fmt in (Q8_0, Q4_K, Q5_K, Q6_K):
        # fp16 d = 65504 reaches large weights, subnormal d tiny ones
        assert nz.max() > 1e5 and nz.min() < 1e-6
    if fmt == NVFP4:
        assert (np.signbit(deq) & (deq == 0)).any()  # -0 codes / scales
    if fmt == FP8:
        assert nz.max() > 1e30
