"""The allocation-free grouped entry point against the one with a workspace.

quant_grouped_gemm_noalloc runs the same kernels as quant_grouped_gemm with the
library's static per-GPU scratch in place of the caller's workspace, so its
outputs must equal the workspace entry point's bit for bit (and the oracle's
band).  Two calls in a row, the second smaller, check that nothing a call
reads is left over from the previous call's scratch contents.
"""
import ctypes

import numpy as np
import pytest

import gemm_block_quant_amd as qg
import oracle
import synth
from helpers import assert_band, dev_bytes, dev_x, same_bits

pytestmark = pytest.mark.gpu


def _case(fmt, E, N, K, M, seed):
    w = synth.weights(fmt, synth.rng(seed, 0), E * N, K, E=E)
    x = synth.x_bf16(synth.rng(seed, 1), M, K)
    ids = np.random.default_rng(seed).integers(0, E, M).astype(np.int32)
    ids[M // 3] = E  # out of range: a NaN row
    return w, x, ids


@pytest.mark.parametrize("fmt", [qg.Q4_K, qg.Q6_K, qg.Q8_0, qg.NVFP4, qg.FP8])
def test_noalloc_equals_workspace_entry_point_twice(fmt):
    import torch
    L = qg.lib()
    fn = L.quant_grouped_gemm_noalloc
    # each call smaller than the one before; the first puts experts on the
    # matrix-core tiles (about 100 rows each), whose tile lists live in the scratch too
    for E, N, K, M, seed in ((4, 96, 1024, 400, 80), (40, 130, 2048, 300, 81), (6, 70, 1024, 9, 82)):
        w, x, ids = _case(fmt, E, N, K, M, seed + fmt)
        wd, xd, idd = dev_bytes(w), dev_x(x), torch.from_numpy(ids).cuda()
        y_ws = qg.quant_grouped_gemm(wd, fmt, E, N, K, M, xd, idd).cpu().numpy()
        y = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
        st = fn(ctypes.c_void_p(wd.data_ptr()), fmt, E, N, K, M, ctypes.c_void_p(xd.data_ptr()),
                ctypes.c_void_p(idd.data_ptr()), ctypes.c_void_p(y.data_ptr()),
                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == qg.QG_OK, qg.quant_status_string(st)
        y = y.cpu().numpy()
        assert same_bits(y, y_ws), (fmt, E, N, K, M)
        bad = ids >= E
        assert np.isnan(y[bad]).all()
        y_ref, bound = oracle.gemm(fmt, w, N, K, x, E=E, ids=ids)
        assert_band(y[~bad], y_ref[~bad], bound[~bad], "noalloc fmt %d M %d" % (fmt, M))


def test_noalloc_binding_and_validation():
    """The Python binding, and host-side validation before any launch."""
    import torch
    fmt, E, N, K, M = qg.Q4_K, 5, 64, 512, 12
    w, x, ids = _case(fmt, E, N, K, M, 83)
    ids[M // 3] = 0
    wd, xd, idd = dev_bytes(w), dev_x(x), torch.from_numpy(ids).cuda()
    y = qg.quant_grouped_gemm_noalloc(wd, fmt, E, N, K, M, xd, idd).cpu().numpy()
    assert same_bits(y, qg.quant_grouped_gemm(wd, fmt, E, N, K, M, xd, idd).cpu().numpy())
    fn = qg.lib().quant_grouped_gemm_noalloc
    p = ctypes.c_void_p(wd.data_ptr())
    assert fn(p, fmt, E, N, K, 16385, p, None, p, None) == qg.QG_ESHAPE
    assert fn(None, fmt, E, N, K, M, p, None, p, None) == qg.QG_EINVAL
    assert fn(p, fmt, E, N, K, 0, None, None, None, None) == qg.QG_OK
