"""GPU parity of the mixture-of-experts block (gate|up grouped product, SwiGLU
to bf16, down grouped product, routing-weighted combine) against the oracle."""
import numpy as np
import pytest

import gemm_block_quant_amd as qg
import oracle
import synth
from helpers import assert_band, dev_bytes, dev_x, same_bits

pytestmark = pytest.mark.gpu


def _dev(a, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=dtype)).cuda()


def _case(fg, fd, E, D, F, T, topk, seed):
    w_gu = synth.weights(fg, synth.rng(seed, 0), E * 2 * F, D, E=E)
    w_dn = synth.weights(fd, synth.rng(seed, 1), E * D, F, E=E)
    x = synth.x_bf16(synth.rng(seed, 2), T, D)
    idx = synth.routing(synth.rng(seed, 3), T, topk, E).reshape(T, topk)
    wts = synth.routing_weights(synth.rng(seed, 4), T, topk)
    return w_gu, w_dn, x, idx, wts


def _run(fg, w_gu, fd, w_dn, E, D, F, x, idx, wts):
    return qg.quant_moe_block(dev_bytes(w_gu), fg, dev_bytes(w_dn), fd, E, D, F, dev_x(x), _dev(idx, np.int32),
                              _dev(wts, np.float32)).cpu().numpy()


@pytest.mark.parametrize("fg,fd,E,D,F,T,topk", [
    (qg.Q4_K, qg.Q4_K, 6, 512, 768, 5, 3),
    (qg.Q4_K, qg.Q6_K, 6, 512, 768, 7, 2),
    (qg.Q5_K, qg.Q6_K, 4, 256, 512, 4, 4),
    (qg.NVFP4, qg.NVFP4, 5, 592, 288, 6, 2),  # D % 64 = 16: the row-buffer path for gate|up
    (qg.Q8_0, qg.Q8_0, 5, 1024, 512, 3, 3),
    (qg.Q4_K, qg.Q4_K, 40, 1024, 512, 16, 8),  # experts shared across tokens
    (qg.FP8, qg.FP8, 6, 512, 768, 5, 3),
])
def test_moe_block_band(fg, fd, E, D, F, T, topk):
    w_gu, w_dn, x, idx, wts = _case(fg, fd, E, D, F, T, topk, 31 + E + T)
    if T > 2:
        idx[T - 1] = idx[0]  # a token routed exactly like the first
    y = _run(fg, w_gu, fd, w_dn, E, D, F, x, idx, wts)
    y_ref, bound = oracle.moe_block(fg, w_gu, fd, w_dn, E, D, F, x, idx, wts)
    assert_band(y, y_ref, bound, "moe %d/%d E %d D %d F %d T %d k %d" % (fg, fd, E, D, F, T, topk))


def test_moe_block_invalid_id_and_repeat():
    fg, fd, E, D, F, T, topk = qg.Q4_K, qg.Q6_K, 6, 512, 512, 5, 3
    w_gu, w_dn, x, idx, wts = _case(fg, fd, E, D, F, T, topk, 40)
    idx[1, 2] = E       # out of range
    idx[3, 0] = -1      # negative
    idx[4] = idx[4, 0]  # one expert three times
    y = _run(fg, w_gu, fd, w_dn, E, D, F, x, idx, wts)
    y_ref, bound = oracle.moe_block(fg, w_gu, fd, w_dn, E, D, F, x, idx, wts)
    bad = np.array([False, True, False, True, False])
    assert np.isnan(y[bad]).all()
    assert not np.isnan(y[~bad]).any()
    assert_band(y[~bad], y_ref[~bad], bound[~bad], "moe with invalid ids")
    again = _run(fg, w_gu, fd, w_dn, E, D, F, x, idx, wts)
    assert same_bits(again, y)


def test_moe_block_token_independent_of_batch():
    """A token's row does not depend on the other tokens of the call (each
    expert's rows are summed in a fixed order whatever else is routed to it)."""
    fg, fd, E, D, F, T, topk = qg.Q4_K, qg.Q4_K, 12, 1024, 512, 9, 4
    w_gu, w_dn, x, idx, wts = _case(fg, fd, E, D, F, T, topk, 41)
    y = _run(fg, w_gu, fd, w_dn, E, D, F, x, idx, wts)
    for t in (0, 4, 8):
        yt = _run(fg, w_gu, fd, w_dn, E, D, F, x[t:t + 1], idx[t:t + 1], wts[t:t + 1])
        assert same_bits(yt[0], y[t]), t


def test_moe_block_glm_shape():
    """D = 4096, F = 2048, 16 tokens x top-8 over 32 experts (the expert shape of
    the 288-expert layer; fewer experts keep the host copy small)."""
    fg, fd, E, D, F, T, topk = qg.Q4_K, qg.Q4_K, 32, 4096, 2048, 16, 8
    w_gu, w_dn, x, idx, wts = _case(fg, fd, E, D, F, T, topk, 42)
    y = _run(fg, w_gu, fd, w_dn, E, D, F, x, idx, wts)
    y_ref, bound = oracle.moe_block(fg, w_gu, fd, w_dn, E, D, F, x, idx, wts)
    assert_band(y, y_ref, bound, "moe GLM shape")


@pytest.mark.parametrize("fg,fd", [(qg.Q4_K, qg.Q6_K), (qg.NVFP4, qg.FP8)])
def test_moe_block_prefill_large_experts(fg, fd):
    """Prefill-sized routing: 64 tokens x top-4 over 8 experts, so most experts
    get 32 or more pairs (the matrix-core tiles) and some fewer (streaming);
    every output against the oracle."""
    E, D, F, T, topk = 8, 256, 512, 64, 4
    w_gu, w_dn, x, idx, wts = _case(fg, fd, E, D, F, T, topk, 90 + fg)
    idx[5] = [0, 1, 2, 3]  # make sure expert 0..3 are shared widely
    counts = np.bincount(idx.ravel(), minlength=E)
    assert counts.max() >= 32
    y = _run(fg, w_gu, fd, w_dn, E, D, F, x, idx, wts)
    y_ref, bound = oracle.moe_block(fg, w_gu, fd, w_dn, E, D, F, x, idx, wts)
    assert_band(y, y_ref, bound, "moe prefill %d/%d" % (fg, fd))
