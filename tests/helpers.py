"""Shared helpers for the GPU parity tests: device transfer and the error band."""
from __future__ import annotations

import numpy as np

import oracle
import synth

# |y - y_ref| <= BAND * sum_k |w x| per output element
BAND = 2e-3

FMT_NAMES = {1: "Q8_0", 2: "Q4_K", 3: "Q6_K", 4: "NVFP4"}


def dev_bytes(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def dev_x(xb: np.ndarray):
    """bf16 bit patterns (uint16 [M, K]) -> device int16 tensor (the binding passes them as bf16)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).cuda()


def make_case(fmt: int, N: int, K: int, M: int, seed: int, E: int = 1):
    w = synth.weights(fmt, synth.rng(seed, 0), E * N, K, E=E)
    x = synth.x_bf16(synth.rng(seed, 1), M, K)
    return w, x


def band_violations(y_gpu: np.ndarray, y_ref: np.ndarray, bound: np.ndarray) -> int:
    """Elements outside the band (NaN anywhere counts as a violation)."""
    y_gpu = np.asarray(y_gpu, np.float64)
    err = np.abs(y_gpu - y_ref)
    ok = err <= BAND * bound
    return int(np.size(ok) - np.count_nonzero(ok))


def assert_band(y_gpu, y_ref, bound, what=""):
    bad = band_violations(y_gpu, y_ref, bound)
    if bad:
        y_gpu = np.asarray(y_gpu, np.float64)
        rel = np.abs(y_gpu - y_ref) / np.maximum(bound, 1e-300)
        i = np.unravel_index(np.nanargmax(np.where(np.isnan(rel), np.inf, rel)), rel.shape)
        raise AssertionError("%s: %d of %d outside |y-ref| <= %g*sum|wx|; worst at %s: gpu %r ref %r bound %r"
                             % (what, bad, y_gpu.size, BAND, i, y_gpu[i], y_ref[i], bound[i]))


def same_bits(a: np.ndarray, b: np.ndarray) -> bool:
    """Bit-for-bit equality of fp32 arrays, with any NaN matching any NaN."""
    a = np.ascontiguousarray(a, np.float32)
    b = np.ascontiguousarray(b, np.float32)
    if a.shape != b.shape:
        return False
    na, nb = np.isnan(a), np.isnan(b)
    if not np.array_equal(na, nb):
        return False
    return np.array_equal(a.view(np.uint32)[~na], b.view(np.uint32)[~nb])


def oracle_product(fmt, w, N, K, x, E=1, ids=None, cols=None):
    return oracle.gemm(fmt, w, N, K, x, E=E, ids=ids, cols=cols)
