"""ctypes binding of liboracle.so (oracle.c), plus its gcc build.

TEST INFRASTRUCTURE ONLY (see oracle.c's header for what is computed and the
passages it follows).  Only tests/, ``__graft_entry__.smoke()`` and bench.py's
cpu_baseline leg may use it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

Q8_0, Q4_K, Q6_K, NVFP4, Q5_K, FP8 = 1, 2, 3, 4, 5, 6
FORMATS = {"Q8_0": Q8_0, "Q4_K": Q4_K, "Q6_K": Q6_K, "NVFP4": NVFP4, "Q5_K": Q5_K, "FP8": FP8}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# QG_ORACLE_LIB names another build of oracle.c to load (the sanitizer runs use it)
_LIB = os.environ.get("QG_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def build(verbose: bool = False, out: str | None = None, sanitize: bool = False) -> str:
    """Compile oracle.c with gcc (plain -O2, no fast-math, no contraction); with
    sanitize, instrumented for AddressSanitizer and UndefinedBehaviorSanitizer."""
    out = out or os.path.join(_HERE, "liboracle.so")
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-shared", "-fPIC", "-Wall", "-Wextra"] + (SANITIZE_FLAGS if sanitize else []) + ["-o", tmp, _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or (not os.environ.get("QG_ORACLE_LIB") and
                                    os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
        build()
    lib = ctypes.CDLL(_LIB)
    ll, i32, vp = ctypes.c_longlong, ctypes.c_int, ctypes.c_void_p
    lib.orc_block_values.argtypes = [i32]
    lib.orc_block_values.restype = ll
    lib.orc_block_bytes.argtypes = [i32]
    lib.orc_block_bytes.restype = ll
    lib.orc_packed_bytes.argtypes = [i32, ll, ll, ll]
    lib.orc_packed_bytes.restype = ll
    lib.orc_dequant_rows.argtypes = [i32, vp, ll, ll, ll, ll, ll, vp]
    lib.orc_dequant_rows.restype = i32
    lib.orc_gemm.argtypes = [i32, vp, ll, ll, ll, ll, vp, vp, ll, vp, vp, vp, i32]
    lib.orc_gemm.restype = i32
    lib.orc_round_bf16.argtypes = [vp, ll, vp]
    lib.orc_round_bf16.restype = None
    lib.orc_moe_block.argtypes = [i32, vp, i32, vp, ll, ll, ll, ll, ll, vp, vp, vp, ll, vp, vp, vp, vp, i32]
    lib.orc_moe_block.restype = i32
    lib.orc_max_threads.argtypes = []
    lib.orc_max_threads.restype = i32
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def block_values(fmt: int) -> int:
    return int(load().orc_block_values(fmt))


def block_bytes(fmt: int) -> int:
    return int(load().orc_block_bytes(fmt))


def packed_bytes(fmt: int, E: int, N: int, K: int) -> int:
    return int(load().orc_packed_bytes(fmt, E, N, K))


def max_threads() -> int:
    return int(load().orc_max_threads())


def _as_bytes(w) -> np.ndarray:
    w = np.ascontiguousarray(w)
    if w.dtype != np.uint8:
        w = w.view(np.uint8)
    return w.reshape(-1)


def dequant_rows(fmt: int, w, E: int, N: int, K: int, r0: int = 0, nr: int | None = None) -> np.ndarray:
    """fp32 [nr, K]: rows r0..r0+nr of the stacked weight[E*N, K]."""
    w = _as_bytes(w)
    if nr is None:
        nr = E * N - r0
    need = packed_bytes(fmt, E, N, K)
    if w.size < need:
        raise ValueError("packed buffer has %d bytes, need %d" % (w.size, need))
    out = np.empty((nr, K), dtype=np.float32)
    rc = load().orc_dequant_rows(fmt, _ptr(w), E, N, K, r0, nr, _ptr(out))
    if rc != 0:
        raise ValueError("orc_dequant_rows rejected its arguments")
    return out


def gemm(fmt: int, w, N: int, K: int, x, E: int = 1, ids=None, cols=None, nthreads: int = 0):
    """(y, bound), both fp64 [M, ncols]: y[m, j] = sum_k w[e*N+cols[j], k] * x[m, k].

    x: bf16 bit patterns, uint16 [M, K] (or a torch bfloat16 CPU tensor).
    ids: int32 [M] stacked-matrix ids, or None (all 0).  cols: output columns, or None (all N).
    """
    w = _as_bytes(w)
    if hasattr(x, "view") and not isinstance(x, np.ndarray):  # torch tensor
        import torch
        x = x.contiguous().view(torch.int16).numpy().view(np.uint16)
    x = np.ascontiguousarray(x, dtype=np.uint16)
    M = x.shape[0] if x.ndim == 2 else 1
    x = x.reshape(M, K)
    need = packed_bytes(fmt, E, N, K)
    if w.size < need:
        raise ValueError("packed buffer has %d bytes, need %d" % (w.size, need))
    if ids is not None:
        ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(-1)
        assert ids.size == M
    if cols is not None:
        cols = np.ascontiguousarray(cols, dtype=np.int64).reshape(-1)
        ncols = cols.size
    else:
        ncols = N
    y = np.empty((M, ncols), dtype=np.float64)
    b = np.empty((M, ncols), dtype=np.float64)
    rc = load().orc_gemm(fmt, _ptr(w), E, N, K, M, _ptr(x),
                         _ptr(ids) if ids is not None else None, ncols,
                         _ptr(cols) if cols is not None else None, _ptr(y), _ptr(b), int(nthreads))
    if rc != 0:
        raise ValueError("orc_gemm rejected its arguments")
    return y, b


def round_bf16(v) -> np.ndarray:
    """bf16 bit patterns (uint16) of fp64 values, rounded once to nearest even."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    load().orc_round_bf16(_ptr(v), v.size, _ptr(out))
    return out


def moe_block(fmt_gu: int, w_gu, fmt_dn: int, w_dn, E: int, D: int, F: int, x, idx, wts, cols=None,
              nthreads: int = 0, want_h: bool = False):
    """(y, bound[, h]) of the mixture-of-experts block (oracle.c, orc_moe_block).

    w_gu: packed weight[E * 2F, D] (rows e*2F .. e*2F+F-1 gate, the next F up);
    w_dn: packed weight[E * D, F]; x: bf16 bits uint16 [T, D]; idx: int32 [T, topk];
    wts: fp32 [T, topk].  y, bound: fp64 [T, ncols]; h: bf16 bits [T * topk, F].
    """
    w_gu, w_dn = _as_bytes(w_gu), _as_bytes(w_dn)
    x = np.ascontiguousarray(x, dtype=np.uint16)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    wts = np.ascontiguousarray(wts, dtype=np.float32)
    T, topk = idx.shape
    x = x.reshape(T, D)
    assert wts.shape == (T, topk)
    if w_gu.size < packed_bytes(fmt_gu, E, 2 * F, D) or w_dn.size < packed_bytes(fmt_dn, E, D, F):
        raise ValueError("packed buffer too small")
    if cols is not None:
        cols = np.ascontiguousarray(cols, dtype=np.int64).reshape(-1)
        ncols = cols.size
    else:
        ncols = D
    y = np.empty((T, ncols), dtype=np.float64)
    b = np.empty((T, ncols), dtype=np.float64)
    h = np.empty((T * topk, F), dtype=np.uint16) if want_h else None
    rc = load().orc_moe_block(fmt_gu, _ptr(w_gu), fmt_dn, _ptr(w_dn), E, D, F, T, topk, _ptr(x), _ptr(idx),
                              _ptr(wts), ncols, _ptr(cols) if cols is not None else None, _ptr(y), _ptr(b),
                              _ptr(h) if want_h else None, int(nthreads))
    if rc != 0:
        raise ValueError("orc_moe_block rejected its arguments")
    return (y, b, h) if want_h else (y, b)
