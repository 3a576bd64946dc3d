"""The C ABI without a GPU: symbols, host-only queries and host-side validation.

Nothing here launches device work: every call either is host-only or is
rejected by argument validation before the HIP runtime is touched.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import gemm_block_quant_amd as qg
import oracle

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "quantgemm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(quant_[a-z_]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 9, names
    L = qg.lib()
    for n in names:
        assert getattr(L, n) is not None, n


def test_packed_bytes_agrees_with_oracle():
    g = np.random.default_rng(0)
    for _ in range(300):
        fmt = int(g.integers(0, 8))
        E = int(g.integers(0, 5))
        N = int(g.integers(0, 3000))
        K = int(g.integers(0, 40)) * 16
        assert qg.quant_packed_bytes(fmt, E, N, K) == oracle.packed_bytes(fmt, E, N, K), (fmt, E, N, K)
    for fmt in (1, 2, 3, 4, 5, 6):
        assert qg.quant_block_values(fmt) == oracle.block_values(fmt)
    assert qg.quant_block_values(0) == 0 and qg.quant_block_values(7) == 0


def test_status_strings():
    for s in range(9):
        assert isinstance(qg.quant_status_string(s), str) and qg.quant_status_string(s)


def _raw(name):
    return getattr(qg.lib(), name)


FAKE_W = ctypes.c_void_p(0x100000)
FAKE_X = ctypes.c_void_p(0x200000)
FAKE_Y = ctypes.c_void_p(0x300000)


def test_validation_rejects_before_launch():
    gemm = _raw("quant_gemm")
    # unknown format, bad K, negative sizes
    assert gemm(FAKE_W, 9, 4, 256, 1, FAKE_X, FAKE_Y, None) == qg.QG_EFORMAT
    assert gemm(FAKE_W, qg.Q4_K, 4, 100, 1, FAKE_X, FAKE_Y, None) == qg.QG_ESHAPE
    assert gemm(FAKE_W, qg.Q4_K, 4, 0, 1, FAKE_X, FAKE_Y, None) == qg.QG_ESHAPE
    assert gemm(FAKE_W, qg.Q4_K, -1, 256, 1, FAKE_X, FAKE_Y, None) == qg.QG_ESHAPE
    assert gemm(FAKE_W, qg.Q4_K, 4, 256, -2, FAKE_X, FAKE_Y, None) == qg.QG_ESHAPE
    assert gemm(FAKE_W, qg.NVFP4, 4, 24, 1, FAKE_X, FAKE_Y, None) == qg.QG_ESHAPE
    assert gemm(FAKE_W, qg.FP8, 4, 96, 1, FAKE_X, FAKE_Y, None) == qg.QG_ESHAPE  # K a multiple of 64
    # empty products are valid no-ops, even with null pointers
    assert gemm(None, qg.Q4_K, 0, 256, 3, None, None, None) == qg.QG_OK
    assert gemm(None, qg.Q4_K, 5, 256, 0, None, None, None) == qg.QG_OK
    # null pointers
    assert gemm(None, qg.Q4_K, 4, 256, 1, FAKE_X, FAKE_Y, None) == qg.QG_EINVAL
    assert gemm(FAKE_W, qg.Q4_K, 4, 256, 1, None, FAKE_Y, None) == qg.QG_EINVAL
    assert gemm(FAKE_W, qg.Q4_K, 4, 256, 1, FAKE_X, None, None) == qg.QG_EINVAL
    # alignment: w and x 16 bytes, y 4 bytes
    assert gemm(ctypes.c_void_p(0x100008), qg.Q4_K, 4, 256, 1, FAKE_X, FAKE_Y, None) == qg.QG_EALIGN
    assert gemm(FAKE_W, qg.Q4_K, 4, 256, 1, ctypes.c_void_p(0x200004), FAKE_Y, None) == qg.QG_EALIGN
    assert gemm(FAKE_W, qg.Q4_K, 4, 256, 1, FAKE_X, ctypes.c_void_p(0x300002), None) == qg.QG_EALIGN
    # K above 2^24: the kernels' LDS arithmetic is int (rejected before any launch)
    assert gemm(FAKE_W, qg.FP8, 4, (1 << 24) + 64, 1, FAKE_X, FAKE_Y, None) == qg.QG_ESHAPE
    assert gemm(FAKE_W, qg.NVFP4, 4, 1 << 29, 1, FAKE_X, FAKE_Y, None) == qg.QG_ESHAPE
    gemv = _raw("quant_gemv")
    assert gemv(FAKE_W, qg.Q8_0, 4, 48, FAKE_X, FAKE_Y, None) == qg.QG_ESHAPE
    deq = _raw("quant_dequantize")
    assert deq(FAKE_W, 0, 4, 256, FAKE_Y, None) == qg.QG_EFORMAT
    assert deq(None, qg.Q6_K, 4, 256, FAKE_Y, None) == qg.QG_EINVAL
    assert deq(FAKE_W, qg.Q6_K, 0, 256, FAKE_Y, None) == qg.QG_OK


def test_read_probe_validation():
    probe = _raw("quant_read_probe")
    sink = ctypes.c_void_p(0x600000)
    assert probe(None, 1024, sink, None) == qg.QG_EINVAL
    assert probe(FAKE_W, 1024, None, None) == qg.QG_EINVAL
    assert probe(ctypes.c_void_p(0x100008), 1024, sink, None) == qg.QG_EALIGN
    assert probe(FAKE_W, 1024, ctypes.c_void_p(0x600002), None) == qg.QG_EALIGN
    assert probe(FAKE_W, 1000, sink, None) == qg.QG_ESHAPE
    assert probe(FAKE_W, 0, sink, None) == qg.QG_OK


def test_grouped_validation():
    grouped = _raw("quant_grouped_gemm")
    E, N, K, M = 4, 8, 256, 3
    wsb = qg.quant_grouped_workspace_bytes(E, M)
    assert wsb > 0
    ws = ctypes.c_void_p(0x400000)
    ids = ctypes.c_void_p(0x500000)
    args = lambda **kw: [kw.get("w", FAKE_W), kw.get("fmt", qg.Q4_K), kw.get("E", E), N, K, kw.get("M", M), FAKE_X,
                         kw.get("ids", ids), FAKE_Y, kw.get("ws", ws), kw.get("wsb", wsb), None]
    assert grouped(*args(E=0)) == qg.QG_ESHAPE
    assert grouped(*args(fmt=7)) == qg.QG_EFORMAT
    assert grouped(*args(ws=None)) == qg.QG_EWORKSPACE
    assert grouped(*args(wsb=wsb - 1)) == qg.QG_EWORKSPACE
    assert grouped(*args(ws=ctypes.c_void_p(0x400004))) == qg.QG_EALIGN
    assert grouped(*args(ids=ctypes.c_void_p(0x500002))) == qg.QG_EALIGN
    assert grouped(*args(M=0, ws=None, wsb=0)) == qg.QG_OK
    assert grouped(*args(M=20000)) == qg.QG_ESHAPE


def test_grouped_k_beyond_lds_is_rejected_before_launch():
    """The grouped product stages a whole activation row in LDS: a K whose row
    cannot fit is rejected with QG_ESHAPE before the bucketing is launched
    (a launch would need a GPU; this container has none)."""
    grouped = _raw("quant_grouped_gemm")
    ws = ctypes.c_void_p(0x400000)
    for fmt, K in ((qg.Q4_K, 19456), (qg.Q5_K, 19456), (qg.Q6_K, 20480), (qg.FP8, 20480), (qg.NVFP4, 20480),
                   (qg.Q8_0, 81920)):
        wsb = qg.quant_grouped_workspace_bytes(2, 3)
        assert grouped(FAKE_W, fmt, 2, 8, K, 3, FAKE_X, None, FAKE_Y, ws, wsb, None) == qg.QG_ESHAPE, (fmt, K)
    moe = _raw("quant_moe_block")
    for D, F in ((19456, 256), (256, 19456)):
        wsb = qg.quant_moe_workspace_bytes(qg.Q4_K, qg.Q4_K, 4, D, F, 2, 2)
        assert wsb == 0, (D, F)
        assert moe(FAKE_W, qg.Q4_K, ctypes.c_void_p(0x700000), qg.Q4_K, 4, D, F, 2, 2, FAKE_X,
                   ctypes.c_void_p(0x500000), ctypes.c_void_p(0x600000), FAKE_Y, ws, 1 << 30, None) == qg.QG_ESHAPE


def test_moe_block_validation():
    moe = _raw("quant_moe_block")
    fg, fd, E, D, F, T, topk = qg.Q4_K, qg.Q6_K, 6, 512, 768, 5, 3
    wsb = qg.quant_moe_workspace_bytes(fg, fd, E, D, F, T, topk)
    # gate|up fp32, bf16 intermediate, down fp32, grouped workspace
    P = T * topk
    assert wsb >= P * 2 * F * 4 + P * F * 2 + P * D * 4 + qg.quant_grouped_workspace_bytes(E, P)
    assert qg.quant_moe_workspace_bytes(fg, fd, E, D + 16, F, T, topk) == 0  # D not a multiple of 256
    assert qg.quant_moe_workspace_bytes(fg, 9, E, D, F, T, topk) == 0
    ws = ctypes.c_void_p(0x400000)
    idx = ctypes.c_void_p(0x500000)
    wts = ctypes.c_void_p(0x600000)
    wd = ctypes.c_void_p(0x700000)

    def args(**kw):
        return [kw.get("wgu", FAKE_W), kw.get("fg", fg), kw.get("wd", wd), kw.get("fd", fd), kw.get("E", E),
                kw.get("D", D), kw.get("F", F), kw.get("T", T), kw.get("topk", topk), kw.get("x", FAKE_X),
                kw.get("idx", idx), kw.get("wts", wts), FAKE_Y, kw.get("ws", ws), kw.get("wsb", wsb), None]

    assert moe(*args(fg=0)) == qg.QG_EFORMAT
    assert moe(*args(fd=9)) == qg.QG_EFORMAT
    assert moe(*args(E=0)) == qg.QG_ESHAPE
    assert moe(*args(topk=0)) == qg.QG_ESHAPE
    assert moe(*args(D=D + 16)) == qg.QG_ESHAPE      # not a multiple of the gate|up block
    assert moe(*args(F=F + 32)) == qg.QG_ESHAPE      # not a multiple of the down block
    assert moe(*args(T=4097, topk=4)) == qg.QG_ESHAPE  # more than 16384 pairs
    assert moe(*args(wd=None)) == qg.QG_EINVAL
    assert moe(*args(wts=None)) == qg.QG_EINVAL
    assert moe(*args(ws=None)) == qg.QG_EWORKSPACE
    assert moe(*args(wsb=wsb - 1)) == qg.QG_EWORKSPACE
    assert moe(*args(idx=ctypes.c_void_p(0x500002))) == qg.QG_EALIGN
    assert moe(*args(wts=ctypes.c_void_p(0x600001))) == qg.QG_EALIGN
    assert moe(*args(x=ctypes.c_void_p(0x200008))) == qg.QG_EALIGN
    assert moe(*args(T=0, ws=None, wsb=0)) == qg.QG_OK


def test_missing_library_raises_instead_of_falling_back():
    """Without the built library every entry point raises: there is no CPU path."""
    import subprocess
    import sys
    code = ("import gemm_block_quant_amd as qg\n"
            "qg.LIB_PATH = '/nonexistent/libquantgemm.so'\n"
            "try:\n"
            "    qg.quant_packed_bytes(qg.Q4_K, 1, 4, 256)\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n"
            "else:\n"
            "    print('no error')\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120, cwd=root)
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("raised:") and "not built" in r.stdout


def test_streamk_validation():
    """quant_gemm_streamk: workspace sizing and the checks made before any launch."""
    sk = _raw("quant_gemm_streamk")
    fmt, N, K, M = qg.NVFP4, 5120, 17408, 512  # 320 tiles of 128 x 64 for 2 workgroups per CU
    wsb = qg.quant_gemm_streamk_workspace_bytes(fmt, N, K, M)
    # per-tile counters and two 128 x 64 fp32 partial tiles per workgroup
    assert wsb > 2 * 128 * 64 * 4, wsb
    assert qg.quant_gemm_streamk_workspace_bytes(fmt, N, K, 16) == 0  # not on the tiles
    assert qg.quant_gemm_streamk_workspace_bytes(fmt, 17408, 5120, 4096) == 0  # more tiles than slots
    assert qg.quant_gemm_streamk_workspace_bytes(qg.Q4_K, 200, 256, 300) == 0  # few tiles: plain schedule
    assert qg.quant_gemm_streamk_workspace_bytes(9, N, K, M) == 0
    assert qg.quant_gemm_streamk_workspace_bytes(fmt, N, 100, M) == 0
    ws = ctypes.c_void_p(0x400000)
    args = lambda **kw: [kw.get("w", FAKE_W), kw.get("fmt", fmt), N, K, kw.get("M", M), FAKE_X, FAKE_Y,
                         kw.get("ws", ws), kw.get("wsb", wsb), None]
    assert sk(*args(ws=None)) == qg.QG_EWORKSPACE
    assert sk(*args(wsb=wsb - 1)) == qg.QG_EWORKSPACE
    assert sk(*args(ws=ctypes.c_void_p(0x400008))) == qg.QG_EALIGN
    assert sk(*args(w=None)) == qg.QG_EINVAL
    assert sk(*args(w=ctypes.c_void_p(0x100008))) == qg.QG_EALIGN
    assert sk(*args(fmt=9)) == qg.QG_EFORMAT
    assert sk(*args(M=0, ws=None, wsb=0)) == qg.QG_OK
