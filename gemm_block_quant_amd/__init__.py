"""Python binding of libquantgemm (MI355X / gfx950 block-quantized GEMV and GEMM).

Argument marshalling only: every step of the product runs in the library's HIP
kernels.  Tensors are torch tensors on the ROCm device; torch provides device
memory and the current stream, nothing else.  The entry points mirror the C ABI
in include/quantgemm.h:

    quant_gemv(w, fmt, N, K, x, y=None)                     -> y [N] fp32
    quant_gemm(w, fmt, N, K, M, x, y=None)                  -> y [M, N] fp32
    quant_gemm_streamk(w, fmt, N, K, M, x, y=None, workspace=None) -> y [M, N] fp32
    quant_grouped_gemm(w, fmt, E, N, K, M, x, ids, y=None, workspace=None) -> y [M, N]
    quant_grouped_gemm_noalloc(w, fmt, E, N, K, M, x, ids, y=None)  -> y [M, N]
    quant_dequantize(w, fmt, rows, K, out=None)             -> out [rows, K] fp32
    quant_dequantize_stacked(w, fmt, E, N, K, out=None)     -> out [E*N, K] fp32
    quant_packed_bytes(fmt, E, N, K), quant_grouped_workspace_bytes(E, M),
    quant_gemm_streamk_workspace_bytes(fmt, N, K, M),
    quant_block_values(fmt), quant_status_string(status)

w is a uint8 tensor holding the packed bytes; x holds bf16 activations
(torch.bfloat16, or int16/uint16 bit patterns).  A missing library raises.
"""
from __future__ import annotations

import ctypes
import os

Q8_0, Q4_K, Q6_K, NVFP4, Q5_K, FP8 = 1, 2, 3, 4, 5, 6
FORMATS = {"Q8_0": Q8_0, "Q4_K": Q4_K, "Q6_K": Q6_K, "NVFP4": NVFP4, "Q5_K": Q5_K, "FP8": FP8}

QG_OK, QG_EINVAL, QG_EFORMAT, QG_EALIGN, QG_ESHAPE, QG_EHIP, QG_ENOTIMPL, QG_EWORKSPACE = range(8)

# QUANTGEMM_LIB names another build of the library to load (e.g. the sanitizer build)
LIB_PATH = os.environ.get("QUANTGEMM_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libquantgemm.so")

_lib = None


class QuantGemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, quant_status_string(status), status))


def lib():
    """The loaded libquantgemm.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libquantgemm.so is not built (%s); run `python -m gemm_block_quant_amd.build`" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    L.quant_block_values.argtypes = [i32]
    L.quant_block_values.restype = i64
    L.quant_packed_bytes.argtypes = [i32, i64, i64, i64]
    L.quant_packed_bytes.restype = sz
    L.quant_gemv.argtypes = [vp, i32, i64, i64, vp, vp, vp]
    L.quant_gemv.restype = i32
    L.quant_gemm.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp]
    L.quant_gemm.restype = i32
    L.quant_grouped_workspace_bytes.argtypes = [i64, i64]
    L.quant_grouped_workspace_bytes.restype = sz
    L.quant_gemm_streamk_workspace_bytes.argtypes = [i32, i64, i64, i64]
    L.quant_gemm_streamk_workspace_bytes.restype = sz
    L.quant_gemm_streamk.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp, sz, vp]
    L.quant_gemm_streamk.restype = i32
    L.quant_grouped_gemm.argtypes = [vp, i32, i64, i64, i64, i64, vp, vp, vp, vp, sz, vp]
    L.quant_grouped_gemm.restype = i32
    L.quant_grouped_gemm_noalloc.argtypes = [vp, i32, i64, i64, i64, i64, vp, vp, vp, vp]
    L.quant_grouped_gemm_noalloc.restype = i32
    L.quant_dequantize.argtypes = [vp, i32, i64, i64, vp, vp]
    L.quant_dequantize.restype = i32
    L.quant_dequantize_stacked.argtypes = [vp, i32, i64, i64, i64, vp, vp]
    L.quant_dequantize_stacked.restype = i32
    L.quant_status_string.argtypes = [i32]
    L.quant_status_string.restype = ctypes.c_char_p
    L.quant_moe_workspace_bytes.argtypes = [i32, i32, i64, i64, i64, i64, i64]
    L.quant_moe_workspace_bytes.restype = sz
    L.quant_moe_block.argtypes = [vp, i32, vp, i32, i64, i64, i64, i64, i64, vp, vp, vp, vp, vp, sz, vp]
    L.quant_moe_block.restype = i32
    L.quant_read_probe.argtypes = [vp, sz, vp, vp]
    L.quant_read_probe.restype = i32
    _lib = L
    return L


# ---------------------------------------------------------------- host-only queries

def quant_block_values(fmt: int) -> int:
    return int(lib().quant_block_values(fmt))


def quant_packed_bytes(fmt: int, E: int, N: int, K: int) -> int:
    return int(lib().quant_packed_bytes(fmt, E, N, K))


def quant_grouped_workspace_bytes(E: int, M: int) -> int:
    return int(lib().quant_grouped_workspace_bytes(E, M))


def quant_status_string(status: int) -> str:
    return lib().quant_status_string(status).decode()


# ---------------------------------------------------------------- marshalling helpers

def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _dev_ptr(t, name, nbytes=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if nbytes is not None and t.numel() * t.element_size() < nbytes:
        raise ValueError("%s holds %d bytes, needs %d" % (name, t.numel() * t.element_size(), nbytes))
    return ctypes.c_void_p(t.data_ptr())


def _x_ptr(x, M, K):
    torch = _torch()
    if x.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise ValueError("x must be bfloat16 (or 16-bit bf16 bit patterns)")
    return _dev_ptr(x, "x", 2 * M * K)


def _out(y, shape, device):
    torch = _torch()
    if y is None:
        return torch.empty(shape, dtype=torch.float32, device=device)
    if y.dtype != torch.float32:
        raise ValueError("y must be float32")
    return y


def _check(status, where):
    if status != QG_OK:
        raise QuantGemmError(status, where)


# ---------------------------------------------------------------- products

def quant_gemm(w, fmt: int, N: int, K: int, M: int, x, y=None, stream=None):
    """y[m, n] = sum_k W[n, k] x[m, k]; W packed [N, K] in w, x bf16 [M, K]."""
    y = _out(y, (M, N), x.device)
    st = lib().quant_gemm(_dev_ptr(w, "w", quant_packed_bytes(fmt, 1, N, K)), fmt, N, K, M, _x_ptr(x, M, K),
                          _dev_ptr(y, "y", 4 * M * N), _stream(stream))
    _check(st, "quant_gemm")
    return y


def quant_gemm_streamk_workspace_bytes(fmt: int, N: int, K: int, M: int) -> int:
    return int(lib().quant_gemm_streamk_workspace_bytes(fmt, N, K, M))


def quant_gemm_streamk(w, fmt: int, N: int, K: int, M: int, x, y=None, workspace=None, stream=None):
    """quant_gemm with the matrix-core tiles dealt evenly over the GPU (stream-K);
    workspace: uint8 device tensor of quant_gemm_streamk_workspace_bytes bytes
    (allocated here when None)."""
    torch = _torch()
    y = _out(y, (M, N), x.device)
    wsb = quant_gemm_streamk_workspace_bytes(fmt, N, K, M)
    if workspace is None:
        workspace = torch.empty(max(wsb, 16), dtype=torch.uint8, device=x.device)
    st = lib().quant_gemm_streamk(_dev_ptr(w, "w", quant_packed_bytes(fmt, 1, N, K)), fmt, N, K, M, _x_ptr(x, M, K),
                                  _dev_ptr(y, "y", 4 * M * N), _dev_ptr(workspace, "workspace"),
                                  workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "quant_gemm_streamk")
    return y


def quant_gemv(w, fmt: int, N: int, K: int, x, y=None, stream=None):
    """y[n] = sum_k W[n, k] x[k]; W packed [N, K] in w, x bf16 [K]."""
    y = _out(y, (N,), x.device)
    st = lib().quant_gemv(_dev_ptr(w, "w", quant_packed_bytes(fmt, 1, N, K)), fmt, N, K, _x_ptr(x, 1, K),
                          _dev_ptr(y, "y", 4 * N), _stream(stream))
    _check(st, "quant_gemv")
    return y


def quant_grouped_gemm(w, fmt: int, E: int, N: int, K: int, M: int, x, ids=None, y=None, workspace=None,
                       stream=None):
    """y[i, n] = sum_k W_{ids[i]}[n, k] x[i, k] over stacked weight[E*N, K]; ids int32 [M] or None."""
    torch = _torch()
    y = _out(y, (M, N), x.device)
    wsb = quant_grouped_workspace_bytes(E, M)
    if workspace is None:
        workspace = torch.empty(max(wsb, 16), dtype=torch.uint8, device=x.device)
    if ids is not None and ids.dtype != torch.int32:
        raise ValueError("ids must be int32")
    st = lib().quant_grouped_gemm(_dev_ptr(w, "w", quant_packed_bytes(fmt, E, N, K)), fmt, E, N, K, M,
                                  _x_ptr(x, M, K), _dev_ptr(ids, "ids", 4 * M) if ids is not None else None,
                                  _dev_ptr(y, "y", 4 * M * N), _dev_ptr(workspace, "workspace"),
                                  workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "quant_grouped_gemm")
    return y


def quant_grouped_gemm_noalloc(w, fmt: int, E: int, N: int, K: int, M: int, x, ids=None, y=None, stream=None):
    """quant_grouped_gemm with the library's static per-GPU scratch instead of a
    workspace (nothing is allocated by the library; y is allocated here when
    not given).  Calls on one GPU must be ordered on one stream."""
    torch = _torch()
    y = _out(y, (M, N), x.device)
    if ids is not None and ids.dtype != torch.int32:
        raise ValueError("ids must be int32")
    st = lib().quant_grouped_gemm_noalloc(_dev_ptr(w, "w", quant_packed_bytes(fmt, E, N, K)), fmt, E, N, K, M,
                                          _x_ptr(x, M, K), _dev_ptr(ids, "ids", 4 * M) if ids is not None else None,
                                          _dev_ptr(y, "y", 4 * M * N), _stream(stream))
    _check(st, "quant_grouped_gemm_noalloc")
    return y


def quant_moe_workspace_bytes(fmt_gate_up: int, fmt_down: int, E: int, D: int, F: int, T: int, topk: int) -> int:
    return int(lib().quant_moe_workspace_bytes(fmt_gate_up, fmt_down, E, D, F, T, topk))


def quant_moe_block(w_gate_up, fmt_gate_up: int, w_down, fmt_down: int, E: int, D: int, F: int, x, idx, wts,
                    y=None, workspace=None, stream=None):
    """y[t] = sum_j wts[t, j] * down_e(bf16(silu(gate_e x[t]) * up_e x[t])), e = idx[t, j].

    w_gate_up: packed weight[E*2F, D] (gate rows then up rows per expert); w_down:
    packed weight[E*D, F]; x: bf16 [T, D]; idx: int32 [T, topk]; wts: fp32 [T, topk].
    """
    torch = _torch()
    T, topk = idx.shape
    if idx.dtype != torch.int32 or wts.dtype != torch.float32:
        raise ValueError("idx must be int32 and wts float32")
    if tuple(wts.shape) != (T, topk):
        raise ValueError("wts must have the shape of idx")
    y = _out(y, (T, D), x.device)
    wsb = quant_moe_workspace_bytes(fmt_gate_up, fmt_down, E, D, F, T, topk)
    if workspace is None:
        workspace = torch.empty(max(wsb, 16), dtype=torch.uint8, device=x.device)
    st = lib().quant_moe_block(_dev_ptr(w_gate_up, "w_gate_up", quant_packed_bytes(fmt_gate_up, E, 2 * F, D)),
                               fmt_gate_up, _dev_ptr(w_down, "w_down", quant_packed_bytes(fmt_down, E, D, F)),
                               fmt_down, E, D, F, T, topk, _x_ptr(x, T, D), _dev_ptr(idx, "idx", 4 * T * topk),
                               _dev_ptr(wts, "wts", 4 * T * topk), _dev_ptr(y, "y", 4 * T * D),
                               _dev_ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                               _stream(stream))
    _check(st, "quant_moe_block")
    return y


def quant_dequantize(w, fmt: int, rows: int, K: int, out=None, stream=None):
    """fp32 [rows, K] dequantization of a packed weight[rows, K] (bit-exact)."""
    out = _out(out, (rows, K), w.device)
    st = lib().quant_dequantize(_dev_ptr(w, "w", quant_packed_bytes(fmt, 1, rows, K)), fmt, rows, K,
                                _dev_ptr(out, "out", 4 * rows * K), _stream(stream))
    _check(st, "quant_dequantize")
    return out


def quant_dequantize_stacked(w, fmt: int, E: int, N: int, K: int, out=None, stream=None):
    """fp32 [E*N, K] dequantization of a stacked weight[E*N, K] (bit-exact)."""
    out = _out(out, (E * N, K), w.device)
    st = lib().quant_dequantize_stacked(_dev_ptr(w, "w", quant_packed_bytes(fmt, E, N, K)), fmt, E, N, K,
                                        _dev_ptr(out, "out", 4 * E * N * K), _stream(stream))
    _check(st, "quant_dequantize_stacked")
    return out


def quant_read_probe(buf, sink, stream=None):
    """Plain streaming read of every byte of the device tensor `buf` (a
    measurement reference, not part of the product path); `sink` is a device
    int32/uint32 tensor of at least one element."""
    nbytes = buf.numel() * buf.element_size()
    st = lib().quant_read_probe(_dev_ptr(buf, "buf", nbytes), nbytes, _dev_ptr(sink, "sink", 4), _stream(stream))
    _check(st, "quant_read_probe")
