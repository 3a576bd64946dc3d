"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module draws random field values and places them at their byte positions
in the packed tensors.  It holds none of the product's arithmetic: it never
decodes a block.  Both the CPU oracle and the GPU library consume its output.

Stream keys: numpy PCG64 seeded with SeedSequence([config_seed, tensor_id]).
Tensor ids: 0 = weights, 1 = x, 2 = routing ids, 3 = the second activation of
the expert down projection.

Distributions (the workloads of the weight-streaming decode path: Qwen3.8-27B
hidden 5,120 / MLP 17,408 / vocab 248,320 and the 288-expert, 4096x2048 MoE):
  Q8_0  : q uniform int8 in [-127, 127]; d = fp16(|N(0,1)| * 0.01)
  Q4_K  : 4-bit codes and 6-bit scales/mins uniform (all 12 scale bytes and 128
          code bytes uniform); d, dmin = fp16(0.01 * (0.5 + U)) per super-block
  Q5_K  : as Q4_K, with the 32 fifth-bit bytes uniform (5-bit codes uniform)
  Q6_K  : 6-bit codes uniform (ql, qh bytes uniform); int8 sub-scales uniform in
          [-128, 127]; d = fp16(|N(0,1)| * 0.01)
  NVFP4 : code bytes uniform (each E2M1 nibble uniform over 16 values); block
          scale = e4m3fn(|N(0,1)|); per-tensor scale g = f32(0.01 * (1 + U))
  FP8   : E4M3 code bytes uniform over the 254 finite codes (the two NaN codes
          drawn are replaced by 0); row scale = f32(0.01 * (0.5 + U) / 448)
  x     : bf16(N(0,1))
  ids   : per token, k distinct experts drawn uniformly from E (token-major rows)
All float narrowing rounds to nearest even (numpy / torch conversions).
"""
from __future__ import annotations

import numpy as np

Q8_0, Q4_K, Q6_K, NVFP4, Q5_K, FP8 = 1, 2, 3, 4, 5, 6
QK = {Q8_0: 32, Q4_K: 256, Q6_K: 256, NVFP4: 16, Q5_K: 256, FP8: 64}
BLOCK_BYTES = {Q8_0: 34, Q4_K: 144, Q6_K: 210, Q5_K: 176}


def rng(config_seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(config_seed), int(tensor_id)])))


def _random_bytes(g: np.random.Generator, n: int) -> np.ndarray:
    """n uniform bytes: the stream of g.bytes(n) (ceil(n / 4) uniform uint32,
    little endian), drawn through integers(), which is several times faster."""
    n = int(n)
    if n == 0:
        return np.empty(0, dtype=np.uint8)
    w = g.integers(0, 1 << 32, size=(n - 1) // 4 + 1, dtype=np.uint32).astype("<u4", copy=False)
    return w.view(np.uint8)[:n].copy()


def _fp16_bytes(v: np.ndarray) -> np.ndarray:
    """[n] float64 -> [n, 2] little-endian fp16 bytes (round to nearest even)."""
    return np.ascontiguousarray(v.astype(np.float16)).view(np.uint8).reshape(-1, 2)


def q8_0(g: np.random.Generator, rows: int, K: int) -> np.ndarray:
    nb = rows * (K // 32)
    buf = np.empty((nb, 34), dtype=np.uint8)
    buf[:, 0:2] = _fp16_bytes(np.abs(g.standard_normal(nb)) * 0.01)
    buf[:, 2:34] = g.integers(-127, 128, size=(nb, 32), dtype=np.int8).view(np.uint8)
    return buf.reshape(-1)


def q4_k(g: np.random.Generator, rows: int, K: int) -> np.ndarray:
    nb = rows * (K // 256)
    buf = _random_bytes(g, nb * 144).reshape(nb, 144)
    buf[:, 0:2] = _fp16_bytes(0.01 * (0.5 + g.random(nb)))
    buf[:, 2:4] = _fp16_bytes(0.01 * (0.5 + g.random(nb)))
    return buf.reshape(-1)


def q5_k(g: np.random.Generator, rows: int, K: int) -> np.ndarray:
    nb = rows * (K // 256)
    buf = _random_bytes(g, nb * 176).reshape(nb, 176)
    buf[:, 0:2] = _fp16_bytes(0.01 * (0.5 + g.random(nb)))
    buf[:, 2:4] = _fp16_bytes(0.01 * (0.5 + g.random(nb)))
    return buf.reshape(-1)


def q6_k(g: np.random.Generator, rows: int, K: int) -> np.ndarray:
    nb = rows * (K // 256)
    buf = _random_bytes(g, nb * 210).reshape(nb, 210)
    buf[:, 208:210] = _fp16_bytes(np.abs(g.standard_normal(nb)) * 0.01)
    return buf.reshape(-1)


def e4m3_bytes(v: np.ndarray) -> np.ndarray:
    """float values -> E4M3-fn bytes (torch's round-to-nearest-even conversion)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def nvfp4(g: np.random.Generator, rows: int, K: int, E: int = 1) -> np.ndarray:
    """Planes [codes rows*K/2][scales rows*K/16][g: E fp32], rows = E*N."""
    codes = _random_bytes(g, rows * K // 2)
    scales = e4m3_bytes(np.abs(g.standard_normal(rows * K // 16)))
    gs = (0.01 * (1.0 + g.random(E))).astype(np.float32).view(np.uint8)
    return np.concatenate([codes, scales, gs])


def fp8(g: np.random.Generator, rows: int, K: int) -> np.ndarray:
    """Planes [codes rows*K][row scales: rows fp32]."""
    codes = _random_bytes(g, rows * K)
    codes[(codes & 0x7F) == 0x7F] = 0
    scales = (0.01 * (0.5 + g.random(rows)) / 448.0).astype(np.float32).view(np.uint8)
    return np.concatenate([codes, scales])


def weights(fmt: int, g: np.random.Generator, rows: int, K: int, E: int = 1) -> np.ndarray:
    """Packed weight[rows, K] (rows = E*N for a stacked tensor) as flat uint8."""
    if K % QK[fmt]:
        raise ValueError("K=%d is not a multiple of the block (%d)" % (K, QK[fmt]))
    if fmt == Q8_0:
        return q8_0(g, rows, K)
    if fmt == Q4_K:
        return q4_k(g, rows, K)
    if fmt == Q6_K:
        return q6_k(g, rows, K)
    if fmt == Q5_K:
        return q5_k(g, rows, K)
    if fmt == NVFP4:
        return nvfp4(g, rows, K, E)
    if fmt == FP8:
        return fp8(g, rows, K)
    raise ValueError("unknown format %r" % fmt)


def bf16_bits(v: np.ndarray) -> np.ndarray:
    """float values -> bf16 bit patterns (uint16), via fp32, round to nearest even."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def x_bf16(g: np.random.Generator, M: int, K: int) -> np.ndarray:
    """bf16(N(0,1)) activations as uint16 bit patterns [M, K]."""
    return bf16_bits(g.standard_normal((M, K))).reshape(M, K)


def routing(g: np.random.Generator, tokens: int, k: int, E: int) -> np.ndarray:
    """int32 [tokens*k]: row k*t+j is token t's j-th expert; a token's k ids are distinct."""
    ids = np.empty((tokens, k), dtype=np.int32)
    for t in range(tokens):
        ids[t] = g.choice(E, size=k, replace=False)
    return ids.reshape(-1)


def routing_weights(g: np.random.Generator, tokens: int, k: int) -> np.ndarray:
    """fp32 [tokens, k]: a softmax over k standard normals per token (positive, rows sum to ~1)."""
    z = g.standard_normal((tokens, k))
    e = np.exp(z - z.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
