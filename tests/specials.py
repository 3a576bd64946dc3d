"""Packed weights with edge values for the product kernels (test input builders).

Two kinds of rows are written into otherwise random synthetic weights:

* special rows: scattered blocks get edge-case field values -- zero, fp16
  subnormal, smallest normal, largest (65504) and negative d / dmin; int8
  sub-scales -128 and 127; extreme codes (Q8_0 -128 and 127, Q6_K 0 and 63,
  Q4_K / Q5_K 0 and the top code); E4M3 subnormal, smallest normal, 448, -448,
  +0 and -0 block scales; E2M1 -0; FP8 codes 0, -0, subnormal, 448, -448.
  Every dequantized weight stays finite (the products are compared against the
  oracle's band, which needs finite sums).
* zero-point rows: every code of the row sits at the format's zero point while
  the scales stay non-zero (Q4_K / Q5_K: q = 0 with all mins m = 0; Q6_K:
  q = 32; Q8_0: q = 0; NVFP4: codes +0 / -0; FP8: codes +0 / -0).  Every
  weight of such a row is exactly zero, so sum_k |w x| = 0 and the band
  |y - y_ref| <= 2e-3 * sum_k |w x| asks for y = 0 exactly.

Blocks are placed by field offsets only (the block layouts of the header and
of synth); nothing here decodes a block.
"""
from __future__ import annotations

import numpy as np

import synth

Q8_0, Q4_K, Q6_K, NVFP4, Q5_K, FP8 = 1, 2, 3, 4, 5, 6
BB = {Q8_0: 34, Q4_K: 144, Q5_K: 176, Q6_K: 210}

# fp16 bit patterns for d / dmin: zero, smallest subnormal, largest subnormal,
# smallest normal, largest finite, a negative value, one
F16_SPECIALS = [0x0000, 0x0001, 0x03FF, 0x0400, 0x7BFF, 0xAE66, 0x3C00]
# E4M3 block scales (NVFP4): zero, smallest / largest subnormal, smallest
# normal, 448, -0, -448, one
E4M3_SCALES = [0x00, 0x01, 0x07, 0x08, 0x7E, 0x80, 0xFE, 0x38]
# FP8 codes: +0, -0, smallest subnormal (+-), largest subnormal, smallest
# normal, 448, -448, +-1
FP8_CODES = [0x00, 0x80, 0x01, 0x81, 0x07, 0x08, 0x7E, 0xFE, 0x38, 0xB8]


def _put16(buf, off, bits):
    buf[off] = bits & 0xFF
    buf[off + 1] = (bits >> 8) & 0xFF


def _row_blocks(fmt, N, K):
    return K // {Q8_0: 32, Q4_K: 256, Q5_K: 256, Q6_K: 256}[fmt]


def special_positions(N: int, nblk: int, count: int, seed: int):
    """(row, block) pairs spread over rows and over block positions along K."""
    g = np.random.default_rng(seed)
    rows = g.integers(0, N, count)
    rows[: min(count, 2)] = [0, N - 1][: min(count, 2)]
    blks = (np.arange(count) * 7 + g.integers(0, nblk, count)) % nblk
    return list(zip(rows.tolist(), blks.tolist()))


def with_specials(fmt: int, w: np.ndarray, E: int, N: int, K: int, seed: int = 0, count: int = 64) -> np.ndarray:
    """A copy of the packed weight[E*N, K] with edge-case field values in
    `count` blocks (or block scales / codes) spread over rows and K."""
    w = np.array(w, dtype=np.uint8, copy=True)
    R = E * N
    if fmt == NVFP4:
        codes, scales = w[: R * K // 2], w[R * K // 2: R * K // 2 + R * K // 16]
        nb = K // 16
        for i, (r, b) in enumerate(special_positions(R, nb, count, seed)):
            scales[r * nb + b] = E4M3_SCALES[i % len(E4M3_SCALES)]
            # codes of the block: -0, +0, +-6 in the first bytes
            c0 = r * K // 2 + b * 8
            codes[c0: c0 + 4] = [0x08, 0x80, 0x7F, 0xF7][:4]
        return w
    if fmt == FP8:
        codes = w[: R * K]
        for i, (r, b) in enumerate(special_positions(R, K // 64, count, seed)):
            c0 = r * K + b * 64
            for j in range(len(FP8_CODES)):
                codes[c0 + (7 * j + i) % 64] = FP8_CODES[(i + j) % len(FP8_CODES)]
        # one row scale of 1e30 (448 * 1e30 stays finite), one negative
        rs = w[R * K: R * K + 4 * R].view(np.float32)
        rs[0] = np.float32(1e30)
        rs[R - 1] = np.float32(-2.5e-3)
        return w
    bb, nb = BB[fmt], _row_blocks(fmt, N, K)
    for i, (r, b) in enumerate(special_positions(R, nb, count, seed)):
        o = (r * nb + b) * bb
        d = F16_SPECIALS[i % len(F16_SPECIALS)]
        if fmt == Q8_0:
            _put16(w, o, d)
            w[o + 2 + (i % 32)] = 0x80  # -128
            w[o + 2 + ((i + 5) % 32)] = 0x7F
        elif fmt in (Q4_K, Q5_K):
            _put16(w, o, d)
            _put16(w, o + 2, F16_SPECIALS[(i + 3) % len(F16_SPECIALS)])  # dmin
            if i % 3 == 0:
                w[o + 4: o + 16] = 0xFF  # every 6-bit scale and min = 63
            codes = o + (16 if fmt == Q4_K else 48)
            w[codes + (i % 128)] = 0x00
            w[codes + ((i + 9) % 128)] = 0xFF
            if fmt == Q5_K:
                w[o + 16 + (i % 32)] = 0xFF if i % 2 else 0x00
        elif fmt == Q6_K:
            _put16(w, o + 208, d)
            w[o + 192 + (i % 16)] = 0x80  # sub-scale -128
            w[o + 192 + ((i + 1) % 16)] = 0x7F
            w[o + (i % 128)] = 0x00 if i % 2 else 0xFF
            w[o + 128 + (i % 64)] = 0x00 if i % 2 else 0xFF
    return w


def zero_point_rows(fmt: int, w: np.ndarray, E: int, N: int, K: int, rows) -> np.ndarray:
    """A copy of the packed weight[E*N, K] whose rows `rows` (indices into E*N)
    hold only zero-point codes, their scales left as drawn (non-zero)."""
    w = np.array(w, dtype=np.uint8, copy=True)
    R = E * N
    if fmt == NVFP4:
        for r in rows:
            # alternate +0 (0x0) and -0 (0x8) nibbles
            w[r * K // 2:(r + 1) * K // 2] = 0x80
        return w
    if fmt == FP8:
        for r in rows:
            c = np.zeros(K, np.uint8)
            c[1::2] = 0x80
            w[r * K:(r + 1) * K] = c
        return w
    bb, nb = BB[fmt], _row_blocks(fmt, N, K)
    for r in rows:
        for b in range(nb):
            o = (r * nb + b) * bb
            if fmt == Q8_0:
                w[o + 2: o + 34] = 0
                if w[o] == 0 and w[o + 1] == 0:
                    _put16(w, o, 0x2E66)
            elif fmt in (Q4_K, Q5_K):
                # d, dmin non-zero; scales sc = 1 + j, mins m = 0; codes 0 (and no fifth bits)
                if w[o] == 0 and w[o + 1] == 0:
                    _put16(w, o, 0x2E66)
                _put16(w, o + 2, 0x2A00)
                S = np.zeros(12, np.uint8)
                for j in range(8):
                    sc = 1 + 7 * j  # 6-bit values, all non-zero
                    if j < 4:
                        S[j] = sc
                    else:
                        S[j + 4] |= sc & 15
                        S[j - 4] |= (sc >> 4) << 6
                w[o + 4: o + 16] = S
                w[o + 16: o + bb] = 0
            elif fmt == Q6_K:
                w[o: o + 128] = 0          # low nibbles 0
                w[o + 128: o + 192] = 0xAA  # high pairs 2: q = 32
                s = w[o + 192: o + 208].view(np.int8)
                s[s == 0] = 5
                if w[o + 208] == 0 and w[o + 209] == 0:
                    _put16(w, o + 208, 0x2E66)
    return w


def zero_rows_of(N: int):
    """Zero-point rows used by the tests: first, last, an odd interior row, and
    a run of four (one whole row group of the streaming kernels)."""
    rows = {0, N - 1, N // 3 | 1}
    if N >= 12:
        r0 = (N // 2) & ~3
        rows.update(range(r0, r0 + 4))
    return sorted(r for r in rows if 0 <= r < N)


def special_case(fmt: int, N: int, K: int, M: int, seed: int, E: int = 1, zero_rows=True):
    """(w, x, zrows): synthetic weights with specials and zero-point rows, x bf16 [M, K]."""
    w = synth.weights(fmt, synth.rng(seed, 0), E * N, K, E=E)
    w = with_specials(fmt, w, E, N, K, seed=seed)
    zrows = zero_rows_of(E * N) if zero_rows else []
    if zrows:
        w = zero_point_rows(fmt, w, E, N, K, zrows)
    x = synth.x_bf16(synth.rng(seed, 1), M, K)
    return w, x, zrows
