// qg_stream.h -- the weight-streaming core shared by the dense GEMV / skinny
// product (qg_gemv.hip) and the grouped-expert product (qg_grouped.hip), for
// packed Q8_0 / Q4_K / Q6_K / NVFP4 weights on gfx950.
//
// Each packed weight block is read from HBM exactly once per call and
// dequantized on chip; the result is dotted with bf16 activations and
// accumulated in fp32 ("A 320B MoE on a free Kaggle TPU", section "The kernel,
// and why 64 tok/s is not a bandwidth number": a fused dequant-matvec whose
// dequantized weight never exists in memory).  Decode is weight-delivery
// bound ("Qwen3.8-27B on one Tenstorrent P150", section "4. Measuring the
// ceiling"), so the kernel is organised around the weight stream:
//
//  * persistent workgroups of 4 waves; every wave owns the rows n = gw + i*GW
//    and streams each row (or each K-segment of a long row) with 16-byte
//    non-temporal loads into a ring of PF register slots, so that several rows
//    are in flight per wave while an earlier one is decoded;
//  * a landed row is written to a wave-private LDS buffer, from which lanes
//    read fixed "units" (32 or 64 values plus their block header) at whatever
//    byte alignment the format has (34- and 210-byte blocks are not 16-byte
//    aligned);
//  * codes become bf16 pairs in registers (E2M1 by the gfx950 FP4 convert,
//    integer codes biased by 128 so that a byte permute builds exact bf16),
//    and v_dot2_f32_bf16 accumulates them against the activations staged once
//    per workgroup in LDS; the bias is removed with per-16-value activation
//    sums, also staged once;
//  * each weight is decoded once and used for all M activation rows (weight
//    reuse across rows: "Qwen3.8-27B on one Tenstorrent P150", section "3.
//    Porting the 9B stack to 27B geometry", packed prefill re-reading the
//    weight per 32 rows was the bug);
//  * a row's lane partials are combined by a fixed xor-butterfly, so every
//    output has one summation order that depends only on (format, K): row m of
//    an M-row call is bitwise the M = 1 result (section "8. Quality, then a
//    better quant" of the same page: verify rows must round like decode).
#pragma once

#include "qg_internal.h"

namespace qg {

// ------------------------------------------------------------------ per-format units

// Values per unit and units per block.
template <int F> struct Unit;
template <> struct Unit<QG_Q8_0> { static constexpr int V = 32, PER_BLOCK = 1; };
template <> struct Unit<QG_Q4_K> { static constexpr int V = 32, PER_BLOCK = 8; };
template <> struct Unit<QG_Q6_K> { static constexpr int V = 64, PER_BLOCK = 4; };
template <> struct Unit<QG_NVFP4> { static constexpr int V = 32, PER_BLOCK = 1; };  // a unit spans 2 blocks

// bf16 activation pairs for 16 values starting at k (k a multiple of 8).
struct XPairs {
    uint32_t v[8];
};
__device__ __forceinline__ XPairs load_x16(const lds_u8* xrow, int k) {
    const lds_u8* p = xrow + 2 * k;
    u32x4 a = lds_ld128(p), b = lds_ld128(p + 16);
    XPairs r;
    r.v[0] = a.x; r.v[1] = a.y; r.v[2] = a.z; r.v[3] = a.w;
    r.v[4] = b.x; r.v[5] = b.y; r.v[6] = b.z; r.v[7] = b.w;
    return r;
}

// Sum over 16 values of (128 + q) * x with the codes of 4 dwords (4 bytes each).
__device__ __forceinline__ float dot16_biased(const uint32_t q[4], const XPairs& x) {
    float d = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        d = dot2bf(bias128_pair(q[i], kSelB0B1), x.v[2 * i], d);
        d = dot2bf(bias128_pair(q[i], kSelB2B3), x.v[2 * i + 1], d);
    }
    return d;
}

struct DecodeCtx {
    const lds_u8* seg;    // segment bytes in LDS (main plane), at the first block of the segment
    const lds_u8* segs;   // NVFP4: scale bytes in LDS at the first block of the segment
    const lds_u8* xl;     // activations [MT][K] bf16 in LDS
    const lds_f32* xs;    // per-16-value activation sums [MT][K/16]
    int K;
    int kseg;             // K index of the segment's first value
};

// Q4_K unit u of a segment: block u/8, 16 code bytes j = u%8 = values
// 64g + 16h + [0,16) (low nibbles, sub-block 2g) and 64g + 32 + 16h + [0,16)
// (high nibbles, sub-block 2g+1), g = j/2, h = j%2.
// w = d*sc*q - dmin*m  ->  sum w x = d*sc*(D - 128 X) - dmin*m*X with D = sum (128+q) x.
template <int MT>
__device__ __forceinline__ void unit_q4_k(const DecodeCtx& c, int u, float (&acc)[MT]) {
    const int b = u >> 3, j = u & 7, g = j >> 1, hh = j & 1;
    const lds_u8* blk = c.seg + b * 144;
    const u32x4 h = lds_ld128(blk);
    const u32x4 q = lds_ld128(blk + 16 + 16 * j);
    const float d = f16_to_f32(h.x), dmin = f16_to_f32(h.x >> 16);
    const uint32_t sh = (uint32_t)(g & 1) * 16u;
    const uint32_t ys = h.y >> sh, zs = h.z >> sh, ws = h.w >> sh;
    uint32_t sc0, sc1, m0, m1;
    if (g < 2) {
        sc0 = ys & 63u; sc1 = (ys >> 8) & 63u;
        m0 = zs & 63u;  m1 = (zs >> 8) & 63u;
    } else {
        sc0 = (ws & 15u) | ((ys >> 2) & 0x30u);
        sc1 = ((ws >> 8) & 15u) | ((ys >> 10) & 0x30u);
        m0 = ((ws >> 4) & 15u) | ((zs >> 2) & 0x30u);
        m1 = ((ws >> 12) & 15u) | ((zs >> 10) & 0x30u);
    }
    const float a0 = d * (float)sc0, a1 = d * (float)sc1;
    const float b0 = -fmaf(dmin, (float)m0, 128.f * a0);
    const float b1 = -fmaf(dmin, (float)m1, 128.f * a1);
    const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
    uint32_t lo[4], hi[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        lo[i] = qw[i] & 0x0F0F0F0Fu;
        hi[i] = (qw[i] >> 4) & 0x0F0F0F0Fu;
    }
    const int klo = c.kseg + b * 256 + 64 * g + 16 * hh, khi = klo + 32;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const lds_u8* xr = c.xl + (size_t)m * c.K * 2;
        const float dlo = dot16_biased(lo, load_x16(xr, klo));
        const float dhi = dot16_biased(hi, load_x16(xr, khi));
        const lds_f32* xsr = c.xs + (size_t)m * (c.K >> 4);
        float a = acc[m];
        a = fmaf(a0, dlo, a);
        a = fmaf(b0, xsr[klo >> 4], a);
        a = fmaf(a1, dhi, a);
        a = fmaf(b1, xsr[khi >> 4], a);
        acc[m] = a;
    }
}

// Q6_K unit u of a segment: block u/4, half h = (u/2)%2, t = u%2: values
// 128h + 32p + 16t + [0,16) for p = 0..3, each group with sub-scale s[8h + 2p + t].
// w = d*s*(q - 32)  ->  sum w x = d*s*(D - 160 X) with D = sum (128+q) x.
template <int MT>
__device__ __forceinline__ void unit_q6_k(const DecodeCtx& c, int u, float (&acc)[MT]) {
    const int b = u >> 2, h = (u >> 1) & 1, t = u & 1;
    const lds_u8* blk = c.seg + b * 210;
    const u32x4 qa = lds_ld128_a2(blk + 64 * h + 16 * t);
    const u32x4 qb = lds_ld128_a2(blk + 64 * h + 32 + 16 * t);
    const u32x4 qh = lds_ld128_a2(blk + 128 + 32 * h + 16 * t);
    const uint32_t s03 = lds_ld32_a2(blk + 192 + 8 * h), s47 = lds_ld32_a2(blk + 196 + 8 * h);
    const float d = f16_to_f32(lds_ld32_a2(blk + 208));
    // sub-scales s[8h + t + 2p] = byte (t + 2p) of the 8 bytes at 192 + 8h
    const uint32_t st = t ? (s03 >> 8) : s03, su = t ? (s47 >> 8) : s47;
    float a[4];
    a[0] = d * (float)(int8_t)(st & 0xffu);
    a[1] = d * (float)(int8_t)((st >> 16) & 0xffu);
    a[2] = d * (float)(int8_t)(su & 0xffu);
    a[3] = d * (float)(int8_t)((su >> 16) & 0xffu);
    const uint32_t A[4] = {qa.x, qa.y, qa.z, qa.w}, B[4] = {qb.x, qb.y, qb.z, qb.w},
                   H[4] = {qh.x, qh.y, qh.z, qh.w};
    uint32_t v[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[0][i] = (A[i] & 0x0F0F0F0Fu) | ((H[i] << 4) & 0x30303030u);
        v[1][i] = (B[i] & 0x0F0F0F0Fu) | ((H[i] << 2) & 0x30303030u);
        v[2][i] = ((A[i] >> 4) & 0x0F0F0F0Fu) | (H[i] & 0x30303030u);
        v[3][i] = ((B[i] >> 4) & 0x0F0F0F0Fu) | ((H[i] >> 2) & 0x30303030u);
    }
    const int k0 = c.kseg + b * 256 + 128 * h + 16 * t;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const lds_u8* xr = c.xl + (size_t)m * c.K * 2;
        const lds_f32* xsr = c.xs + (size_t)m * (c.K >> 4);
        float acc_m = acc[m];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int k = k0 + 32 * p;
            const float dp = dot16_biased(v[p], load_x16(xr, k));
            acc_m = fmaf(a[p], dp, acc_m);
            acc_m = fmaf(-160.f * a[p], xsr[k >> 4], acc_m);
        }
        acc[m] = acc_m;
    }
}

// Q8_0 unit u: block u (32 int8 codes, fp16 d).  sum w x = d * sum q x.
template <int MT>
__device__ __forceinline__ void unit_q8_0(const DecodeCtx& c, int u, float (&acc)[MT]) {
    const lds_u8* blk = c.seg + u * 34;
    const float d = f16_to_f32(lds_ld32_a2(blk));
    const u32x4 q0 = lds_ld128_a2(blk + 2), q1 = lds_ld128_a2(blk + 18);
    const uint32_t qw[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
    float qf[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int bsel = 0; bsel < 4; ++bsel) qf[4 * i + bsel] = (float)(int8_t)((qw[i] >> (8 * bsel)) & 0xffu);
    }
    const int k0 = c.kseg + 32 * u;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const lds_u8* xr = c.xl + (size_t)m * c.K * 2;
        const XPairs x0 = load_x16(xr, k0), x1 = load_x16(xr, k0 + 16);
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            s = fmaf(qf[2 * i], bf16_to_f32(x0.v[i]), s);
            s = fmaf(qf[2 * i + 1], bf16_to_f32(x0.v[i] >> 16), s);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            s = fmaf(qf[16 + 2 * i], bf16_to_f32(x1.v[i]), s);
            s = fmaf(qf[16 + 2 * i + 1], bf16_to_f32(x1.v[i] >> 16), s);
        }
        acc[m] = fmaf(d, s, acc[m]);
    }
}

// NVFP4 unit u: values 32u + [0,32) of the segment = blocks 2u and 2u+1 (the
// second one absent at an odd row end).  sum w x = g * sum_b s_b * sum c x;
// the tensor scale g is applied once per output.
template <int MT>
__device__ __forceinline__ void unit_nvfp4(const DecodeCtx& c, int u, bool two, float (&acc)[MT]) {
    const u32x2 c0 = lds_ld64(c.seg + 16 * u);
    const u32x2 c1 = lds_ld64(c.seg + 16 * u + 8);
    const uint32_t sb0 = c.segs[2 * u];
    const uint32_t sb1 = two ? (uint32_t)c.segs[2 * u + 1] : 0u;
    const float s0 = e4m3_to_f32<0>(sb0), s1 = e4m3_to_f32<0>(sb1);
    uint32_t p0[8], p1[8];
    p0[0] = e2m1x2_to_bf16x2<0>(c0.x); p0[1] = e2m1x2_to_bf16x2<1>(c0.x);
    p0[2] = e2m1x2_to_bf16x2<2>(c0.x); p0[3] = e2m1x2_to_bf16x2<3>(c0.x);
    p0[4] = e2m1x2_to_bf16x2<0>(c0.y); p0[5] = e2m1x2_to_bf16x2<1>(c0.y);
    p0[6] = e2m1x2_to_bf16x2<2>(c0.y); p0[7] = e2m1x2_to_bf16x2<3>(c0.y);
    p1[0] = e2m1x2_to_bf16x2<0>(c1.x); p1[1] = e2m1x2_to_bf16x2<1>(c1.x);
    p1[2] = e2m1x2_to_bf16x2<2>(c1.x); p1[3] = e2m1x2_to_bf16x2<3>(c1.x);
    p1[4] = e2m1x2_to_bf16x2<0>(c1.y); p1[5] = e2m1x2_to_bf16x2<1>(c1.y);
    p1[6] = e2m1x2_to_bf16x2<2>(c1.y); p1[7] = e2m1x2_to_bf16x2<3>(c1.y);
    const int k0 = c.kseg + 32 * u;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const lds_u8* xr = c.xl + (size_t)m * c.K * 2;
        const XPairs x0 = load_x16(xr, k0);
        float d0 = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) d0 = dot2bf(p0[i], x0.v[i], d0);
        float a = fmaf(s0, d0, acc[m]);
        if (two) {
            const XPairs x1 = load_x16(xr, k0 + 16);
            float d1 = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) d1 = dot2bf(p1[i], x1.v[i], d1);
            a = fmaf(s1, d1, a);
        }
        acc[m] = a;
    }
}

// ------------------------------------------------------------------ the kernel

template <int F> struct BlockGeom;
template <> struct BlockGeom<QG_Q8_0> { static constexpr int QK = 32, BB = 34; };
template <> struct BlockGeom<QG_Q4_K> { static constexpr int QK = 256, BB = 144; };
template <> struct BlockGeom<QG_Q6_K> { static constexpr int QK = 256, BB = 210; };
template <> struct BlockGeom<QG_NVFP4> { static constexpr int QK = 16, BB = 8; };  // code bytes per block

constexpr int kWavesPerBlock = 4;
constexpr int kLdsBytes = 160 * 1024;

__host__ __device__ constexpr int rowbuf_bytes(int cpl, int cpls) {
    return cpl * 1024 + 32 + (cpls > 0 ? cpls * 1024 + 32 : 0);
}

// LDS layout: [x bf16: MT*K][x sums fp32: MT*K/16][pad to 16][per-wave row buffers]
__host__ __device__ constexpr size_t rowbuf_offset(int mt, int K) {
    return ((size_t)mt * K * 2 + (size_t)mt * (K / 16) * 4 + 15) & ~(size_t)15;
}
__host__ __device__ constexpr size_t gemv_lds_bytes(int mt, int K, int cpl, int cpls) {
    return rowbuf_offset(mt, K) + (size_t)kWavesPerBlock * rowbuf_bytes(cpl, cpls);
}


// One weight matrix as the streaming core sees it.
struct MatView {
    const uint8_t* w0;      // row 0: blocks (Q8_0/Q4_K/Q6_K) or E2M1 codes (NVFP4)
    int64_t rb0;            // bytes per row in that plane
    const uint8_t* w1;      // NVFP4: row 0 of the E4M3 scale plane
    int64_t rb1;            // NVFP4: scale bytes per row
    const uint8_t* gbytes;  // NVFP4: the fp32 tensor scale (any alignment)
};

// Stage activation rows 0..MT-1 into LDS as bf16 [MT][K] (rows >= cnt are
// zero) and, for the integer formats, their per-16-value fp32 sums
// (sequential order).  row_of(m) gives the source row of pass row m.
template <int MT, bool SUMS, class RowOf>
__device__ __forceinline__ void stage_x(lds_u8* xl, lds_f32* xs, const uint16_t* x, int64_t ldx, int cnt, int K,
                                        RowOf row_of) {
    const int nvec = MT * K / 8;  // 16-byte vectors
    for (int i = threadIdx.x; i < nvec; i += blockDim.x) {
        const int m = (i * 8) / K, k = (i * 8) % K;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (m < cnt) v = ld_global128(x + (size_t)row_of(m) * ldx + k);
        *(lds_u32x4*)(xl + (size_t)i * 16) = v;
    }
    if (SUMS) {
        __syncthreads();
        const int ng = MT * (K / 16);
        for (int i = threadIdx.x; i < ng; i += blockDim.x) {
            const XPairs xp = load_x16(xl, 16 * i);  // group i of the row-major [MT][K] array
            float s = 0.f;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                s += bf16_to_f32(xp.v[t]);
                s += bf16_to_f32(xp.v[t] >> 16);
            }
            xs[i] = s;
        }
    }
    __syncthreads();
}

// One wave streams rows n0, n0 + step, ... (< n_end) of matrix mv through a
// wave-private LDS row buffer; each row is nseg segments of segb blocks.  Lane
// m < cnt writes y[yrow * ldy + n] for activation row m.  stage() stages the
// activations (a workgroup barrier inside): every wave calls it exactly once,
// after its first PF slots of weight loads are in flight.
template <int F, int MT, int CPL, int CPLS, int PF, class Stage>
__device__ __forceinline__ void wave_stream(const MatView& mv, int K, int segb, int nseg, const lds_u8* xl,
                                            const lds_f32* xs, lds_u8* rowbuf, lds_u8* rowbuf_s, int n0, int step,
                                            int n_end, float* y, int64_t ldy, int64_t yrow, int cnt, Stage stage) {
    constexpr int QK = BlockGeom<F>::QK, BB = BlockGeom<F>::BB;
    constexpr int CS = CPLS > 0 ? CPLS : 1;
    const int lane = threadIdx.x & 63;
    const int nb = K / QK;
    const int nrows = n0 < n_end ? (n_end - 1 - n0) / step + 1 : 0;
    const int nitems = nrows * nseg;
    if (nitems == 0) {
        stage();
        return;
    }

    float gscale = 1.f;
    if (F == QG_NVFP4) {
        const uint8_t* gb = mv.gbytes;
        const uint32_t bits = (uint32_t)gb[0] | ((uint32_t)gb[1] << 8) | ((uint32_t)gb[2] << 16) |
                              ((uint32_t)gb[3] << 24);
        gscale = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(bits));
    }

    u32x4 R[PF][CPL];
    u32x4 RS[PF][CS];

    // Loads of one item (row, segment) into a ring slot.  Every lane loads CPL
    // (+CPLS) aligned 16-byte granules; each holds at least one byte of the
    // tensor, so no load leaves the tensor's pages.  Items past the end reload
    // the first granule of row n0 so that every path issues the same loads.
    int in_ = n0, is_ = 0, it_ = 0;
    auto issue = [&](u32x4 (&r)[CPL], u32x4 (&rs)[CS]) {
        const bool live = it_ < nitems;
        const int n = live ? in_ : n0;
        const int b0 = live ? is_ * segb : 0;
        const int b1 = live ? min(nb, b0 + segb) : 1;
        const uint8_t* beg = mv.w0 + (size_t)n * mv.rb0 + (size_t)b0 * BB;
        const uint8_t* end = mv.w0 + (size_t)n * mv.rb0 + (size_t)b1 * BB;
        const uint8_t* b16 = (const uint8_t*)((uintptr_t)beg & ~(uintptr_t)15);
        const int nch = (int)((end - b16 + 15) >> 4);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int idx = lane + 64 * c;
            r[c] = ld_stream128(b16 + 16 * (idx < nch ? idx : 0));
        }
        if (CPLS > 0) {
            const uint8_t* sbeg = mv.w1 + (size_t)n * mv.rb1 + b0;
            const uint8_t* send = mv.w1 + (size_t)n * mv.rb1 + b1;
            const uint8_t* s16 = (const uint8_t*)((uintptr_t)sbeg & ~(uintptr_t)15);
            const int nchs = (int)((send - s16 + 15) >> 4);
#pragma unroll
            for (int c = 0; c < CPLS; ++c) {
                const int idx = lane + 64 * c;
                rs[c] = ld_stream128(s16 + 16 * (idx < nchs ? idx : 0));
            }
        }
        ++it_;
        if (++is_ == nseg) {
            is_ = 0;
            in_ += step;
        }
    };

    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.f;

    int pn_ = n0, ps_ = 0;
    auto process = [&](const u32x4 (&r)[CPL], const u32x4 (&rs)[CS]) {
        const int b0 = ps_ * segb, b1 = min(nb, b0 + segb);
#pragma unroll
        for (int c = 0; c < CPL; ++c) *(lds_u32x4*)(rowbuf + 16 * (lane + 64 * c)) = r[c];
        if (CPLS > 0) {
#pragma unroll
            for (int c = 0; c < CPLS; ++c) *(lds_u32x4*)(rowbuf_s + 16 * (lane + 64 * c)) = rs[c];
        }
        DecodeCtx dc;
        const uintptr_t beg = (uintptr_t)(mv.w0 + (size_t)pn_ * mv.rb0 + (size_t)b0 * BB);
        dc.seg = rowbuf + (beg & 15);
        if (CPLS > 0) {
            const uintptr_t sbeg = (uintptr_t)(mv.w1 + (size_t)pn_ * mv.rb1 + b0);
            dc.segs = rowbuf_s + (sbeg & 15);
        } else {
            dc.segs = rowbuf_s;
        }
        dc.xl = xl;
        dc.xs = xs;
        dc.K = K;
        dc.kseg = b0 * QK;
        const int nblk = b1 - b0;
        if (F == QG_NVFP4) {
            const int nunits = (nblk + 1) >> 1;
            for (int u = lane; u < nunits; u += 64) unit_nvfp4<MT>(dc, u, 2 * u + 1 < nblk, acc);
        } else {
            const int nunits = nblk * Unit<F>::PER_BLOCK;
            for (int u = lane; u < nunits; u += 64) {
                if (F == QG_Q4_K) unit_q4_k<MT>(dc, u, acc);
                else if (F == QG_Q6_K) unit_q6_k<MT>(dc, u, acc);
                else unit_q8_0<MT>(dc, u, acc);
            }
        }
        if (++ps_ == nseg) {
            float mine = 0.f;
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const float tot = wave_sum(acc[m]);
                if (lane == m) mine = tot;
                acc[m] = 0.f;
            }
            if (F == QG_NVFP4) mine *= gscale;
            if (lane < cnt) st_global_f32(y + yrow * ldy + pn_, mine);
            ps_ = 0;
            pn_ += step;
        }
    };

    // fill the ring, stage the activations, then: land a slot, refill it PF items ahead
#pragma unroll
    for (int sl = 0; sl < PF; ++sl) issue(R[sl], RS[sl]);
    stage();
    const int nfull = nitems - nitems % PF;
    for (int t0 = 0; t0 < nfull; t0 += PF) {
#pragma unroll
        for (int sl = 0; sl < PF; ++sl) {
            process(R[sl], RS[sl]);
            issue(R[sl], RS[sl]);
        }
    }
#pragma unroll
    for (int sl = 0; sl < PF; ++sl)
        if (nfull + sl < nitems) process(R[sl], RS[sl]);
}

// ------------------------------------------------------------------ host-side geometry

// Chunks of 16 bytes per lane for one segment of a row: the whole row when it
// fits in 6 KB of row buffer, else 4 KB segments.
inline int choose_cpl(int fmt, int K) {
    const int qk = fmt == QG_Q8_0 ? 32 : fmt == QG_NVFP4 ? 16 : 256;
    const int bb = fmt == QG_Q8_0 ? 34 : fmt == QG_Q4_K ? 144 : fmt == QG_Q6_K ? 210 : 8;
    const long row_bytes = (long)(K / qk) * bb;
    const int need = (int)((row_bytes + 30 + 1023) / 1024);
    return need <= 1 ? 1 : need <= 2 ? 2 : need <= 3 ? 3 : need <= 4 ? 4 : need <= 6 ? 6 : 4;
}

// Blocks per segment for a given chunk budget: a segment's 16-byte granules
// (its bytes plus up to 15 of misalignment at each end) must fit in 64*cpl.
inline int segment_blocks(int fmt, int K, int cpl) {
    const int qk = fmt == QG_Q8_0 ? 32 : fmt == QG_NVFP4 ? 16 : 256;
    const int bb = fmt == QG_Q8_0 ? 34 : fmt == QG_Q4_K ? 144 : fmt == QG_Q6_K ? 210 : 8;
    const int nb = K / qk;
    int sb = (64 * cpl * 16 - 30) / bb;
    if (fmt == QG_NVFP4) sb &= ~1;  // units span 2 blocks
    return sb < nb ? sb : nb;
}

// Workgroups of `block` threads with `lds` bytes of dynamic LDS that one CU holds
// at once for kernel `fn` on the current device (at least 1).  The first call
// per kernel and device also lifts the kernel's dynamic-LDS limit to 160 KB.
// Cached per (device, kernel, lds); safe to call from several threads.
hipError_t kernel_residency(const void* fn, size_t lds, int* per_cu, int block = 256);
// Opts kernel fn into the whole LDS on the current device (once per device).
hipError_t allow_full_lds(const void* fn);


}  // namespace qg
