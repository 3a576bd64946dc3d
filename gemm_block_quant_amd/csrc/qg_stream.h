// qg_stream.h -- the weight-streaming core shared by the dense GEMV / skinny
// product (qg_gemv.hip) and the grouped-expert product (qg_grouped.hip), for
// packed Q8_0 weights and NVFP4 weights whose K is not a multiple of 64, on
// gfx950 (the other formats stream straight into registers, qg_direct.h).
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
//  * E2M1 codes become exact bf16 pairs by the gfx950 FP4 convert and
//    v_dot2_f32_bf16 accumulates them against the activations staged once
//    per workgroup in LDS; Q8_0's int8 codes become exact fp32 and meet the
//    activations in fp32 fused multiply-adds;
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

struct DecodeCtx {
    const lds_u8* seg;    // segment bytes in LDS (main plane), at the first block of the segment
    const lds_u8* segs;   // NVFP4: scale bytes in LDS at the first block of the segment
    const lds_u8* xl;     // activations [MT][K] bf16 in LDS
    int K;
    int kseg;             // K index of the segment's first value
};

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
template <> struct BlockGeom<QG_NVFP4> { static constexpr int QK = 16, BB = 8; };  // code bytes per block

constexpr int kWavesPerBlock = 4;
constexpr int kLdsBytes = 160 * 1024;

__host__ __device__ constexpr int rowbuf_bytes(int cpl, int cpls) {
    return cpl * 1024 + 32 + (cpls > 0 ? cpls * 1024 + 32 : 0);
}

// LDS layout: [x bf16: MT*K][pad to 16][per-wave row buffers]
__host__ __device__ constexpr size_t rowbuf_offset(int mt, int K) { return ((size_t)mt * K * 2 + 15) & ~(size_t)15; }
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
// zero).  row_of(m) gives the source row of pass row m.
template <int MT, class RowOf>
__device__ __forceinline__ void stage_x(lds_u8* xl, const uint16_t* x, int64_t ldx, int cnt, int K, RowOf row_of) {
    const int nvec = MT * K / 8;  // 16-byte vectors
    for (int i = threadIdx.x; i < nvec; i += blockDim.x) {
        const int m = (i * 8) / K, k = (i * 8) % K;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (m < cnt) v = ld_global128(x + (size_t)row_of(m) * ldx + k);
        *(lds_u32x4*)(xl + (size_t)i * 16) = v;
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
                                            lds_u8* rowbuf, lds_u8* rowbuf_s, int n0, int step,
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
        dc.K = K;
        dc.kseg = b0 * QK;
        const int nblk = b1 - b0;
        if (F == QG_NVFP4) {
            const int nunits = (nblk + 1) >> 1;
            for (int u = lane; u < nunits; u += 64) unit_nvfp4<MT>(dc, u, 2 * u + 1 < nblk, acc);
        } else {
            const int nunits = nblk * Unit<F>::PER_BLOCK;
            for (int u = lane; u < nunits; u += 64) unit_q8_0<MT>(dc, u, acc);
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
    const int qk = fmt == QG_Q8_0 ? 32 : 16;
    const int bb = fmt == QG_Q8_0 ? 34 : 8;
    const long row_bytes = (long)(K / qk) * bb;
    const int need = (int)((row_bytes + 30 + 1023) / 1024);
    return need <= 1 ? 1 : need <= 2 ? 2 : need <= 3 ? 3 : need <= 4 ? 4 : need <= 6 ? 6 : 4;
}

// Blocks per segment for a given chunk budget: a segment's 16-byte granules
// (its bytes plus up to 15 of misalignment at each end) must fit in 64*cpl.
inline int segment_blocks(int fmt, int K, int cpl) {
    const int qk = fmt == QG_Q8_0 ? 32 : 16;
    const int bb = fmt == QG_Q8_0 ? 34 : 8;
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
