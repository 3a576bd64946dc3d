// qg_direct.h -- register-direct weight streaming for Q4_K, Q6_K and NVFP4
// (K a multiple of 64), with the products formed on the matrix cores by the
// 16-block 4x4x4 bf16 MFMA.
//
// A wave works on 4 weight rows at once.  Lane l serves row j = l % 4 and
// unit slot b = l / 4 (16 slots): in pass p it loads unit u = 16 p + b of its
// row (64 values) straight into registers -- Q4_K one quarter of a
// super-block (32 code bytes) plus the block's 16-byte header; Q6_K the code
// bytes, high bits and sub-scales of one quarter of a 210-byte block (2-byte
// aligned loads, which gfx950 serves at full width); NVFP4 32 code bytes plus
// their four E4M3 scales.  The 16 lanes of a row cover a contiguous stretch of
// it, so the stream stays coalesced and the weights never pass through LDS.
//
// v_mfma_f32_4x4x4_16b_bf16 computes 16 independent products
// D[b] = A[b] (4 x 4) * B[b] (4 x 4): lane l supplies row l % 4 of A[b] and
// column l % 4 of B[b] (4 values along k each) and receives column l % 4 of
// D[b] (4 values).  Here block b is unit slot b, B[b] holds 4 decoded weights
// of each of the 4 rows (exact bf16: 128 + q for Q4_K and Q6_K, e2m1 for
// NVFP4), and
// A[b] holds the activations of up to 4 activation rows at the same 4
// positions.  So one instruction forms, for every lane, the partial dot
// products of its own weight row with 4 activation rows, and a lane's decoded
// codes serve every activation row without further VALU work.  Eight (Q4_K) or
// four (Q6_K, NVFP4) instructions accumulate one scale block; the lane then applies
// that block's scale to its 4 results in fp32.
//
// Every output element therefore has one fixed arithmetic: the matrix-core
// sum over each 4-value group, fixed accumulation order over a scale block,
// fixed fp32 scaling order, and a fixed xor-butterfly over the unit slots.
// Nothing depends on how many activation rows share the call, so row m of an
// M-row call is bitwise the M = 1 result ("Qwen3.8-27B on one Tenstorrent
// P150", section "8. Quality, then a better quant": verify rows must round
// exactly like single-token decode).
//
// Activations live in LDS interleaved for the A operand: for each unit, 16
// bytes (8 values) per (position group, activation row), the position groups
// of unit u rotated by u % 4 so that the four slots of a 16-lane row read
// different banks.
#pragma once

#include "qg_stream.h"

namespace qg {

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// D += A * B on the 16-block 4x4x4 bf16 MFMA.  a, b: 4 bf16 values each (two
// dwords, value order = k order).
__device__ __forceinline__ f32x4_t mfma4(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, f32x4_t c) {
    const i16x4_t a = __builtin_bit_cast(i16x4_t, u32x2{a0, a1});
    const i16x4_t b = __builtin_bit_cast(i16x4_t, u32x2{b0, b1});
    return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a, b, c, 0, 0, 0);
}

// The value of lane l ^ (4 << J) (the lane of the same row in unit slot
// s ^ (1 << J)).
template <int J>
__device__ __forceinline__ float slot_xor(float x) {
    if constexpr (J == 3) {
        return __shfl_xor(x, 32, kWave);
    } else {
        return __builtin_bit_cast(float,
                                  __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), ((4 << J) << 10) | 0x1F));
    }
}

// Butterfly stages J.. of the sums over the 16 unit slots of a lane's row of
// the N values c[]: while N > 1 a stage hands half of the values to the
// partner lane (the lane whose slot has bit J clear keeps the values whose
// index has bit 0 clear), so a stage costs N / 2 exchanges; a single value
// is exchanged whole.  Every value is added along the same xor tree as a
// plain butterfly (each addition has the same two operands), so the totals do
// not depend on N.  On return c[0] holds the total of original value
// slot % N0 (N0 the initial N).
template <int J, int N>
__device__ __forceinline__ float slot_stages(const float (&c)[N], int slot) {
    if constexpr (J == 4) {
        return c[0];
    } else if constexpr (N == 1) {
        const float v = c[0] + slot_xor<J>(c[0]);
        const float n[1] = {v};
        return slot_stages<J + 1, 1>(n, slot);
    } else {
        const bool hi = (slot >> J) & 1;
        float n[N / 2];
#pragma unroll
        for (int i = 0; i < N / 2; ++i) {
            const float keep = hi ? c[2 * i + 1] : c[2 * i];
            const float send = hi ? c[2 * i] : c[2 * i + 1];
            n[i] = keep + slot_xor<J>(send);
        }
        return slot_stages<J + 1, N / 2>(n, slot);
    }
}

// Sum over the 16 unit slots of a lane's row (lanes l, l ^ 4, l ^ 8, ...) of
// each of the MT values v[]: lane of slot s gets the total of v[s % MT].
template <int MT>
__device__ __forceinline__ float slot_sum_rows(const float (&v)[MT], int slot) {
    static_assert(MT == 1 || MT == 2 || MT == 4 || MT == 8 || MT == 16, "power of two up to 16");
    return slot_stages<0, MT>(v, slot);
}

constexpr int kDirectRows = 4;    // weight rows per wave at a time
constexpr int kDirectSlots = 16;  // unit slots per row per pass

template <int F> struct Direct;

// Q4_K.  Unit u of a row = quarter g = u % 4 of super-block u / 4: code bytes
// [32g, 32g + 32), whose low nibbles are the 32 values of sub-block 2g and
// high nibbles the 32 values of sub-block 2g + 1.
// sum w x = a0 D0 - dmin m0 X0 + a1 D1 - dmin m1 X1 with a = d * sc,
// D = sum q x (the nibbles as exact bf16) and X = sum x over the sub-block.
template <> struct Direct<QG_Q4_K> {
    static constexpr int UV = 64;  // activation values per unit
    static constexpr int REGS = 12;
    static constexpr bool SUMS = true;
    // 6-bit scale and min of sub-blocks 2g and 2g+1: for g < 2 they sit whole
    // in S[2g..2g+1] (scales) and S[2g+4..2g+5] (mins); for g >= 2 their low 4
    // bits come from S[2g+4..2g+5] and their top 2 bits from the top of
    // S[2g-4..2g-3] (scales) and S[2g..2g+1] (mins).  Read with bit-field
    // extracts whose offsets and widths are per-lane constants (width 0 reads
    // as zero), so no lane diverges.
    struct Lane {
        bool hi4;
        uint32_t off, oam, wa, wb;
    };
    __device__ static Lane lane_consts(int lane) {
        Lane L;
        const int g = (lane >> 2) & 3;  // slot b = lane / 4, and u % 4 = b % 4 in every pass
        L.hi4 = g >= 2;
        L.off = 16u * (uint32_t)(g & 1);
        L.oam = L.off + (L.hi4 ? 4u : 0u);
        L.wa = L.hi4 ? 4u : 6u;
        L.wb = L.hi4 ? 2u : 0u;
        return L;
    }
    __device__ __host__ static int units_per_row(int K) { return (K / 256) * 4; }
    // Bytes of one pass (16 units = 4 super-blocks) of a row.
    static constexpr int PASS0 = 4 * 144, PASS1 = 0;
    // Offsets from the start of a pass's stretch of the row: code bytes of
    // the unit (a) and its super-block header (b).
    struct Offs {
        uint32_t a, b;
    };
    __device__ static Offs slot_offs(int s) {
        return Offs{144u * (uint32_t)(s >> 2) + 16u + 32u * (uint32_t)(s & 3), 144u * (uint32_t)(s >> 2)};
    }
    __device__ static Offs shift(const Offs& o, uint32_t r0, uint32_t) { return Offs{o.a + r0, o.b + r0}; }
    __device__ static Offs pick(bool c, const Offs& x, const Offs& y) { return Offs{c ? x.a : y.a, c ? x.b : y.b}; }
    __device__ static void load_at(uint32_t (&r)[REGS], const uint8_t* b0, const uint8_t*, const Offs& o) {
        // Plain (cached) loads: the three loads of a lane touch the same lines as
        // those of its neighbours, and non-temporal loads fetched them again.
        const u32x4 qa = ld_global128(b0 + o.a), qb = ld_global128(b0 + o.a + 16), h = ld_global128(b0 + o.b);
        r[0] = qa.x; r[1] = qa.y; r[2] = qa.z; r[3] = qa.w;
        r[4] = qb.x; r[5] = qb.y; r[6] = qb.z; r[7] = qb.w;
        r[8] = h.x; r[9] = h.y; r[10] = h.z; r[11] = h.w;
    }
    // xa: this lane's A-operand base for unit u; xmg_bytes: bytes per group of
    // 4 activation rows; xs: per sub-block activation sums [group][sub-block][4];
    // live: the unit exists (the matrix-core work is wave-wide, only the
    // accumulation is skipped).
    template <int MT>
    __device__ static void decode(const uint32_t (&r)[REGS], const Lane& L, int u, bool live, const lds_u8* xa,
                                  int xmg_bytes, const lds_f32* xs, int xs_mg, float (&acc)[MT]) {
        constexpr int MG = (MT + 3) / 4;
        const uint32_t y = r[9], z = r[10], w = r[11];
        const uint32_t as = L.hi4 ? w : y, am = L.hi4 ? w : z;
        const uint32_t sc0 = __builtin_amdgcn_ubfe(as, L.off, L.wa) | (__builtin_amdgcn_ubfe(y, L.off + 6, L.wb) << 4);
        const uint32_t sc1 =
            __builtin_amdgcn_ubfe(as, L.off + 8, L.wa) | (__builtin_amdgcn_ubfe(y, L.off + 14, L.wb) << 4);
        const uint32_t m0 = __builtin_amdgcn_ubfe(am, L.oam, L.wa) | (__builtin_amdgcn_ubfe(z, L.off + 6, L.wb) << 4);
        const uint32_t m1 =
            __builtin_amdgcn_ubfe(am, L.oam + 8, L.wa) | (__builtin_amdgcn_ubfe(z, L.off + 14, L.wb) << 4);
        const float d = f16_to_f32(r[8]), dmin = f16_to_f32(r[8] >> 16);
        const float a0 = d * (float)sc0, a1 = d * (float)sc1;
        const float b0 = -(dmin * (float)m0), b1 = -(dmin * (float)m1);

        f32x4_t c0[MG], c1[MG];
#pragma unroll
        for (int g = 0; g < MG; ++g) c0[g] = c1[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const int rot = u & 3;
#pragma unroll
        for (int rp = 0; rp < 4; ++rp) {
            // values 8rp..8rp+7 of each sub-block: code dwords 2rp, 2rp+1 (low
            // nibbles: sub-block 2g; high nibbles: sub-block 2g+1)
            const uint32_t l0 = r[2 * rp] & 0x0F0F0F0Fu, l1 = r[2 * rp + 1] & 0x0F0F0F0Fu;
            const uint32_t h0 = (r[2 * rp] >> 4) & 0x0F0F0F0Fu, h1 = (r[2 * rp + 1] >> 4) & 0x0F0F0F0Fu;
            const uint32_t bl0 = int_pair_bf16<0>(l0), bl1 = int_pair_bf16<1>(l0);
            const uint32_t bl2 = int_pair_bf16<0>(l1), bl3 = int_pair_bf16<1>(l1);
            const uint32_t bh0 = int_pair_bf16<0>(h0), bh1 = int_pair_bf16<1>(h0);
            const uint32_t bh2 = int_pair_bf16<0>(h1), bh3 = int_pair_bf16<1>(h1);
#pragma unroll
            for (int g = 0; g < MG; ++g) {
                const u32x4 xl = lds_ld128(xa + g * xmg_bytes + ((rp ^ rot) * 4 * 16));
                const u32x4 xh = lds_ld128(xa + g * xmg_bytes + (((4 + rp) ^ rot) * 4 * 16));
                c0[g] = mfma4(xl.x, xl.y, bl0, bl1, c0[g]);
                c1[g] = mfma4(xh.x, xh.y, bh0, bh1, c1[g]);
                c0[g] = mfma4(xl.z, xl.w, bl2, bl3, c0[g]);
                c1[g] = mfma4(xh.z, xh.w, bh2, bh3, c1[g]);
            }
        }
        if (live) {
#pragma unroll
            for (int g = 0; g < MG; ++g) {
                const f32x4_t s0 = *(const QG_LDS f32x4_t*)(xs + (size_t)g * xs_mg + 8 * u);
                const f32x4_t s1 = *(const QG_LDS f32x4_t*)(xs + (size_t)g * xs_mg + 8 * u + 4);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (4 * g + i < MT) {
                        float a = acc[4 * g + i];
                        a = fmaf(a0, c0[g][i], a);
                        a = fmaf(b0, s0[i], a);
                        a = fmaf(a1, c1[g][i], a);
                        a = fmaf(b1, s1[i], a);
                        acc[4 * g + i] = a;
                    }
                }
            }
        }
    }
};

// Q5_K: Q4_K with a fifth code bit.  Unit u of a row = quarter g = u % 4 of
// super-block u / 4: code bytes [48 + 32g, 48 + 32g + 32) (low nibbles:
// sub-block 2g, high: 2g + 1), the 32 fifth-bit bytes H at [16, 48) (bit 2g of
// H[l] for the low nibble of position l, bit 2g + 1 for the high one) and the
// 16-byte header.  q = lo + 16 f goes to the matrix cores as two exact parts,
// the nibble lo and 16 f, chained into one sum per sub-block; the sums X are
// those of Q4_K.
template <> struct Direct<QG_Q5_K> {
    static constexpr int UV = 64;
    static constexpr int REGS = 20;
    static constexpr bool SUMS = true;
    struct Lane {
        Direct<QG_Q4_K>::Lane s;  // scale and min extraction (as Q4_K)
        uint32_t hsh;             // 2g: the fifth bits of sub-block 2g
    };
    __device__ static Lane lane_consts(int lane) {
        return Lane{Direct<QG_Q4_K>::lane_consts(lane), 2u * (uint32_t)((lane >> 2) & 3)};
    }
    __device__ __host__ static int units_per_row(int K) { return (K / 256) * 4; }
    // Bytes of one pass (16 units = 4 super-blocks) of a row.
    static constexpr int PASS0 = 4 * 176, PASS1 = 0;
    // Offsets from the start of a pass's stretch: the unit's code bytes (a),
    // its super-block's fifth-bit bytes (b) and header (c).
    struct Offs {
        uint32_t a, b, c;
    };
    __device__ static Offs slot_offs(int s) {
        const uint32_t blk = 176u * (uint32_t)(s >> 2);
        return Offs{blk + 48u + 32u * (uint32_t)(s & 3), blk + 16u, blk};
    }
    __device__ static Offs shift(const Offs& o, uint32_t r0, uint32_t) { return Offs{o.a + r0, o.b + r0, o.c + r0}; }
    __device__ static Offs pick(bool c, const Offs& x, const Offs& y) {
        return Offs{c ? x.a : y.a, c ? x.b : y.b, c ? x.c : y.c};
    }
    __device__ static void load_at(uint32_t (&r)[REGS], const uint8_t* b0, const uint8_t*, const Offs& o) {
        const u32x4 qa = ld_global128(b0 + o.a), qb = ld_global128(b0 + o.a + 16);
        const u32x4 h0 = ld_global128(b0 + o.b), h1 = ld_global128(b0 + o.b + 16);
        const u32x4 hd = ld_global128(b0 + o.c);
        r[0] = qa.x; r[1] = qa.y; r[2] = qa.z; r[3] = qa.w;
        r[4] = qb.x; r[5] = qb.y; r[6] = qb.z; r[7] = qb.w;
        r[8] = h0.x; r[9] = h0.y; r[10] = h0.z; r[11] = h0.w;
        r[12] = h1.x; r[13] = h1.y; r[14] = h1.z; r[15] = h1.w;
        r[16] = hd.x; r[17] = hd.y; r[18] = hd.z; r[19] = hd.w;
    }
    template <int MT>
    __device__ static void decode(const uint32_t (&r)[REGS], const Lane& LL, int u, bool live, const lds_u8* xa,
                                  int xmg_bytes, const lds_f32* xs, int xs_mg, float (&acc)[MT]) {
        constexpr int MG = (MT + 3) / 4;
        const Direct<QG_Q4_K>::Lane& L = LL.s;
        const uint32_t y = r[17], z = r[18], w = r[19];
        const uint32_t as = L.hi4 ? w : y, am = L.hi4 ? w : z;
        const uint32_t sc0 = __builtin_amdgcn_ubfe(as, L.off, L.wa) | (__builtin_amdgcn_ubfe(y, L.off + 6, L.wb) << 4);
        const uint32_t sc1 =
            __builtin_amdgcn_ubfe(as, L.off + 8, L.wa) | (__builtin_amdgcn_ubfe(y, L.off + 14, L.wb) << 4);
        const uint32_t m0 = __builtin_amdgcn_ubfe(am, L.oam, L.wa) | (__builtin_amdgcn_ubfe(z, L.off + 6, L.wb) << 4);
        const uint32_t m1 =
            __builtin_amdgcn_ubfe(am, L.oam + 8, L.wa) | (__builtin_amdgcn_ubfe(z, L.off + 14, L.wb) << 4);
        const float d = f16_to_f32(r[16]), dmin = f16_to_f32(r[16] >> 16);
        const float a0 = d * (float)sc0, a1 = d * (float)sc1;
        const float b0 = -(dmin * (float)m0), b1 = -(dmin * (float)m1);

        f32x4_t c0[MG], c1[MG];
#pragma unroll
        for (int g = 0; g < MG; ++g) c0[g] = c1[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const int rot = u & 3;
#pragma unroll
        for (int rp = 0; rp < 4; ++rp) {
            // values 8rp..8rp+7 of each sub-block: code dwords 2rp, 2rp+1 and the
            // fifth-bit bytes of the same positions (H dwords 2rp, 2rp+1): bit 2g
            // (sub-block 2g) or 2g + 1 (sub-block 2g + 1) of each byte, placed
            // as the E4M3 code 0x10 (16 * 2^-9) or 0
            const uint32_t e0 = r[8 + 2 * rp] >> LL.hsh, e1 = r[8 + 2 * rp + 1] >> LL.hsh;
            const uint32_t l0 = r[2 * rp] & 0x0F0F0F0Fu, l1 = r[2 * rp + 1] & 0x0F0F0F0Fu;
            const uint32_t h0 = (r[2 * rp] >> 4) & 0x0F0F0F0Fu, h1 = (r[2 * rp + 1] >> 4) & 0x0F0F0F0Fu;
            const uint32_t fl0 = (e0 << 4) & 0x10101010u, fl1 = (e1 << 4) & 0x10101010u;
            const uint32_t fh0 = (e0 << 3) & 0x10101010u, fh1 = (e1 << 3) & 0x10101010u;
            const uint32_t bl0 = int_pair_bf16<0>(l0), bl1 = int_pair_bf16<1>(l0);
            const uint32_t bl2 = int_pair_bf16<0>(l1), bl3 = int_pair_bf16<1>(l1);
            const uint32_t bh0 = int_pair_bf16<0>(h0), bh1 = int_pair_bf16<1>(h0);
            const uint32_t bh2 = int_pair_bf16<0>(h1), bh3 = int_pair_bf16<1>(h1);
            const uint32_t gl0 = int_pair_bf16<0>(fl0), gl1 = int_pair_bf16<1>(fl0);
            const uint32_t gl2 = int_pair_bf16<0>(fl1), gl3 = int_pair_bf16<1>(fl1);
            const uint32_t gh0 = int_pair_bf16<0>(fh0), gh1 = int_pair_bf16<1>(fh0);
            const uint32_t gh2 = int_pair_bf16<0>(fh1), gh3 = int_pair_bf16<1>(fh1);
#pragma unroll
            for (int g = 0; g < MG; ++g) {
                const u32x4 xl = lds_ld128(xa + g * xmg_bytes + ((rp ^ rot) * 4 * 16));
                const u32x4 xh = lds_ld128(xa + g * xmg_bytes + (((4 + rp) ^ rot) * 4 * 16));
                c0[g] = mfma4(xl.x, xl.y, bl0, bl1, c0[g]);
                c1[g] = mfma4(xh.x, xh.y, bh0, bh1, c1[g]);
                c0[g] = mfma4(xl.x, xl.y, gl0, gl1, c0[g]);
                c1[g] = mfma4(xh.x, xh.y, gh0, gh1, c1[g]);
                c0[g] = mfma4(xl.z, xl.w, bl2, bl3, c0[g]);
                c1[g] = mfma4(xh.z, xh.w, bh2, bh3, c1[g]);
                c0[g] = mfma4(xl.z, xl.w, gl2, gl3, c0[g]);
                c1[g] = mfma4(xh.z, xh.w, gh2, gh3, c1[g]);
            }
        }
        if (live) {
#pragma unroll
            for (int g = 0; g < MG; ++g) {
                const f32x4_t s0 = *(const QG_LDS f32x4_t*)(xs + (size_t)g * xs_mg + 8 * u);
                const f32x4_t s1 = *(const QG_LDS f32x4_t*)(xs + (size_t)g * xs_mg + 8 * u + 4);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (4 * g + i < MT) {
                        float a = acc[4 * g + i];
                        a = fmaf(a0, c0[g][i], a);
                        a = fmaf(b0, s0[i], a);
                        a = fmaf(a1, c1[g][i], a);
                        a = fmaf(b1, s1[i], a);
                        acc[4 * g + i] = a;
                    }
                }
            }
        }
    }
};

// NVFP4 (K a multiple of 64).  Unit u of a row = code bytes [32u, 32u + 32)
// (values 64u + [0,64), blocks 4u .. 4u + 3) and the four E4M3 scales of
// those blocks (one 4-byte load).  sum w x = g * sum_b s_b * sum c x; g is
// applied once per output.
template <> struct Direct<QG_NVFP4> {
    static constexpr int UV = 64;
    static constexpr int REGS = 9;
    static constexpr bool SUMS = false;
    struct Lane {};
    __device__ static Lane lane_consts(int) { return Lane{}; }
    __device__ __host__ static int units_per_row(int K) { return K / 64; }
    // Bytes of one pass (16 units) of a row: codes, scales.
    static constexpr int PASS0 = 16 * 32, PASS1 = 16 * 4;
    // Offsets from the start of a pass's stretch: codes (a), scales (b).
    struct Offs {
        uint32_t a, b;
    };
    __device__ static Offs slot_offs(int s) { return Offs{32u * (uint32_t)s, 4u * (uint32_t)s}; }
    __device__ static Offs shift(const Offs& o, uint32_t r0, uint32_t r1) { return Offs{o.a + r0, o.b + r1}; }
    __device__ static Offs pick(bool c, const Offs& x, const Offs& y) { return Offs{c ? x.a : y.a, c ? x.b : y.b}; }
    __device__ static void load_at(uint32_t (&r)[REGS], const uint8_t* b0, const uint8_t* b1, const Offs& o) {
        // ordinary loads: each instruction uses half of the lines it touches
        // (non-temporal loads of such lines were refetched)
        const u32x4 q0 = ld_global128(b0 + o.a), q1 = ld_global128(b0 + o.a + 16);
        r[0] = q0.x; r[1] = q0.y; r[2] = q0.z; r[3] = q0.w;
        r[4] = q1.x; r[5] = q1.y; r[6] = q1.z; r[7] = q1.w;
        r[8] = *(const QG_GLOBAL uint32_t*)(uintptr_t)(b1 + o.b);
    }
    template <int MT>
    __device__ static void decode(const uint32_t (&r)[REGS], const Lane&, int u, bool live, const lds_u8* xa,
                                  int xmg_bytes, const lds_f32*, int, float (&acc)[MT]) {
        constexpr int MG = (MT + 3) / 4;
        f32x4_t c[4][MG];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int g = 0; g < MG; ++g) c[q][g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const int rot = u & 3;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            // values 8h..8h+7 of each block q: code dword 2q + h
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t wv = r[2 * q + h];
                const uint32_t p0 = e2m1x2_to_bf16x2<0>(wv), p1 = e2m1x2_to_bf16x2<1>(wv);
                const uint32_t p2 = e2m1x2_to_bf16x2<2>(wv), p3 = e2m1x2_to_bf16x2<3>(wv);
#pragma unroll
                for (int g = 0; g < MG; ++g) {
                    const u32x4 xv = lds_ld128(xa + g * xmg_bytes + (((2 * q + h) ^ rot) * 4 * 16));
                    c[q][g] = mfma4(xv.x, xv.y, p0, p1, c[q][g]);
                    c[q][g] = mfma4(xv.z, xv.w, p2, p3, c[q][g]);
                }
            }
        }
        if (live) {
            const float s0 = e4m3_to_f32<0>(r[8]), s1 = e4m3_to_f32<1>(r[8]);
            const float s2 = e4m3_to_f32<2>(r[8]), s3 = e4m3_to_f32<3>(r[8]);
#pragma unroll
            for (int g = 0; g < MG; ++g)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (4 * g + i < MT) {
                        float a = acc[4 * g + i];
                        a = fmaf(s0, c[0][g][i], a);
                        a = fmaf(s1, c[1][g][i], a);
                        a = fmaf(s2, c[2][g][i], a);
                        a = fmaf(s3, c[3][g][i], a);
                        acc[4 * g + i] = a;
                    }
        }
    }
};

// Row-scaled FP8.  Unit u of a row = codes 64u .. 64u + 63, one E4M3 byte per
// value (exact in bf16); with them each lane loads the row's fp32 scale (the
// same 4 bytes for all units of a row: one line, no extra HBM traffic) and
// adds the unit's sum scaled by it.
template <> struct Direct<QG_FP8> {
    static constexpr int UV = 64;
    static constexpr int REGS = 17;
    static constexpr bool SUMS = false;
    struct Lane {};
    __device__ static Lane lane_consts(int) { return Lane{}; }
    __device__ __host__ static int units_per_row(int K) { return K / 64; }
    // Bytes of one pass (16 units) of a row: codes; the scale does not move.
    static constexpr int PASS0 = 16 * 64, PASS1 = 0;
    // Offsets from the start of a pass's stretch: codes (a), row scale (b).
    struct Offs {
        uint32_t a, b;
    };
    __device__ static Offs slot_offs(int s) { return Offs{64u * (uint32_t)s, 0u}; }
    __device__ static Offs shift(const Offs& o, uint32_t r0, uint32_t r1) { return Offs{o.a + r0, o.b + r1}; }
    __device__ static Offs pick(bool c, const Offs& x, const Offs& y) { return Offs{c ? x.a : y.a, c ? x.b : y.b}; }
    __device__ static void load_at(uint32_t (&r)[REGS], const uint8_t* b0, const uint8_t* b1, const Offs& o) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // ordinary (temporal) loads: an instruction covers a quarter of
            // each line it touches, and non-temporal loads of partly used
            // lines were refetched (0.41 -> 0.25 ms on a 1.27 GB head)
            const u32x4 q = ld_global128(b0 + o.a + 16 * i);
            r[4 * i] = q.x;
            r[4 * i + 1] = q.y;
            r[4 * i + 2] = q.z;
            r[4 * i + 3] = q.w;
        }
        r[16] = *(const QG_GLOBAL uint32_t*)(uintptr_t)(b1 + o.b);
    }
    template <int MT>
    __device__ static void decode(const uint32_t (&r)[REGS], const Lane&, int u, bool live, const lds_u8* xa,
                                  int xmg_bytes, const lds_f32*, int, float (&acc)[MT]) {
        constexpr int MG = (MT + 3) / 4;
        f32x4_t c[MG];
#pragma unroll
        for (int g = 0; g < MG; ++g) c[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const int rot = u & 3;
#pragma unroll
        for (int ch = 0; ch < 8; ++ch) {
            // values 8ch .. 8ch + 7: code dwords 2ch, 2ch + 1
            const uint32_t p0 = e4m3x2_to_bf16x2<0>(r[2 * ch]), p1 = e4m3x2_to_bf16x2<1>(r[2 * ch]);
            const uint32_t p2 = e4m3x2_to_bf16x2<0>(r[2 * ch + 1]), p3 = e4m3x2_to_bf16x2<1>(r[2 * ch + 1]);
#pragma unroll
            for (int g = 0; g < MG; ++g) {
                const u32x4 xv = lds_ld128(xa + g * xmg_bytes + ((ch ^ rot) * 4 * 16));
                c[g] = mfma4(xv.x, xv.y, p0, p1, c[g]);
                c[g] = mfma4(xv.z, xv.w, p2, p3, c[g]);
            }
        }
        if (live) {
            const float s = __builtin_bit_cast(float, r[16]);
#pragma unroll
            for (int g = 0; g < MG; ++g)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (4 * g + i < MT) acc[4 * g + i] = fmaf(s, c[g][i], acc[4 * g + i]);
        }
    }
};

// Q6_K.  Unit u of a row = quarter of super-block u / 4: half h = (u / 2) % 2,
// part t = u % 2, i.e. the 64 values 128h + 32p + 16t + [0,16), p = 0..3,
// each group of 16 with its own int8 sub-scale s[8h + 2p + t].  Its bytes: low
// nibbles ql[64h + 16t ..] (p = 0, 2: low / high nibble) and
// ql[64h + 32 + 16t ..] (p = 1, 3), 2-bit high parts qh[32h + 16t ..], the 8
// sub-scales of the half and d.  Blocks are 210 bytes, so these loads are
// only 2-byte aligned.
// w = d s (q - 32)  ->  sum w x = d s D with D = sum (q - 32) x, formed as
// sum lo x + sum 16 (hi - 2) x (lo the low nibble, hi the 2-bit high part,
// both exact bf16) in one fp32 chain.
template <> struct Direct<QG_Q6_K> {
    static constexpr int UV = 64;
    static constexpr int REGS = 15;
    static constexpr bool SUMS = false;
    struct Lane {
        uint32_t tsh;  // 8 * t: selects the part's sub-scales
    };
    __device__ static Lane lane_consts(int lane) { return Lane{8u * (uint32_t)((lane >> 2) & 1)}; }
    __device__ __host__ static int units_per_row(int K) { return (K / 256) * 4; }
    // Bytes of one pass (16 units = 4 blocks) of a row.
    static constexpr int PASS0 = 4 * 210, PASS1 = 0;
    // Offsets from the start of a pass's stretch: low-nibble codes (a; the
    // second half at a + 32), high bits (b), sub-scales (c), block start (d;
    // the fp16 scale at d + 208).
    struct Offs {
        uint32_t a, b, c, d;
    };
    __device__ static Offs slot_offs(int s) {
        const uint32_t blk = 210u * (uint32_t)(s >> 2), h = (uint32_t)(s >> 1) & 1u, t = (uint32_t)s & 1u;
        return Offs{blk + 64u * h + 16u * t, blk + 128u + 32u * h + 16u * t, blk + 192u + 8u * h, blk};
    }
    __device__ static Offs shift(const Offs& o, uint32_t r0, uint32_t) {
        return Offs{o.a + r0, o.b + r0, o.c + r0, o.d + r0};
    }
    __device__ static Offs pick(bool c, const Offs& x, const Offs& y) {
        return Offs{c ? x.a : y.a, c ? x.b : y.b, c ? x.c : y.c, c ? x.d : y.d};
    }
    // The 16- and 8-byte fields (2-byte aligned: 210-byte blocks) are read as
    // 4-byte aligned loads of the surrounding words shifted into place: the
    // loads of the LM head (whole rows, 1 GB) were address-unit bound, 238 ->
    // 210 us; the 5120-row down projections (K segments) 23.8 -> 22.3 us, and
    // 34.4 -> 33.3 us at 8 rows with one segment per workgroup.
    __device__ static void load_at(uint32_t (&r)[REGS], const uint8_t* b0, const uint8_t*, const Offs& o) {
        const u32x4 qa = ld_global128_a2dw(b0 + o.a);
        const u32x4 qb = ld_global128_a2dw(b0 + o.a + 32);
        const u32x4 qh = ld_global128_a2dw(b0 + o.b);
        const u32x2 sc = ld_global64_a2dw(b0 + o.c);
        r[0] = qa.x; r[1] = qa.y; r[2] = qa.z; r[3] = qa.w;
        r[4] = qb.x; r[5] = qb.y; r[6] = qb.z; r[7] = qb.w;
        r[8] = qh.x; r[9] = qh.y; r[10] = qh.z; r[11] = qh.w;
        r[12] = sc.x; r[13] = sc.y;
        r[14] = ld_global16(b0 + o.d + 208);
    }
    template <int MT>
    __device__ static void decode(const uint32_t (&r)[REGS], const Lane& L, int u, bool live, const lds_u8* xa,
                                  int xmg_bytes, const lds_f32* xs, int xs_mg, float (&acc)[MT]) {
        constexpr int MG = (MT + 3) / 4;
        f32x4_t c[4][MG];
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
            for (int g = 0; g < MG; ++g) c[p][g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const int rot = u & 3;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // values 4i..4i+3 of each of the 4 groups: low nibbles and the
            // 2-bit high parts, one byte per value
            const uint32_t A = r[i], B = r[4 + i], H = r[8 + i];
            const uint32_t lo[4] = {A & 0x0F0F0F0Fu, B & 0x0F0F0F0Fu, (A >> 4) & 0x0F0F0F0Fu,
                                    (B >> 4) & 0x0F0F0F0Fu};
            const uint32_t hi[4] = {H & 0x03030303u, (H >> 2) & 0x03030303u, (H >> 4) & 0x03030303u,
                                    (H >> 6) & 0x03030303u};
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t b0 = int_pair_bf16<0>(lo[p]), b1 = int_pair_bf16<1>(lo[p]);
                const uint32_t hc = q6_high_codes(hi[p]);
                const uint32_t e0 = int_pair_bf16<0>(hc), e1 = int_pair_bf16<1>(hc);
#pragma unroll
                for (int g = 0; g < MG; ++g) {
                    // position group 2p + i/2 holds values 8(i/2)..8(i/2)+7 of group p
                    const u32x4 xv = lds_ld128(xa + g * xmg_bytes + (((2 * p + (i >> 1)) ^ rot) * 4 * 16));
                    const uint32_t x0 = (i & 1) ? xv.z : xv.x, x1 = (i & 1) ? xv.w : xv.y;
                    c[p][g] = mfma4(x0, x1, b0, b1, c[p][g]);
                    c[p][g] = mfma4(x0, x1, e0, e1, c[p][g]);
                }
            }
        }
        if (live) {
            const float d = f16_to_f32(r[14]);
            const uint32_t st = r[12] >> L.tsh, su = r[13] >> L.tsh;
            float a[4];
            a[0] = d * (float)(int8_t)(st & 0xffu);
            a[1] = d * (float)(int8_t)((st >> 16) & 0xffu);
            a[2] = d * (float)(int8_t)(su & 0xffu);
            a[3] = d * (float)(int8_t)((su >> 16) & 0xffu);
#pragma unroll
            for (int g = 0; g < MG; ++g) {
#pragma unroll
                for (int p = 0; p < 4; ++p) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        if (4 * g + i < MT) acc[4 * g + i] = fmaf(a[p], c[p][g][i], acc[4 * g + i]);
                    }
                }
            }
        }
    }
};

// ---------------------------------------------------------------- activation layout
//
// Group mg of 4 activation rows, unit u, position group pg (values 8pg..8pg+7
// of the unit), row slot m4: 16 bytes at
//     mg * MGB + u * UB + ((pg ^ (u % 4)) * 4 + m4) * 16.
// The 4 row slots are always allocated (rows >= MT are simply never written);
// A operands of lanes whose slot is >= MT read slot 0 instead.

__host__ __device__ constexpr int direct_uv(int) { return 64; }
__host__ __device__ constexpr int direct_mg(int mt) { return (mt + 3) / 4; }
__host__ __device__ constexpr int direct_units(int K) { return K / 64; }
// Activation sums per unit (the sub-blocks whose mins need sum x): Q4_K and
// Q5_K 2 x 32 values; the other formats need none.
__host__ __device__ constexpr int direct_sub(int fmt) { return fmt == QG_Q4_K || fmt == QG_Q5_K ? 2 : 0; }
// Bytes of one unit for one group of 4 activation rows.
__host__ __device__ constexpr int direct_unit_bytes(int) { return 8 * 4 * 16; }
// Bytes of one group of 4 activation rows (all units).
__host__ __device__ constexpr int direct_mg_bytes(int fmt, int K) { return direct_units(K) * direct_unit_bytes(fmt); }
// Floats of per-sub-block sums per group of 4 rows.
__host__ __device__ constexpr int direct_xs_mg(int fmt, int K) { return direct_units(K) * direct_sub(fmt) * 4; }
__host__ __device__ constexpr size_t direct_lds_bytes(int fmt, int mt, int K) {
    return (size_t)direct_mg(mt) * direct_mg_bytes(fmt, K) + (size_t)direct_mg(mt) * direct_xs_mg(fmt, K) * 4;
}
// Unit and position group (8 values) holding activation position k (a
// multiple of 8).  Q4_K / NVFP4: units are 64 consecutive values.  Q6_K: unit
// 4 b + 2 h + t holds values 256 b + 128 h + 32 p + 16 t + 8 e + [0,8) as
// position group 2 p + e.
__host__ __device__ constexpr int direct_pos_unit(int fmt, int k) {
    return fmt == QG_Q6_K ? 4 * (k >> 8) + 2 * ((k >> 7) & 1) + ((k >> 4) & 1) : k >> 6;
}
__host__ __device__ constexpr int direct_pos_group(int fmt, int k) {
    return fmt == QG_Q6_K ? 2 * ((k >> 5) & 3) + ((k >> 3) & 1) : (k & 63) >> 3;
}
// Byte offset of (activation row m, unit u, position group pg).
__host__ __device__ constexpr int direct_x_at(int fmt, int K, int m, int u, int pg) {
    return (m / 4) * direct_mg_bytes(fmt, K) + u * direct_unit_bytes(fmt) + (((pg ^ (u & 3)) * 4) + (m % 4)) * 16;
}
// Byte offset of activation row m, values k..k+7 (k a multiple of 8).
__host__ __device__ constexpr int direct_x_offset(int fmt, int K, int m, int k) {
    return direct_x_at(fmt, K, m, direct_pos_unit(fmt, k), direct_pos_group(fmt, k));
}

// Source row of pass row m (< MT) from MT wave-uniform values resolved once.
// Lane q of one register holds row q (set lane by lane from scalars) and a
// lane fetches its row with a cross-lane permute, which waits on LDS-unit
// counters only.  A row lookup that loads from memory, or a select chain that
// the compiler turns into an indexed private array, made every staging load
// wait for all the loads in flight before it.
template <int MT>
struct RowTable {
    int r0 = 0, lanes = 0;
    __device__ __forceinline__ void set(int q, int row) {
        row = __builtin_amdgcn_readfirstlane(row);
        if (q == 0) r0 = row;
        lanes = (int)(threadIdx.x & 63) == q ? row : lanes;
    }
    __device__ __forceinline__ int operator()(int m) const {
        if constexpr (MT == 1) return r0;
        else return __builtin_amdgcn_ds_bpermute(m << 2, lanes);
    }
};

// Activation staging in the interleaved layout, split in two so that the
// weight loads can be issued in between: issue() loads up to XV 16-byte
// vectors per thread into registers, commit() writes them (and any vectors
// beyond XV per thread) to LDS, then, for Q4_K and Q5_K, computes the
// per-32-value sums (sequential order).  Rows >= cnt are zero.  commit() ends
// with a workgroup barrier.
// EAGER issues every load of a batch without waiting: the row comes from a
// RowTable, the loads sit under wave-uniform guards only, and the zero mask of
// absent rows is applied when the values are written.  Otherwise each vector's
// load sits under a per-lane test and the row lookup may read memory, which
// makes the compiler wait for all earlier loads before each one: measured
// 1-2 % slower for one activation row at 8 waves per workgroup, but 6-17 %
// faster for NVFP4 at 8 rows with 16 waves and 2 % faster in the grouped
// kernel, where the staging loads otherwise crowd out the first weight loads.
template <int F, int MT, int XV, bool EAGER = false>
struct XStage {
    u32x4 v[XV];
    // Vector i of the pass (rows >= cnt and i >= nvec read vector 0 of row 0;
    // valid() says whether to keep it).  Nothing here waits for the load.
    template <class RowOf>
    __device__ __forceinline__ static u32x4 load(const uint16_t* x, int64_t ldx, int cnt, int K, int i,
                                                 RowOf row_of) {
        const int ii = valid(cnt, K, i) ? i : 0;
        return ld_global128(x + (size_t)row_of((ii * 8) / K) * ldx + (ii * 8) % K);
    }
    __device__ __forceinline__ static bool valid(int cnt, int K, int i) {
        return i < MT * K / 8 && (i * 8) / K < cnt;
    }
    // vectors per thread that hold rows present (wave-uniform)
    __device__ __forceinline__ static int needed(int cnt, int K) {
        return (min(cnt, MT) * K / 8 + (int)blockDim.x - 1) / (int)blockDim.x;
    }
    template <class RowOf>
    __device__ __forceinline__ void issue(const uint16_t* x, int64_t ldx, int cnt, int K, RowOf row_of) {
        if constexpr (EAGER) {
            const int need = needed(cnt, K);
#pragma unroll
            for (int j = 0; j < XV; ++j)
                if (j < need) v[j] = load(x, ldx, cnt, K, threadIdx.x + j * blockDim.x, row_of);
        } else {
#pragma unroll
            for (int j = 0; j < XV; ++j) {
                const int i = threadIdx.x + j * blockDim.x;
                v[j] = u32x4{0u, 0u, 0u, 0u};
                if (valid(cnt, K, i)) v[j] = ld_global128(x + (size_t)row_of((i * 8) / K) * ldx + (i * 8) % K);
            }
        }
    }
    template <class RowOf>
    __device__ __forceinline__ void commit(lds_u8* xl, lds_f32* xs, const uint16_t* x, int64_t ldx, int cnt, int K,
                                           RowOf row_of) {
        const int nvec = MT * K / 8;
        const u32x4 zero = {0u, 0u, 0u, 0u};
        auto put = [&](int i, const u32x4& val) {
            const int m = (i * 8) / K, k = (i * 8) % K;
            *(lds_u32x4*)(xl + direct_x_offset(F, K, m, k)) = valid(cnt, K, i) ? val : zero;
        };
        if constexpr (EAGER) {
            const int need = needed(cnt, K);
#pragma unroll
            for (int j = 0; j < XV; ++j) {
                const int i = threadIdx.x + j * blockDim.x;
                if (i < nvec) put(i, j < need ? v[j] : zero);
            }
            for (int base = XV * blockDim.x; base < nvec; base += XV * blockDim.x) {
                const int more = need - base / (int)blockDim.x;
                u32x4 t[XV];
#pragma unroll
                for (int j = 0; j < XV; ++j)
                    if (j < more) t[j] = load(x, ldx, cnt, K, base + threadIdx.x + j * blockDim.x, row_of);
#pragma unroll
                for (int j = 0; j < XV; ++j) {
                    const int i = base + threadIdx.x + j * blockDim.x;
                    if (i < nvec) put(i, j < more ? t[j] : zero);
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < XV; ++j) {
                const int i = threadIdx.x + j * blockDim.x;
                if (i < nvec) put(i, v[j]);
            }
            for (int i = threadIdx.x + XV * blockDim.x; i < nvec; i += blockDim.x) {
                u32x4 val = zero;
                if (valid(cnt, K, i)) val = ld_global128(x + (size_t)row_of((i * 8) / K) * ldx + (i * 8) % K);
                put(i, val);
            }
        }
        if constexpr (Direct<F>::SUMS) {
            // sum of each sub-block's values (K order) per activation row
            constexpr int SUB = direct_sub(F), PPS = 8 / SUB;  // position groups per sub-block
            __syncthreads();
            const int U = direct_units(K);
            for (int i = threadIdx.x; i < MT * U * SUB; i += blockDim.x) {
                const int m = i / (U * SUB), rem = i % (U * SUB), u = rem / SUB, p = rem % SUB;
                float s = 0.f;
#pragma unroll
                for (int t = 0; t < PPS; ++t) {
                    const u32x4 q = lds_ld128(xl + direct_x_at(F, K, m, u, p * PPS + t));
                    const uint32_t wv[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        s += bf16_to_f32(wv[e]);
                        s += bf16_to_f32(wv[e] >> 16);
                    }
                }
                xs[(size_t)(m / 4) * direct_xs_mg(F, K) + (u * SUB + p) * 4 + (m % 4)] = s;
            }
        }
        __syncthreads();
    }
};

// Activation row slot a lane writes its result for: its unit slot.
__device__ __forceinline__ int direct_out_slot(int lane) { return lane >> 2; }

// K segments of a row: a row of P passes is cut into S segments of PS passes
// (the last one shorter).  The cut depends only on (format, N, K) and the
// device's CU count, never on the number of activation rows, so every output
// keeps one arithmetic: the segment sums are added in segment order.  Rows
// are split only when there are too few row groups to occupy the waves.
struct Segments {
    int S, PS;
};
// Rows are split only while a CU has fewer than this many row groups (one
// per wave of a 16-wave workgroup); then into as many segments as keep the
// items of a CU within its 16 waves (5 row groups per CU: 3 segments, 15
// items -- measured fastest on the 5120 x 17408 shapes against 2, 4, 5, 9).
constexpr int kDirectSegRgsMax = 16;
inline Segments direct_segments(int fmt, int64_t N, int K, int cus) {
    const int P = (K / 64 + kDirectSlots - 1) / kDirectSlots;
    const int64_t groups = (N + kDirectRows - 1) / kDirectRows;
    const int64_t per_cu = (groups + cus - 1) / cus;
    int S = 1;
    if (per_cu < kDirectSegRgsMax) S = (int)(kDirectSegRgsMax / per_cu);
    if (S > P) S = P;
    if (S < 1) S = 1;
    const int PS = (P + S - 1) / S;
    (void)fmt;
    return Segments{(P + PS - 1) / PS, PS};
}

// LDS of the segment sums for `rgs` row groups (none when rows are not split).
inline size_t direct_seg_lds_bytes(int S, int rgs, int mt) {
    return S > 1 ? ((size_t)rgs * 4 + 15) / 16 * 16 + (size_t)rgs * kDirectRows * mt * 4 : 0;
}

// Ordered accumulation of the segment sums of a workgroup's row groups in
// LDS: total[(rg_local * 4 + row) * MTMAX + m] and progress[rg_local] (the
// number of segments already added).  Both start at zero.
struct SegLds {
    lds_f32* total;
    QG_LDS int* progress;
    int mtmax;
    // segments on different workgroups: sums [row group][segment][4][MT] and
    // per-row-group counters in global memory
    float* gpart;
    int32_t* gcnt;
};

// The K range whose activations are staged in LDS: segments [s_lo, s_lo + ns)
// of every row, i.e. units [u0, u0 + KL / 64).  One phase covers the whole row
// unless the activations of all rows do not fit in LDS at once.
struct Phase {
    int s_lo, ns, u0, KL;
};

// One wave streams work items handed out by next_item() (an item index local
// to the workgroup, or a negative value when there are none left): item t is
// segment ph.s_lo + t % ph.ns of row group rg_base + t / ph.ns of mv; row group rg is rows
// 4 rg .. 4 rg + 3 (rows >= N idle), lane l serving row l % 4.  A segment is
// up to PS passes of 16 units, SP passes per ring slot, PF slots in flight;
// the ring always holds the next PF slots of work, refilled as soon as a slot
// is decoded.  Lane l with slot s = l / 4 < cnt writes y[yrow * ldy + n] for
// activation row s (yrow given for that slot).  between() runs once, after
// the first PF slots are in flight (the activation staging: a workgroup
// barrier inside, so every wave of the workgroup must call this function).
// SEG false: the caller has one segment per row and one phase over all of K
// (sg and ph are then ignored).
template <int F, int MT, int SP, int PF, bool SEG, bool XS = false, class Next, class Between>
__device__ __forceinline__ void wave_stream_direct(const MatView& mv, int N, int K, const lds_u8* xl,
                                                   const lds_f32* xs, Next next_item, int rg_base, Segments sg,
                                                   Phase ph, SegLds sl, float* y, int64_t ldy, int64_t yrow,
                                                   int cnt, Between between) {
    using D = Direct<F>;
    constexpr int RW = kDirectRows, G = kDirectSlots;
    const int lane = threadIdx.x & 63;
    const int grp = lane & 3, slot = lane >> 2;
    const int U = D::units_per_row(K);
    const int P = (U + G - 1) / G;
    // segments and phase (compile-time one segment, one phase when !SEG)
    const int S = SEG ? sg.S : 1, PS = SEG ? sg.PS : P;
    const int NS = SEG ? ph.ns : 1, SLO = SEG ? ph.s_lo : 0, U0 = SEG ? ph.u0 : 0, KL = SEG ? ph.KL : K;
    const typename D::Lane L = D::lane_consts(lane);
    const int ub = direct_unit_bytes(F);
    const int mgb = direct_mg_bytes(F, KL);
    const int xs_mg = direct_xs_mg(F, KL);
    // A-operand row slot of this lane: lane % 4 (slots >= MT read slot 0: their
    // products land in result rows nobody uses)
    const int aslot = (lane & 3) < MT ? (lane & 3) : 0;
    const lds_u8* xa_lane = xl + aslot * 16;

    float gscale = 1.f;
    if (F == QG_NVFP4) {
        const uint8_t* gb = mv.gbytes;
        const uint32_t bits = (uint32_t)gb[0] | ((uint32_t)gb[1] << 8) | ((uint32_t)gb[2] << 16) |
                              ((uint32_t)gb[3] << 24);
        gscale = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(bits));
    }

    uint32_t R[PF][SP][D::REGS];
    // Per ring slot: local row group of its item (< 0: none), segment, first
    // pass, end pass of the segment, and whether the slot ends the item.
    int slot_g[PF], slot_s[PF], slot_p[PF], slot_e[PF];
    bool slot_last[PF];

    // Load addresses: a uniform base per (row group, pass) and per-lane
    // offsets fixed for the whole run (unit slot, row of the group), so a pass
    // costs no per-lane address arithmetic.  On a last, partial pass (U not a
    // multiple of 16) slots past the row's end read a live slot of that pass.
    const typename D::Offs o_slot = D::slot_offs(slot);
    const int live_last = U - (P - 1) * G;  // live slots of the last pass, 1..16
    const typename D::Offs o_last = D::slot_offs(slot < live_last ? slot : slot % live_last);
    const uint32_t lrow0 = (uint32_t)grp * (uint32_t)mv.rb0;
    const uint32_t lrow1 = F == QG_NVFP4 || F == QG_FP8 ? (uint32_t)grp * (uint32_t)mv.rb1 : 0u;

    // current item: local row group, segment, pass cursor and end pass; its
    // row group's bases and this lane's offsets (rows past N read the group's
    // first row).  With no work left the bases stay those of the last item
    // (initially row 0), so every load stays in the matrix.
    int cur_g = -1, cur_s = 0, cur_p = 0, cur_end = 0;
    const uint8_t *cur_b0 = mv.w0, *cur_b1 = mv.w1;
    typename D::Offs cur_o = o_slot, cur_ol = o_last;
    auto fetch = [&]() {
        const int t = next_item();
        cur_g = -1;
        if (t >= 0) {
            int q = t, r = 0;
            if (NS > 1) {
                q = t / NS;
                r = t - q * NS;
            }
            cur_g = q;
            cur_s = SLO + r;
            cur_p = cur_s * PS;
            cur_end = min(P, cur_p + PS);
            const int rg = rg_base + q;
            cur_b0 = mv.w0 + (size_t)(RW * rg) * mv.rb0;
            cur_b1 = F == QG_NVFP4 || F == QG_FP8 ? mv.w1 + (size_t)(RW * rg) * mv.rb1 : nullptr;
            const bool real = RW * rg + grp < N;
            cur_o = D::shift(o_slot, real ? lrow0 : 0u, real ? lrow1 : 0u);
            cur_ol = D::shift(o_last, real ? lrow0 : 0u, real ? lrow1 : 0u);
        }
    };
    fetch();
    // Issues the next SP passes of work into a slot (with no work left, loads
    // that stay in one line: every path issues the same loads).
    auto issue = [&](uint32_t (&r)[SP][D::REGS], int& sgi, int& ss, int& sp, int& se, bool& slast) {
        const bool live = cur_g >= 0;
        sgi = cur_g;
        ss = cur_s;
        sp = cur_p;
        se = cur_end;
#pragma unroll
        for (int p = 0; p < SP; ++p) {
            // passes past the item's end (SP > 1) repeat its first pass
            const int pass = !live ? 0 : (cur_p + p < cur_end ? cur_p + p : cur_p);
            const bool partial = (pass + 1) * G > U;
            // no work: every lane loads the first bytes of the last row group
            // (one line; nothing streams for a dead slot)
            const typename D::Offs o = D::pick(live, D::pick(partial, cur_ol, cur_o), typename D::Offs{});
            D::load_at(r[p], cur_b0 + (size_t)pass * D::PASS0, cur_b1 + (size_t)pass * D::PASS1, o);
        }
        slast = false;
        if (live) {
            cur_p += SP;
            if (cur_p >= cur_end) {
                slast = true;
                fetch();
            }
        }
    };

    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.f;

    auto process = [&](const uint32_t (&r)[SP][D::REGS], int rgl, int s, int p0, int pend, bool last) {
#pragma unroll
        for (int p = 0; p < SP; ++p) {
            const int u = (p0 + p) * G + slot;
            const bool live = p0 + p < pend && u < U;
            // activations of this phase are staged from unit U0 on (a multiple of
            // 16, so the bank rotation u % 4 is unchanged)
            const int ux = live ? u - U0 : 0;
            D::template decode<MT>(r[p], L, ux, live, xa_lane + (size_t)ux * ub, mgb, xs, xs_mg, acc);
        }
        if (last) {
            const int n = RW * (rg_base + rgl) + grp;
            float mine = slot_sum_rows<MT>(acc, slot);
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[m] = 0.f;
            bool store = s == S - 1;
            if constexpr (XS) {
                // The segments of a row group run on different workgroups and a
                // workgroup has one segment: this item's sums wait in LDS (one
                // slot per row group) for the workgroup's end, where they go to
                // the workspace together (no wait here on the wave's stores,
                // which would drain its load ring)
                store = false;
                if (slot < MT) sl.total[(size_t)(rgl * RW + grp) * MT + slot] = mine;
            } else if (S > 1) {
                // add this segment after the ones before it, in segment order
                // (the oldest unfinished item never waits, so this ends; the
                // bound only guarantees that every wave exits)
                QG_LDS int* prog = sl.progress + rgl;
                bool in_order = false;
                for (int spin = 0; spin < (1 << 22); ++spin) {
                    if (__hip_atomic_load(prog, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == s) {
                        in_order = true;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
                lds_f32* tp = sl.total + (size_t)(rgl * RW + grp) * sl.mtmax + (slot < MT ? slot : 0);
                if (slot < MT) {
                    // a wait that gave up would add out of order: the row's
                    // result is poisoned instead of silently reordered
                    const float sum = !in_order ? __builtin_nanf("") : s == 0 ? mine : *tp + mine;
                    *tp = sum;
                    mine = sum;
                }
                __hip_atomic_store(prog, s + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
            if (store) {
                if (F == QG_NVFP4) mine *= gscale;
                if (slot < cnt && n < N) st_global_f32(y + yrow * ldy + n, mine);
            }
        }
    };

#pragma unroll
    for (int k = 0; k < PF; ++k) issue(R[k], slot_g[k], slot_s[k], slot_p[k], slot_e[k], slot_last[k]);
    between();
    while (slot_g[0] >= 0) {
#pragma unroll
        for (int k = 0; k < PF; ++k) {
            if (slot_g[k] >= 0) process(R[k], slot_g[k], slot_s[k], slot_p[k], slot_e[k], slot_last[k]);
            issue(R[k], slot_g[k], slot_s[k], slot_p[k], slot_e[k], slot_last[k]);
        }
    }
}

inline bool direct_eligible(int fmt, int K) {
    return fmt == QG_Q4_K || fmt == QG_Q5_K || fmt == QG_Q6_K || fmt == QG_FP8 || (fmt == QG_NVFP4 && K % 64 == 0);
}

}  // namespace qg
