// qg_direct.h -- register-direct weight streaming for the 16-byte aligned
// formats (Q4_K, and NVFP4 with K a multiple of 32).
//
// A wave works on 64/G rows at once, G lanes per row.  Every lane loads its
// own decode unit straight into registers: Q4_K one quarter of a super-block
// (32 code bytes = 64 values, sub-blocks 2g and 2g+1) plus the block's 16-byte
// header; NVFP4 16 code bytes (32 values) plus their two E4M3 scales.  Across
// the G lanes of a row these loads cover a contiguous stretch of the row, so
// the stream stays coalesced and the weights never pass through LDS.  Unit
// u of a row sits on lane u % G in pass u / G, so every constant derived from
// a lane's place inside a block is fixed for the whole kernel, and the per-row
// summation order depends only on (format, K).
//
// Activations live in LDS with 16 bytes of padding after each unit's span of
// values, so the G lanes of a row read them without bank conflicts; the lanes
// of the other rows of the wave read the same addresses (a broadcast).
#pragma once

#include "qg_stream.h"

namespace qg {

// Lane-group reductions with DPP (the groups are 16-lane DPP rows); the
// result lands in every lane of the group.
__device__ __forceinline__ float dpp_sum16(float v) {
    auto add = [](float x, int ctrl) {
        int y;
        switch (ctrl) {
            case 0: y = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false); break;
            case 1: y = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false); break;
            case 2: y = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false); break;
            default: y = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false); break;
        }
        return x + __builtin_bit_cast(float, y);
    };
    v = add(v, 0);  // quad_perm [1,0,3,2]: pairs
    v = add(v, 1);  // quad_perm [2,3,0,1]: quads
    v = add(v, 2);  // row_half_mirror: 8 lanes
    v = add(v, 3);  // row_mirror: 16 lanes
    return v;
}

template <int G>
__device__ __forceinline__ float group_sum(float v) {
    v = dpp_sum16(v);
    if (G >= 32) v += __shfl_xor(v, 16, kWave);
    if (G >= 64) v += __shfl_xor(v, 32, kWave);
    return v;
}

template <int F> struct Direct;

// Q4_K.  Unit u of a row = quarter g = u % 4 of super-block u / 4: code bytes
// [32g, 32g + 32), whose low nibbles are the 32 values of sub-block 2g and
// high nibbles the 32 values of sub-block 2g + 1.
// sum w x = a0 (D0 - 128 X0) - dmin m0 X0 + a1 (...) with a = d * sc,
// D = sum (128 + q) x and X = sum x over the sub-block.
template <> struct Direct<QG_Q4_K> {
    static constexpr int G = 16;    // lanes per row
    static constexpr int XG = 64;   // activation values per unit (padding granule)
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
        int unit0;  // unit index in pass 0
    };
    __device__ static Lane lane_consts(int lane) {
        Lane L;
        const int i = lane & (G - 1), g = i & 3;
        L.hi4 = g >= 2;
        L.off = 16u * (uint32_t)(g & 1);
        L.oam = L.off + (L.hi4 ? 4u : 0u);
        L.wa = L.hi4 ? 4u : 6u;
        L.wb = L.hi4 ? 2u : 0u;
        L.unit0 = i;
        return L;
    }
    __device__ __host__ static int units_per_row(int K) { return (K / 256) * 4; }
    __device__ static void load(uint32_t (&r)[REGS], const uint8_t* row, const uint8_t*, int u) {
        const uint8_t* blk = row + 144 * (u >> 2);
        const uint8_t* q = blk + 16 + 32 * (u & 3);
        // Plain (cached) loads: the three loads of a lane touch the same lines as
        // those of its neighbours, and non-temporal loads fetched them again.
        const u32x4 qa = ld_global128(q), qb = ld_global128(q + 16), h = ld_global128(blk);
        r[0] = qa.x; r[1] = qa.y; r[2] = qa.z; r[3] = qa.w;
        r[4] = qb.x; r[5] = qb.y; r[6] = qb.z; r[7] = qb.w;
        r[8] = h.x; r[9] = h.y; r[10] = h.z; r[11] = h.w;
    }
    template <int MT>
    __device__ static void decode(const uint32_t (&r)[REGS], const Lane& L, int u, const lds_u8* xl,
                                  const lds_f32* xs, int xrow_bytes, int xs_row, float (&acc)[MT]) {
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
        const float b0 = -fmaf(dmin, (float)m0, 128.f * a0);
        const float b1 = -fmaf(dmin, (float)m1, 128.f * a1);
        uint32_t lo[8], hi[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            lo[i] = r[i] & 0x0F0F0F0Fu;
            hi[i] = (r[i] >> 4) & 0x0F0F0F0Fu;
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const lds_u8* xp = xl + (size_t)m * xrow_bytes + (size_t)u * (2 * XG + 16);
            const XPairs x0 = load_x16(xp, 0), x1 = load_x16(xp, 16), x2 = load_x16(xp, 32), x3 = load_x16(xp, 48);
            // The two sums as a float pair: __builtin_bit_cast of a vector element
            // (s.y) read element 0 under this compiler.
            const f32x2 s = *(const QG_LDS f32x2*)(xs + (size_t)m * xs_row + 2 * u);
            float d0 = 0.f, d1 = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                d0 = dot2bf(bias128_pair(lo[i], kSelB0B1), x0.v[2 * i], d0);
                d0 = dot2bf(bias128_pair(lo[i], kSelB2B3), x0.v[2 * i + 1], d0);
                d1 = dot2bf(bias128_pair(hi[i], kSelB0B1), x2.v[2 * i], d1);
                d1 = dot2bf(bias128_pair(hi[i], kSelB2B3), x2.v[2 * i + 1], d1);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                d0 = dot2bf(bias128_pair(lo[4 + i], kSelB0B1), x1.v[2 * i], d0);
                d0 = dot2bf(bias128_pair(lo[4 + i], kSelB2B3), x1.v[2 * i + 1], d0);
                d1 = dot2bf(bias128_pair(hi[4 + i], kSelB0B1), x3.v[2 * i], d1);
                d1 = dot2bf(bias128_pair(hi[4 + i], kSelB2B3), x3.v[2 * i + 1], d1);
            }
            float a = acc[m];
            a = fmaf(a0, d0, a);
            a = fmaf(b0, s.x, a);
            a = fmaf(a1, d1, a);
            a = fmaf(b1, s.y, a);
            acc[m] = a;
        }
    }
};

// NVFP4 (K a multiple of 32).  Unit u of a row = code bytes [16u, 16u + 16)
// (values 32u + [0,32), blocks 2u and 2u + 1) and the two E4M3 scales of those
// blocks.  sum w x = g * sum_b s_b * sum c x; g is applied once per output.
template <> struct Direct<QG_NVFP4> {
    static constexpr int G = 32;
    static constexpr int XG = 32;
    static constexpr int REGS = 5;
    static constexpr bool SUMS = false;
    struct Lane {
        int unit0;
    };
    __device__ static Lane lane_consts(int lane) { return Lane{lane & (G - 1)}; }
    __device__ __host__ static int units_per_row(int K) { return K / 32; }
    __device__ static void load(uint32_t (&r)[REGS], const uint8_t* row_codes, const uint8_t* row_scales, int u) {
        const u32x4 q = ld_stream128(row_codes + 16 * u);
        r[0] = q.x; r[1] = q.y; r[2] = q.z; r[3] = q.w;
        r[4] = __builtin_nontemporal_load((const QG_GLOBAL uint16_t*)(uintptr_t)(row_scales + 2 * u));
    }
    template <int MT>
    __device__ static void decode(const uint32_t (&r)[REGS], const Lane&, int u, const lds_u8* xl, const lds_f32*,
                                  int xrow_bytes, int, float (&acc)[MT]) {
        const float s0 = e4m3_to_f32<0>(r[4]), s1 = e4m3_to_f32<1>(r[4]);
        uint32_t p0[8], p1[8];
        p0[0] = e2m1x2_to_bf16x2<0>(r[0]); p0[1] = e2m1x2_to_bf16x2<1>(r[0]);
        p0[2] = e2m1x2_to_bf16x2<2>(r[0]); p0[3] = e2m1x2_to_bf16x2<3>(r[0]);
        p0[4] = e2m1x2_to_bf16x2<0>(r[1]); p0[5] = e2m1x2_to_bf16x2<1>(r[1]);
        p0[6] = e2m1x2_to_bf16x2<2>(r[1]); p0[7] = e2m1x2_to_bf16x2<3>(r[1]);
        p1[0] = e2m1x2_to_bf16x2<0>(r[2]); p1[1] = e2m1x2_to_bf16x2<1>(r[2]);
        p1[2] = e2m1x2_to_bf16x2<2>(r[2]); p1[3] = e2m1x2_to_bf16x2<3>(r[2]);
        p1[4] = e2m1x2_to_bf16x2<0>(r[3]); p1[5] = e2m1x2_to_bf16x2<1>(r[3]);
        p1[6] = e2m1x2_to_bf16x2<2>(r[3]); p1[7] = e2m1x2_to_bf16x2<3>(r[3]);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const lds_u8* xp = xl + (size_t)m * xrow_bytes + (size_t)u * (2 * XG + 16);
            const XPairs x0 = load_x16(xp, 0), x1 = load_x16(xp, 16);
            float d0 = 0.f, d1 = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                d0 = dot2bf(p0[i], x0.v[i], d0);
                d1 = dot2bf(p1[i], x1.v[i], d1);
            }
            acc[m] = fmaf(s1, d1, fmaf(s0, d0, acc[m]));
        }
    }
};

__host__ __device__ constexpr int direct_group_lanes(int fmt) { return fmt == QG_Q4_K ? 16 : 32; }
__host__ __device__ constexpr int direct_xg(int fmt) { return fmt == QG_Q4_K ? 64 : 32; }

// Bytes of one padded activation row and of the per-row sums (Q4_K: one fp32
// per 32 values).
__host__ __device__ constexpr int direct_xrow_bytes(int fmt, int K) {
    return (K / direct_xg(fmt)) * (2 * direct_xg(fmt) + 16);
}
__host__ __device__ constexpr int direct_xs_row(int fmt, int K) { return fmt == QG_Q4_K ? K / 32 : 0; }
__host__ __device__ constexpr size_t direct_lds_bytes(int fmt, int mt, int K) {
    return (size_t)mt * direct_xrow_bytes(fmt, K) + (size_t)mt * direct_xs_row(fmt, K) * 4;
}

// Activation staging in the padded layout, split in two so that the weight
// loads can be issued in between: issue() loads up to XV 16-byte vectors per
// thread into registers, commit() writes them (and any vectors beyond XV per
// thread, loaded and written on the spot) to LDS, then, for Q4_K, computes the
// per-32-value sums (sequential order).  Rows >= cnt are zero.  commit() ends
// with a workgroup barrier.
template <int F, int MT, int XV>
struct XStage {
    u32x4 v[XV];
    template <class RowOf>
    __device__ __forceinline__ void issue(const uint16_t* x, int64_t ldx, int cnt, int K, RowOf row_of) {
        const int nvec = MT * K / 8;
#pragma unroll
        for (int j = 0; j < XV; ++j) {
            const int i = threadIdx.x + j * blockDim.x;
            v[j] = u32x4{0u, 0u, 0u, 0u};
            if (i < nvec) {
                const int m = (i * 8) / K, k = (i * 8) % K;
                if (m < cnt) v[j] = ld_global128(x + (size_t)row_of(m) * ldx + k);
            }
        }
    }
    template <class RowOf>
    __device__ __forceinline__ void commit(lds_u8* xl, lds_f32* xs, const uint16_t* x, int64_t ldx, int cnt, int K,
                                           RowOf row_of) {
        constexpr int XG = Direct<F>::XG;
        const int xrow = direct_xrow_bytes(F, K);
        const int nvec = MT * K / 8;
        auto put = [&](int i, const u32x4& val) {
            const int m = (i * 8) / K, k = (i * 8) % K;
            *(lds_u32x4*)(xl + (size_t)m * xrow + (k / XG) * (2 * XG + 16) + (k % XG) * 2) = val;
        };
#pragma unroll
        for (int j = 0; j < XV; ++j) {
            const int i = threadIdx.x + j * blockDim.x;
            if (i < nvec) put(i, v[j]);
        }
        for (int i = threadIdx.x + XV * blockDim.x; i < nvec; i += blockDim.x) {
            const int m = (i * 8) / K, k = (i * 8) % K;
            u32x4 val = {0u, 0u, 0u, 0u};
            if (m < cnt) val = ld_global128(x + (size_t)row_of(m) * ldx + k);
            put(i, val);
        }
        if (Direct<F>::SUMS) {
            __syncthreads();
            const int per = K / 32;
            for (int i = threadIdx.x; i < MT * per; i += blockDim.x) {
                const int m = i / per, k = (i % per) * 32;
                const lds_u8* p = xl + (size_t)m * xrow + (k / XG) * (2 * XG + 16) + (k % XG) * 2;
                const XPairs a = load_x16(p, 0), b = load_x16(p, 16);
                float s = 0.f;
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    s += bf16_to_f32(a.v[t]);
                    s += bf16_to_f32(a.v[t] >> 16);
                }
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    s += bf16_to_f32(b.v[t]);
                    s += bf16_to_f32(b.v[t] >> 16);
                }
                xs[i] = s;
            }
        }
        __syncthreads();
    }
};

// One wave streams row groups handed out by next_group() (a row-group index,
// or a negative value when there are none left) of mv; row group rg is rows
// RW*rg .. RW*rg + RW - 1 (rows >= N idle), RW = 64 / G, lane group lane / G
// taking one row.  A row is P passes of G units, SP passes per ring slot, PF
// slots in flight; the ring always holds the next PF slots of work, refilled
// as soon as a slot is decoded.  Lane m < cnt of each group writes
// y[yrow * ldy + n] for activation row m.  between() runs once, after the
// first PF slots are in flight (the activation staging: a workgroup barrier
// inside, so every wave of the workgroup must call this function).
template <int F, int MT, int SP, int PF, class Next, class Between>
__device__ __forceinline__ void wave_stream_direct(const MatView& mv, int N, int K, const lds_u8* xl,
                                                   const lds_f32* xs, Next next_group, float* y, int64_t ldy,
                                                   int64_t yrow, int cnt, Between between) {
    using D = Direct<F>;
    constexpr int G = D::G, RW = 64 / G;
    const int lane = threadIdx.x & 63;
    const int grp = lane / G;
    const int U = D::units_per_row(K);
    const int P = (U + G - 1) / G;
    const int nseg = (P + SP - 1) / SP;
    const typename D::Lane L = D::lane_consts(lane);
    const int xrow_bytes = direct_xrow_bytes(F, K);
    const int xs_row = direct_xs_row(F, K);

    float gscale = 1.f;
    if (F == QG_NVFP4) {
        const uint8_t* gb = mv.gbytes;
        const uint32_t bits = (uint32_t)gb[0] | ((uint32_t)gb[1] << 8) | ((uint32_t)gb[2] << 16) |
                              ((uint32_t)gb[3] << 24);
        gscale = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(bits));
    }

    uint32_t R[PF][SP][D::REGS];
    int slot_g[PF], slot_s[PF];  // row group and segment held by each slot (group < 0: none)

    int cur_g = next_group(), cur_s = 0;
    // Issues the next segment of work into a slot; with no work left it loads
    // unit 0 of row 0 (every path issues the same loads).
    auto issue = [&](uint32_t (&r)[SP][D::REGS], int& sg, int& ss) {
        const bool live = cur_g >= 0;
        sg = cur_g;
        ss = cur_s;
        int n = 0;
        if (live) {
            n = RW * cur_g + grp;
            if (n >= N) n = RW * cur_g;  // idle lane group: duplicate the group's first row
        }
        const uint8_t* rc = mv.w0 + (size_t)n * mv.rb0;
        const uint8_t* rs = F == QG_NVFP4 ? mv.w1 + (size_t)n * mv.rb1 : nullptr;
#pragma unroll
        for (int p = 0; p < SP; ++p) {
            const int u = ((live ? cur_s : 0) * SP + p) * G + L.unit0;
            D::load(r[p], rc, rs, u < U ? u : 0);
        }
        if (live && ++cur_s == nseg) {
            cur_s = 0;
            cur_g = next_group();
        }
    };

    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.f;

    auto process = [&](const uint32_t (&r)[SP][D::REGS], int sg, int ss) {
#pragma unroll
        for (int p = 0; p < SP; ++p) {
            const int u = (ss * SP + p) * G + L.unit0;
            if (u < U) D::template decode<MT>(r[p], L, u, xl, xs, xrow_bytes, xs_row, acc);
        }
        if (ss == nseg - 1) {
            const int n = RW * sg + grp;
            float mine = 0.f;
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const float tot = group_sum<G>(acc[m]);
                if ((lane & (G - 1)) == m) mine = tot;
                acc[m] = 0.f;
            }
            if (F == QG_NVFP4) mine *= gscale;
            if ((lane & (G - 1)) < cnt && n < N) st_global_f32(y + yrow * ldy + n, mine);
        }
    };

#pragma unroll
    for (int sl = 0; sl < PF; ++sl) issue(R[sl], slot_g[sl], slot_s[sl]);
    between();
    while (slot_g[0] >= 0) {
#pragma unroll
        for (int sl = 0; sl < PF; ++sl) {
            if (slot_g[sl] >= 0) process(R[sl], slot_g[sl], slot_s[sl]);
            issue(R[sl], slot_g[sl], slot_s[sl]);
        }
    }
}

inline bool direct_eligible(int fmt, int K) {
    return fmt == QG_Q4_K || (fmt == QG_NVFP4 && K % 32 == 0);
}

}  // namespace qg
