// qg_mfma_kq.hip -- Q4_K, Q5_K, Q6_K, Q8_0, NVFP4 and row-scaled FP8 products
// for M >= 32 activation rows on the bf16 matrix cores
// (v_mfma_f32_32x32x16_bf16).
//
// Prefill must read each packed weight slab once for all rows rather than once
// per few rows ("Qwen3.8-27B on one Tenstorrent P150", section "3. Porting the
// 9B stack to 27B geometry": re-streaming the weights per 32 rows was the
// prefill bug).  A dequantized weight of the K-quant formats is not exact in
// bf16, but its integer code is: inside one sub-block w = s * v + t with v an
// integer that bf16 holds exactly and s, t fp32 per weight row and sub-block.
// The tile holds v, the matrix cores form D = sum v x over the sub-block in
// fp32, and the scale and the min enter in fp32 afterwards:
//   sum_k w x = s * D + t * X,   X = sum of the sub-block's activations.
//   Q4_K (32 values): v = q (0..15),            s = d sc, t = -dmin m
//   Q5_K (32 values): v = lo + 16 f (two planes: lo and 16 f), s, t as Q4_K
//   Q6_K (16 values): v = q - 32 = lo + 16 (hi - 2) (two planes), s = d sc, t = 0
//   Q8_0 (32 values): v = q (int8),             s = d, t = 0
// The codes enter with their own value, never with an offset, so a zero-point
// code contributes exactly zero and each sum's rounding error stays relative
// to sum |v x|.  Where v needs more than one exact bf16 part, the parts sit in
// two tile planes whose products with the same activations chain into one
// fp32 sum.
// NVFP4 and row-scaled FP8 need none of it: v = e2m1 * e4m3 or e4m3 (exact in
// bf16) over all of K, the products accumulate in place and the tensor or row
// scale multiplies the result.
//
// Tiling: a 256-thread workgroup computes a BM x BN tile of y, four waves own
// (BM/2) x (BN/2) quarters as 32x32 accumulators.  A K step is 64 values staged
// in one of two LDS buffers: activations, their sub-block sums per row (formats
// with mins), the tile values v, and per weight row the s (and t) of each
// sub-block.  Four threads decode each weight row.  The loads of the next steps
// run in a register ring.
#include "qg_mfma.h"

namespace qg {

struct KqArgs {
    const uint16_t* x;  // bf16 [M, K], row stride ldx
    int64_t ldx;
    const uint8_t* w;      // packed rows (NVFP4: the code plane)
    const uint8_t* w1;     // FP8: fp32 row scales; NVFP4: the E4M3 scale plane
    const uint8_t* gbytes; // NVFP4: the fp32 tensor scale (any alignment)
    int64_t rb;            // bytes per weight row
    int64_t rb1;           // NVFP4: scale bytes per row
    float* y;          // fp32 [M, N], row stride ldy
    int64_t ldy;
    int M, N, K;
};

// Per-format pieces.  Each provides:
//   SUB            values per sub-block (32 or 16); a step holds 64 / SUB
//   ROWSCALE       no per-sub-block terms: one scale per weight row (FP8) or
//                  per matrix (NVFP4), applied to the finished sums
//   PLANES         tile planes of exact parts of v (1 or 2)
//   MINS           the sub-blocks carry a min term t * X
//   Ring           registers one thread holds for one step
//   x_step(s)      offset of step s's first activation (uniform)
//   x_chunk(q)     offset of the step's 8-value chunk q (tile columns 8q..8q+7)
//   load(wrow, wrow1, s, part)        this thread's share of row wrow (wrow1: the
//                                     row in the second plane, NVFP4) for step s
//   decode(r, s, part, trow, plane, srow)
//                  tile values of the share into the LDS row trow (the second
//                  plane's row plane bytes further on), the s (then t) of the
//                  row's sub-blocks into srow
template <int F> struct KqFmt;

// Q4_K / Q5_K: step s is quarter g = s & 3 of super-block s >> 2: sub-blocks
// 2g (low nibbles of code bytes 32g..32g+31) and 2g + 1 (high nibbles).  Part
// p decodes code bytes 8p..8p+7 of the quarter: positions 8p..8p+7 of both.
// Q5_K puts 16 f (f the fifth bit) in the second plane.
template <int BB, int CODES, int HIGH> struct KqFmtK4 {
    static constexpr int SUB = 32;
    static constexpr bool ROWSCALE = false;
    static constexpr int PLANES = HIGH >= 0 ? 2 : 1;
    static constexpr bool MINS = true;
    struct Ring {
        u32x4 hdr;  // d, dmin, 12 scale bytes
        u32x2 q;    // 8 code bytes
        u32x2 f;    // Q5_K: the 8 fifth-bit bytes of the same positions
    };
    __device__ static int x_step(int s) { return 64 * s; }
    __device__ static int x_chunk(int q) { return 8 * q; }
    __device__ static Ring load(const uint8_t* wrow, const uint8_t*, int s, int part) {
        const uint8_t* blk = wrow + (size_t)(s >> 2) * BB;
        Ring r;
        r.hdr = ld_global128(blk);
        r.q = ld_global64(blk + CODES + 32 * (s & 3) + 8 * part);
        if constexpr (HIGH >= 0) r.f = ld_global64(blk + HIGH + 8 * part);
        return r;
    }
    __device__ static void decode(const Ring& r, int s, int part, lds_u8* trow, int plane, lds_f32* srow) {
        const int g = s & 3;
        const uint32_t l0 = r.q.x & 0x0F0F0F0Fu, l1 = r.q.y & 0x0F0F0F0Fu;
        const uint32_t h0 = (r.q.x >> 4) & 0x0F0F0F0Fu, h1 = (r.q.y >> 4) & 0x0F0F0F0Fu;
        *(lds_u32x4*)(trow + 16 * part) =
            u32x4{int_pair_bf16<0>(l0), int_pair_bf16<1>(l0), int_pair_bf16<0>(l1), int_pair_bf16<1>(l1)};
        *(lds_u32x4*)(trow + 64 + 16 * part) =
            u32x4{int_pair_bf16<0>(h0), int_pair_bf16<1>(h0), int_pair_bf16<0>(h1), int_pair_bf16<1>(h1)};
        if constexpr (HIGH >= 0) {
            // fifth bit of sub-block 2g + t at bit 2g + t of each H byte, as the
            // E4M3 code 0x10 (16 * 2^-9) or 0
            const uint32_t f0 = r.f.x >> (2 * g), f1 = r.f.y >> (2 * g);
            const uint32_t fl0 = (f0 << 4) & 0x10101010u, fl1 = (f1 << 4) & 0x10101010u;
            const uint32_t fh0 = (f0 << 3) & 0x10101010u, fh1 = (f1 << 3) & 0x10101010u;
            *(lds_u32x4*)(trow + plane + 16 * part) = u32x4{int_pair_bf16<0>(fl0), int_pair_bf16<1>(fl0),
                                                            int_pair_bf16<0>(fl1), int_pair_bf16<1>(fl1)};
            *(lds_u32x4*)(trow + plane + 64 + 16 * part) = u32x4{int_pair_bf16<0>(fh0), int_pair_bf16<1>(fh0),
                                                                 int_pair_bf16<0>(fh1), int_pair_bf16<1>(fh1)};
        }
        if (part < 2) {
            // 6-bit scale and min of sub-block jb = 2g + part (packing over
            // S[0..3], S[4..7], S[8..11]: jb < 4 whole in S[jb], S[jb + 4];
            // jb >= 4 low bits in S[jb + 4], top bits in S[jb - 4] and S[jb])
            const uint32_t S0 = r.hdr.y, S1 = r.hdr.z, S2 = r.hdr.w;
            const uint32_t o = 8u * (uint32_t)((2 * g + part) & 3);
            uint32_t sc, m;
            if (g < 2) {
                sc = __builtin_amdgcn_ubfe(S0, o, 6);
                m = __builtin_amdgcn_ubfe(S1, o, 6);
            } else {
                sc = __builtin_amdgcn_ubfe(S2, o, 4) | (__builtin_amdgcn_ubfe(S0, o + 6, 2) << 4);
                m = __builtin_amdgcn_ubfe(S2, o + 4, 4) | (__builtin_amdgcn_ubfe(S1, o + 6, 2) << 4);
            }
            const float d = f16_to_f32(r.hdr.x), dmin = f16_to_f32(r.hdr.x >> 16);
            srow[part] = d * (float)sc;
            srow[2 + part] = -(dmin * (float)m);
        }
    }
};
template <> struct KqFmt<QG_Q4_K> : KqFmtK4<144, 16, -1> {};
template <> struct KqFmt<QG_Q5_K> : KqFmtK4<176, 48, 16> {};  // fifth bits at [16, 48)

// Q8_0: step s is blocks 2s and 2s + 1 (34 bytes each: fp16 d, 32 int8 codes,
// 2-byte aligned).  Part p decodes codes 16 (p & 1) .. + 15 of block 2s + p / 2.
template <> struct KqFmt<QG_Q8_0> {
    static constexpr int SUB = 32;
    static constexpr bool ROWSCALE = false;
    static constexpr int PLANES = 1;
    static constexpr bool MINS = false;
    struct Ring {
        u32x4 q;     // 16 codes
        uint32_t d;  // fp16 d of the block
    };
    __device__ static int x_step(int s) { return 64 * s; }
    __device__ static int x_chunk(int q) { return 8 * q; }
    __device__ static Ring load(const uint8_t* wrow, const uint8_t*, int s, int part) {
        const uint8_t* blk = wrow + (size_t)(2 * s + (part >> 1)) * 34;
        Ring r;
        r.q = ld_global128_a2(blk + 2 + 16 * (part & 1));
        r.d = ld_global16(blk);
        return r;
    }
    __device__ static void decode(const Ring& r, int, int part, lds_u8* trow, int, lds_f32* srow) {
        // the signed codes, exact in bf16: (q + 128) - 128 with q + 128 the code
        // byte with its sign bit flipped, read unsigned.  (A sign-extending
        // bit-field extract converted to float was compiled into an unsigned
        // conversion of the sign-extended byte, which turns -1 into 2^32 - 1.)
        const uint32_t w[4] = {r.q.x ^ 0x80808080u, r.q.y ^ 0x80808080u, r.q.z ^ 0x80808080u,
                               r.q.w ^ 0x80808080u};
        uint32_t o[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            o[2 * e] = bf16_pair_from_exact((float)(w[e] & 0xFFu) - 128.f, (float)((w[e] >> 8) & 0xFFu) - 128.f);
            o[2 * e + 1] =
                bf16_pair_from_exact((float)((w[e] >> 16) & 0xFFu) - 128.f, (float)(w[e] >> 24) - 128.f);
        }
        *(lds_u32x4*)(trow + 32 * part) = u32x4{o[0], o[1], o[2], o[3]};
        *(lds_u32x4*)(trow + 32 * part + 16) = u32x4{o[4], o[5], o[6], o[7]};
        if ((part & 1) == 0) srow[part >> 1] = f16_to_f32(r.d);
    }
};

// Q6_K (210 bytes, 2-byte aligned): value 128 n + 32 j + l of a super-block
// (n < 2, j < 4, l < 32) has low bits in byte 64 n + l (j = 0, 2: low / high
// nibble) or 64 n + 32 + l (j = 1, 3), high bits 2j..2j+1 of byte 128 + 32 n
// + l, scale int8 at 192 + 8 n + 2 j + l / 16, d fp16 at 208.  Step s takes
// n = (s >> 1) & 1 and l in [16 h, 16 h + 16), h = s & 1: its 64 values are
// four sub-blocks of 16 (tile columns 16 j .. 16 j + 15 hold quadrant j), and
// every code byte of the super-block is read by exactly one step.  Part p
// decodes l = 16 h + 4 p .. + 3 of the four quadrants: the low nibbles into
// the first plane, 16 (hi - 2) into the second.
template <> struct KqFmt<QG_Q6_K> {
    static constexpr int SUB = 16;
    static constexpr bool ROWSCALE = false;
    static constexpr int PLANES = 2;
    static constexpr bool MINS = false;
    struct Ring {
        uint32_t qa, qb, qh;  // low-bit bytes (quadrants 0/2, 1/3) and high-bit bytes of 4 positions
        u32x2 sc;             // scales 8n .. 8n + 7
        uint32_t d;
    };
    __device__ static int x_step(int s) { return 256 * (s >> 2) + 128 * ((s >> 1) & 1) + 16 * (s & 1); }
    __device__ static int x_chunk(int q) { return 32 * (q >> 1) + 8 * (q & 1); }
    __device__ static Ring load(const uint8_t* wrow, const uint8_t*, int s, int part) {
        const uint8_t* blk = wrow + (size_t)(s >> 2) * 210;
        const int n = (s >> 1) & 1, l = 16 * (s & 1) + 4 * part;
        Ring r;
        r.qa = ld_global32_a2(blk + 64 * n + l);
        r.qb = ld_global32_a2(blk + 64 * n + 32 + l);
        r.qh = ld_global32_a2(blk + 128 + 32 * n + l);
        r.sc = ld_global64_a2(blk + 192 + 8 * n);
        r.d = ld_global16(blk + 208);
        return r;
    }
    __device__ static void decode(const Ring& r, int s, int part, lds_u8* trow, int plane, lds_f32* srow) {
        const uint32_t lo[4] = {r.qa & 0x0F0F0F0Fu, r.qb & 0x0F0F0F0Fu, (r.qa >> 4) & 0x0F0F0F0Fu,
                                (r.qb >> 4) & 0x0F0F0F0Fu};
        const uint32_t hi[4] = {q6_high_codes(r.qh & 0x03030303u), q6_high_codes((r.qh >> 2) & 0x03030303u),
                                q6_high_codes((r.qh >> 4) & 0x03030303u), q6_high_codes((r.qh >> 6) & 0x03030303u)};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            *(lds_u32x2*)(trow + 32 * j + 8 * part) = u32x2{int_pair_bf16<0>(lo[j]), int_pair_bf16<1>(lo[j])};
            *(lds_u32x2*)(trow + plane + 32 * j + 8 * part) = u32x2{int_pair_bf16<0>(hi[j]), int_pair_bf16<1>(hi[j])};
        }
        // this part writes s of quadrant j = part: scale byte 2 part + h of sc
        const int idx = 2 * part + (s & 1);
        const uint32_t word = (idx >> 2) ? r.sc.y : r.sc.x;
        const int sc = __builtin_amdgcn_sbfe((int)word, 8 * (idx & 3), 8);
        srow[part] = f16_to_f32(r.d) * (float)sc;
    }
};

// Row-scaled FP8: step s is codes 64s .. 64s + 63 of the row; part p converts
// codes 16p .. 16p + 15 to bf16 (exact).  The row scale is applied at the end.
template <> struct KqFmt<QG_FP8> {
    static constexpr int SUB = 64;
    static constexpr bool ROWSCALE = true;
    static constexpr int PLANES = 1;
    static constexpr bool MINS = false;
    struct Ring {
        u32x4 q;  // 16 codes
    };
    __device__ static int x_step(int s) { return 64 * s; }
    __device__ static int x_chunk(int q) { return 8 * q; }
    __device__ static Ring load(const uint8_t* wrow, const uint8_t*, int s, int part) {
        return Ring{ld_global128(wrow + 64 * (size_t)s + 16 * part)};
    }
    // the row's scale multiplies the finished sums
    __device__ static float out_scale(const KqArgs& a, int n) {
        return *(const QG_GLOBAL float*)(uintptr_t)(a.w1 + 4 * (size_t)n);
    }
    __device__ static void decode(const Ring& r, int, int part, lds_u8* trow, int, lds_f32*) {
        const uint32_t c0 = r.q.x, c1 = r.q.y, c2 = r.q.z, c3 = r.q.w;
        *(lds_u32x4*)(trow + 32 * part) = u32x4{e4m3x2_to_bf16x2<0>(c0), e4m3x2_to_bf16x2<1>(c0),
                                                e4m3x2_to_bf16x2<0>(c1), e4m3x2_to_bf16x2<1>(c1)};
        *(lds_u32x4*)(trow + 32 * part + 16) = u32x4{e4m3x2_to_bf16x2<0>(c2), e4m3x2_to_bf16x2<1>(c2),
                                                     e4m3x2_to_bf16x2<0>(c3), e4m3x2_to_bf16x2<1>(c3)};
    }
};

// NVFP4 (K a multiple of 64): step s is blocks 4s .. 4s + 3 of the row; part p
// decodes block 4s + p (8 code bytes, one E4M3 scale) to bf16(e2m1 * scale),
// exact (at most 6 significant bits).  The tensor scale g multiplies the
// finished sums.
template <> struct KqFmt<QG_NVFP4> {
    static constexpr int SUB = 64;
    static constexpr bool ROWSCALE = true;
    static constexpr int PLANES = 1;
    static constexpr bool MINS = false;
    struct Ring {
        u32x2 q;      // 16 codes
        uint32_t sc;  // the scale bytes of blocks 4s .. 4s + 3
    };
    __device__ static int x_step(int s) { return 64 * s; }
    __device__ static int x_chunk(int q) { return 8 * q; }
    __device__ static Ring load(const uint8_t* wrow, const uint8_t* wrow1, int s, int part) {
        Ring r;
        r.q = ld_global64(wrow + 32 * (size_t)s + 8 * part);
        r.sc = *(const QG_GLOBAL uint32_t*)(uintptr_t)(wrow1 + 4 * (size_t)s);
        return r;
    }
    __device__ static void decode(const Ring& r, int, int part, lds_u8* trow, int, lds_f32*) {
        uint32_t o[8];
        decode_nvfp4_block_bf16(r.q.x, r.q.y, __builtin_amdgcn_cvt_f32_fp8(r.sc >> (8 * part), 0), o);
        *(lds_u32x4*)(trow + 32 * part) = u32x4{o[0], o[1], o[2], o[3]};
        *(lds_u32x4*)(trow + 32 * part + 16) = u32x4{o[4], o[5], o[6], o[7]};
    }
    __device__ static float out_scale(const KqArgs& a, int) {
        const uint8_t* gb = a.gbytes;
        const uint32_t bits = (uint32_t)gb[0] | ((uint32_t)gb[1] << 8) | ((uint32_t)gb[2] << 16) |
                              ((uint32_t)gb[3] << 24);
        return __builtin_bit_cast(float, bits);
    }
};

// Stream-K: the (tile, K step) iterations of the whole product, tiles row
// tile major (t = row tile * ntiles + column tile), are dealt to the grid in
// equal contiguous ranges, so every workgroup gets the same number of products
// whatever the tile count.  A tile whose steps fall to several workgroups is
// finished by the last of them to arrive: each writes its partial sums to its
// slot (two per workgroup: the first and the last tile of its range), counts
// itself in at the tile's counter, and the last one adds the parts in
// workgroup order and stores the tile.  Nothing waits on another workgroup.
struct KqSplit {
    int32_t* counters;  // per tile, zero on entry
    float* partials;    // 2 slots of BM * BN floats per workgroup
    int tiles, ntiles;  // all tiles; column tiles
};

// D: K steps of loads in flight in the register ring (an even number).
// BN: 64, or 128 for the formats without per-sub-block terms.
// G: grouped product, row tile blockIdx.y of g's list (rows through the
// bucketing permutation, the weights of the tile's expert).
// SK: stream-K over sp (dense products only).
template <int F, int BM, int BN, int D, bool G, bool SK = false>
__global__ __launch_bounds__(kMfmaThreads, 2) void k_mfma_kq(const KqArgs a_in, const KqGroup g, const KqSplit sp) {
    using Fmt = KqFmt<F>;
    constexpr int TPR = kMfmaThreads / BN;  // threads per weight row (4 or 2)
    constexpr int QPT = 4 / TPR;            // quarters of a row's step decoded per thread
    static_assert(TPR * QPT == 4 && (BN == 64 || Fmt::ROWSCALE), "tile shape");
    constexpr int NSUB = kMfmaKStep / Fmt::SUB;  // sub-blocks per step
    constexpr int KPS = Fmt::SUB / 16;           // 32x32x16 products per sub-block
    constexpr int CPS = Fmt::SUB / 8;            // 8-value chunks per sub-block
    constexpr int FM = BM / 64, FN = BN / 64;    // 32x32 fragments per wave
    constexpr int XCH = BM * 8 / kMfmaThreads;   // 16-byte activation chunks per thread per step
    constexpr int SROW = Fmt::ROWSCALE ? 0 : NSUB * (Fmt::MINS ? 2 : 1);  // floats per weight row: s, then t
    constexpr int PLANE = BN * kMfmaRowBytes;     // bytes of one tile plane
    constexpr int TILE_X = BM * kMfmaRowBytes;    // activations (bf16, padded rows)
    constexpr int TILE_W = Fmt::PLANES * PLANE;   // tile values v (bf16), one or two planes
    constexpr int TILE_S = BN * 4 * SROW;         // per weight row: s of each sub-block, then t
    constexpr int TILE_XS = Fmt::MINS ? NSUB * BM * 4 : 0;  // per sub-block and activation row: X
    constexpr int BUF = TILE_X + TILE_W + TILE_S + TILE_XS;
    __shared__ __attribute__((aligned(16))) uint8_t smem_generic[2 * BUF];
    lds_u8* smem = (lds_u8*)smem_generic;

    KqArgs a = a_in;
    int m0 = blockIdx.y * BM, M = a.M;
    int nt = blockIdx.x;  // column tile
    const int32_t* prow = nullptr;  // grouped: original index of the tile's row i at prow[i]
    if constexpr (G) {
        // Workgroups are dealt to the 8 XCDs in turn (workgroup i on XCD
        // i % 8); each XCD takes a contiguous band of the listed (row tile,
        // column tile) items, row tile major, so the tiles of one expert -- its
        // weights and its activation rows -- stay in one XCD's L2 instead of
        // being fetched by all of them.  Only the placement changes.
        constexpr int kXcds = 8;
        const int nx = gridDim.x;
        const int items = g.ws[g.count] * nx;
        const int per_xcd = (items + kXcds - 1) / kXcds;
        const int lin = blockIdx.y * nx + blockIdx.x;
        const int it = (lin % kXcds) * per_xcd + lin / kXcds;
        if (it >= items || lin / kXcds >= per_xcd) return;  // uniform: past the listed tiles
        const int t = it / nx;
        nt = it - t * nx;
        const int p = g.ws[g.list + 2 * t], q = g.ws[g.list + 2 * t + 1];
        const int e = g.ws[4 + q];
        const int r1 = g.ws[4 + g.S + q + 1];
        a.w += (size_t)e * g.es0;
        if (a.w1) a.w1 += (size_t)e * g.es1;
        if (a.gbytes) a.gbytes += 4 * (size_t)e;
        prow = g.ws + 5 + 2 * g.S + p;
        m0 = 0;
        M = min(BM, r1 - p);
    }
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    int n0 = nt * BN;
    const int wm = (wid >> 1) * (BM / 2), wn = (wid & 1) * (BN / 2);
    const int N = a.N;
    const int nsteps = a.K / kMfmaKStep;  // K is a multiple of 64

    // Register ring: activation chunks and this thread's weight share.
    u32x4 xr[D][XCH];
    typename Fmt::Ring wring[D][QPT];
    const int wrow_i = tid / TPR, part0 = (tid % TPR) * QPT;  // weight tile row, first quarter decoded by this thread

    // Per-thread row pointers, fixed for the whole K loop.  Rows past M or N
    // read row M - 1 or row 0 instead: such rows feed only outputs that are
    // never written, so no select is needed.
    const uint16_t* xp[XCH];
    const uint8_t* wrow;
    const uint8_t* wrow1;
    auto setup = [&]() {
#pragma unroll
        for (int c = 0; c < XCH; ++c) {
            const int i = tid + c * kMfmaThreads;
            const int r = min(m0 + (i >> 3), M - 1);
            const int64_t xrow = G ? prow[r] / g.xdiv : r;
            xp[c] = a.x + (size_t)xrow * a.ldx + Fmt::x_chunk(i & 7);
        }
        const size_t wrow_n = (size_t)(n0 + wrow_i < N ? n0 + wrow_i : 0);
        wrow = a.w + wrow_n * a.rb;
        wrow1 = a.w1 ? a.w1 + wrow_n * a.rb1 : nullptr;
    };

    // Loads without branches: a load under a branch makes the compiler wait
    // for every outstanding load.
    auto load = [&](int s, auto stage_tag) {
        constexpr int j = decltype(stage_tag)::value;
        const int k0 = Fmt::x_step(s);
#pragma unroll
        for (int c = 0; c < XCH; ++c) xr[j][c] = ld_global128(xp[c] + k0);
#pragma unroll
        for (int q = 0; q < QPT; ++q) wring[j][q] = Fmt::load(wrow, wrow1, s, part0 + q);
    };
    auto store = [&](int buf, int s, auto stage_tag) {
        constexpr int j = decltype(stage_tag)::value;
        lds_u8* tx = smem + buf * BUF;
        lds_u8* tw = tx + TILE_X;
        lds_f32* ts = (lds_f32*)(tw + TILE_W);
        lds_f32* txs = (lds_f32*)((lds_u8*)ts + TILE_S);
#pragma unroll
        for (int c = 0; c < XCH; ++c) {
            const int i = tid + c * kMfmaThreads;
            const int r = i >> 3, q = i & 7;
            *(lds_u32x4*)(tx + r * kMfmaRowBytes + q * 16) = xr[j][c];
            if constexpr (!Fmt::MINS) continue;
            // sum of this chunk's 8 values (pairs dotted with (1, 1)), then over
            // the chunks of the sub-block: lanes xor 1 (and xor 2) of a quad
            // (element copies first: a bit cast of a vector element reads element 0)
            const uint32_t e0 = xr[j][c].x, e1 = xr[j][c].y, e2 = xr[j][c].z, e3 = xr[j][c].w;
            float p = dot2bf(e0, kBf16Ones, 0.f);
            p = dot2bf(e1, kBf16Ones, p);
            p = dot2bf(e2, kBf16Ones, p);
            p = dot2bf(e3, kBf16Ones, p);
            p += __builtin_amdgcn_update_dpp(0.f, p, kDppQuadXor1, 0xF, 0xF, false);
            if constexpr (CPS == 4) p += __builtin_amdgcn_update_dpp(0.f, p, kDppQuadXor2, 0xF, 0xF, false);
            if ((q & (CPS - 1)) == 0) txs[(q / CPS) * BM + r] = p;
        }
#pragma unroll
        for (int q = 0; q < QPT; ++q)
            Fmt::decode(wring[j][q], s, part0 + q, tw + wrow_i * kMfmaRowBytes, PLANE, ts + wrow_i * SROW);
    };

    // One fp32 accumulator per fragment takes both terms: t * X from the
    // matrix cores (formats with mins), s * D from the vector unit.  (At most 256 registers per
    // lane, two waves per SIMD: the compiler then keeps matrix-core results in
    // ordinary VGPRs, which the vector unit can read without copies.)
    f32x16 acc[FM][FN];

    const int frow = lane & 31, fcol = (lane >> 5) * 16, half = lane >> 5;
    auto mma = [&](int buf) {
        const lds_u8* tx = smem + buf * BUF;
        const lds_u8* tw = tx + TILE_X;
        const lds_f32* ts = (const lds_f32*)(tw + TILE_W);
        const lds_f32* txs = (const lds_f32*)((const lds_u8*)ts + TILE_S);
        if constexpr (Fmt::ROWSCALE) {
            // the whole step accumulates in place
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                bf16x8_t fa[FM], fb[FN];
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    fa[i] = __builtin_bit_cast(
                        bf16x8_t, lds_ld128(tx + (wm + 32 * i + frow) * kMfmaRowBytes + kk * 32 + fcol));
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    fb[j] = __builtin_bit_cast(
                        bf16x8_t, lds_ld128(tw + (wn + 32 * j + frow) * kMfmaRowBytes + kk * 32 + fcol));
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
            }
            return;
        }
        if constexpr (Fmt::MINS) {
            // t * X of two sub-blocks per 32x32x2 fp32 product:
            // A[m][k] = X(row m, sub-block 2p + k), lane l holds m = l % 32, k = l / 32;
            // B[k][n] = t(row n, sub-block 2p + k), same lane mapping.
#pragma unroll
            for (int pp = 0; pp < NSUB / 2; ++pp) {
                float xa[FM], tb[FN];
#pragma unroll
                for (int i = 0; i < FM; ++i) xa[i] = txs[(2 * pp + half) * BM + wm + 32 * i + frow];
#pragma unroll
                for (int j = 0; j < FN; ++j) tb[j] = ts[(wn + 32 * j + frow) * SROW + NSUB + 2 * pp + half];
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(xa[i], tb[j], acc[i][j], 0, 0, 0);
            }
        }
        float sv[FN][NSUB];
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int sb = 0; sb < NSUB; ++sb) sv[j][sb] = ts[(wn + 32 * j + frow) * SROW + sb];
        constexpr int PL = Fmt::PLANES;
#pragma unroll
        for (int sb = 0; sb < NSUB; ++sb) {
            bf16x8_t fa[FM][KPS], fb[FN][PL][KPS];
#pragma unroll
            for (int h = 0; h < KPS; ++h) {
                const int kk = KPS * sb + h;
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    fa[i][h] = __builtin_bit_cast(
                        bf16x8_t, lds_ld128(tx + (wm + 32 * i + frow) * kMfmaRowBytes + kk * 32 + fcol));
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int pl = 0; pl < PL; ++pl)
                        fb[j][pl][h] = __builtin_bit_cast(
                            bf16x8_t,
                            lds_ld128(tw + pl * PLANE + (wn + 32 * j + frow) * kMfmaRowBytes + kk * 32 + fcol));
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    // D = sum v x over the sub-block (the planes' products chained
                    // in one fp32 sum), then acc += s * D
                    f32x16 dsum = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i][0], fb[j][0][0], f32x16{}, 0, 0, 0);
#pragma unroll
                    for (int pl = 0; pl < PL; ++pl)
#pragma unroll
                        for (int h = 0; h < KPS; ++h)
                            if (pl > 0 || h > 0)
                                dsum = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i][h], fb[j][pl][h], dsum, 0, 0, 0);
                    const float s = sv[j][sb];
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][j][r] = fmaf(s, dsum[r], acc[i][j][r]);
                }
            // with four sub-blocks, one sub-block's products live at a time (registers)
            if constexpr (NSUB > 2) __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Steps [sb, se) of the current tile into acc.  The LDS buffers alternate
    // from buffer 0 at step sb; the last step ends with a barrier, so the next
    // range may restage at once.
    auto run = [&](int sb, int se) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};
        // prologue: steps sb .. sb+D-1 in flight, step sb in LDS, step sb+D into the freed stage
        static_for<D>([&](auto j) { load(min(sb + (int)decltype(j)::value, se - 1), j); });
        store(0, sb, std::integral_constant<int, 0>{});
        load(min(sb + D, se - 1), std::integral_constant<int, 0>{});
        __syncthreads();
        // main loop over whole groups of D steps: no branches, so the compiler
        // waits only for the loads each store needs
        int s0 = sb;
        for (; s0 + D < se; s0 += D) {
            static_for<D>([&](auto jt) {
                constexpr int j = decltype(jt)::value;
                constexpr int nj = (j + 1) % D;
                const int s = s0 + j;
                // (no scheduling fences between the three: the compiler interleaves
                // the next step's decode and loads with this step's products, 2-6 %
                // faster than keeping them apart)
                mma(j & 1);  // s0 - sb is a multiple of D (even), so (s - sb) & 1 == j & 1
                store((j + 1) & 1, s + 1, std::integral_constant<int, nj>{});
                load(min(s + 1 + D, se - 1), std::integral_constant<int, nj>{});  // (past the end: a harmless reload)
                __syncthreads();
            });
        }
        // the last (up to D) steps
        static_for<D>([&](auto jt) {
            constexpr int j = decltype(jt)::value;
            constexpr int nj = (j + 1) % D;
            const int s = s0 + j;
            if (s < se) {
                mma(j & 1);
                if (s + 1 < se) store((j + 1) & 1, s + 1, std::integral_constant<int, nj>{});
                __syncthreads();
            }
        });
    };

    auto store_y = [&](const f32x16 (&v)[FM][FN]) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n = n0 + wn + 32 * j + (lane & 31);
            float rs = 1.f;
            if constexpr (Fmt::ROWSCALE) rs = Fmt::out_scale(a, n < N ? n : 0);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    if (m < M && n < N) {
                        const int64_t yrow = G ? prow[m] : m;
                        st_global_f32(a.y + (size_t)yrow * a.ldy + n,
                                      Fmt::ROWSCALE ? v[i][j][r] * rs : v[i][j][r]);
                    }
                }
        }
    };

    if constexpr (!SK) {
        setup();
        run(0, nsteps);
        store_y(acc);
    } else {
        __shared__ int last_part;
        const int64_t iters = (int64_t)sp.tiles * nsteps;
        const int grid = (int)gridDim.x;
        auto begin = [&](int b) { return (int64_t)b * iters / grid; };
        // logical workgroup: workgroups are dealt to the 8 XCDs in turn, and
        // each XCD takes a contiguous band of logical ranges, so that the row
        // tiles of one weight column and the parts of one split tile mostly
        // share an L2 (placement only: nothing below depends on it)
        constexpr int kXcds = 8;
        const int per_xcd = grid / kXcds;  // the grid is a multiple of 8
        const int me = ((int)blockIdx.x % kXcds) * per_xcd + (int)blockIdx.x / kXcds;
        const int64_t it0 = begin(me), it1 = begin(me + 1);
        for (int64_t it = it0; it < it1;) {
            const int t = (int)(it / nsteps);
            const int64_t tb = (int64_t)t * nsteps;
            const int sb = (int)(it - tb), se = (int)min<int64_t>(nsteps, it1 - tb);
            const int mt = t / sp.ntiles;  // row tile major, as the plain launch
            nt = t - mt * sp.ntiles;
            m0 = mt * BM;
            n0 = nt * BN;
            setup();
            run(sb, se);
            it = tb + se;
            if (sb == 0 && se == nsteps) {
                store_y(acc);
                continue;
            }
            // workgroups b_lo .. b_hi hold the parts of tile t (first and last
            // whose ranges meet [tb, tb + nsteps))
            int b_lo = (int)(tb * grid / iters), b_hi = (int)((tb + nsteps) * grid / iters);
            while (b_lo + 1 < grid && begin(b_lo + 1) <= tb) ++b_lo;
            while (b_lo > 0 && begin(b_lo) > tb) --b_lo;
            while (b_hi > 0 && begin(b_hi) >= tb + nsteps) --b_hi;
            while (b_hi + 1 < grid && begin(b_hi + 1) < tb + nsteps) ++b_hi;
            auto slot = [&](int b) {
                const int sl = (int)(begin(b) / nsteps) == t ? 0 : 1;  // 0: the first tile of b's range
                return sp.partials + ((size_t)b * 2 + sl) * (BM * BN) + ((size_t)wid * FM * FN * 16) * 64 + lane;
            };
            // The partials go through agent-scope atomic stores and loads, which
            // write through and read at the device's coherence point one access
            // at a time; every store has completed (s_waitcnt 0) before this part
            // counts in, and the last part reads them only after its count.  No
            // cache-wide fence: a release writes back, and an acquire invalidates,
            // the XCD's whole L2, which holds the activations every tile rereads
            // (each cost more than the balance gained).
            float* mine = slot(me);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        __hip_atomic_store(mine + (size_t)(((i * FN + j) * 16 + r) * 64), acc[i][j][r],
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores are complete
            __syncthreads();
            int parts = 0;  // workgroups with a non-empty range among b_lo .. b_hi
            for (int b = b_lo; b <= b_hi; ++b) parts += begin(b + 1) > begin(b);
            if (tid == 0) {
                const int before = __hip_atomic_fetch_add(sp.counters + t, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                last_part = before == parts - 1;
            }
            __syncthreads();
            if (!last_part) continue;
            // every part from its slot (this workgroup's too), in workgroup order
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};
            for (int b = b_lo; b <= b_hi; ++b) {
                if (begin(b + 1) == begin(b)) continue;  // (no part)
                const float* p = slot(b);
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            acc[i][j][r] += __hip_atomic_load(p + (size_t)(((i * FN + j) * 16 + r) * 64),
                                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            store_y(acc);
        }
    }
}

// Tile shape: the largest whose tile count still gives every CU work: 128 x
// 128 (formats without per-sub-block terms, two tiles per CU), 128 x 64, else
// 64 x 64.  (With per-sub-block terms a 128 x 128 tile needs more than the 256
// registers per lane that keep the matrix-core results in VGPRs.)
template <int F>
static hipError_t launch_kq(const KqArgs& a, hipStream_t st) {
    const long cus = num_cus();
    auto tiles = [&](int bm, int bn) { return (long)((a.N + bn - 1) / bn) * ((a.M + bm - 1) / bm); };
    const KqGroup none{};
    const KqSplit plain{};
    // (column tile fastest: the row tiles of one weight column land on one
    // XCD whenever the column tile count is a multiple of 8 -- measured 3-7 %
    // faster than bands of row tiles per XCD)
    if (KqFmt<F>::ROWSCALE && tiles(128, 128) >= 2 * cus) {
        dim3 grid((a.N + 127) / 128, (a.M + 127) / 128);
        hipLaunchKernelGGL((k_mfma_kq<F, 128, KqFmt<F>::ROWSCALE ? 128 : 64, 2, false>), grid, dim3(kMfmaThreads), 0,
                           st, a, none, plain);
    } else if (tiles(128, 64) >= cus) {
        dim3 grid((a.N + 63) / 64, (a.M + 127) / 128);
        hipLaunchKernelGGL((k_mfma_kq<F, 128, 64, 2, false>), grid, dim3(kMfmaThreads), 0, st, a, none, plain);
    } else {
        dim3 grid((a.N + 63) / 64, (a.M + 63) / 64);
        hipLaunchKernelGGL((k_mfma_kq<F, 64, 64, 4, false>), grid, dim3(kMfmaThreads), 0, st, a, none, plain);
    }
    return hipGetLastError();
}

// Stream-K plan of a dense product: the tile shape the plain launch would
// take at two workgroups per CU, one workgroup per resident slot.  Taken when
// the tiles would leave slots idle but number at least half of them (a tile
// is then shared by at most three workgroups): the 5120-row down projections
// at 512 rows, 320 tiles for 512 slots, measured 11 % (NVFP4) and 22 % (Q6_K)
// faster.  With more tiles than slots the plain launch measured faster
// (1.06-2.1 rounds: the partial sums' traffic and the split tiles' second
// pipeline fill cost more than the balance gains).
struct SkPlan {
    int bm, bn, tiles, ntiles, grid;
    size_t counter_bytes, bytes;
};

template <int F>
static bool sk_plan(int N, int M, SkPlan* p) {
    const long slots = 2L * num_cus() / 8 * 8;  // a multiple of the 8 XCDs
    if (slots < 8) return false;
    auto tiles = [&](int bm, int bn) { return (long)((N + bn - 1) / bn) * ((M + bm - 1) / bm); };
    const int bn = KqFmt<F>::ROWSCALE && tiles(128, 128) >= slots / 2 ? 128 : 64;
    const long t = tiles(128, bn);
    if (t < slots / 2 || t >= slots) return false;
    p->bm = 128;
    p->bn = bn;
    p->tiles = (int)t;
    p->ntiles = (N + bn - 1) / bn;
    p->grid = (int)slots;
    p->counter_bytes = ((size_t)t * 4 + 255) / 256 * 256;
    p->bytes = p->counter_bytes + (size_t)p->grid * 2 * 128 * bn * sizeof(float);
    return true;
}

__global__ void k_zero_i32(int32_t* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

template <int F>
static hipError_t launch_kq_sk(const KqArgs& a, const SkPlan& pl, void* ws, hipStream_t st) {
    KqSplit sp;
    sp.counters = (int32_t*)ws;
    sp.partials = (float*)((uint8_t*)ws + pl.counter_bytes);
    sp.tiles = pl.tiles;
    sp.ntiles = pl.ntiles;
    // the counters start at zero in every call (a fill kernel, not a memset:
    // the call may be captured into a graph)
    hipLaunchKernelGGL(k_zero_i32, dim3((pl.tiles + 255) / 256), dim3(256), 0, st, sp.counters, pl.tiles);
    const KqGroup none{};
    if constexpr (KqFmt<F>::ROWSCALE) {
        if (pl.bn == 128) {
            hipLaunchKernelGGL((k_mfma_kq<F, 128, 128, 2, false, true>), dim3(pl.grid), dim3(kMfmaThreads), 0, st, a,
                               none, sp);
            return hipGetLastError();
        }
    }
        hipLaunchKernelGGL((k_mfma_kq<F, 128, 64, 2, false, true>), dim3(pl.grid), dim3(kMfmaThreads), 0, st, a, none,
                           sp);
    return hipGetLastError();
}

// Grouped: one row of workgroups per possible list entry (g.cap), rounded up
// so that the grid holds a whole number of rounds over the 8 XCDs (every
// item of the kernel's XCD bands then has a workgroup); those past the listed
// items exit at once.
template <int F>
static hipError_t launch_kq_grouped(const KqArgs& a, const KqGroup& g, int bm, hipStream_t st) {
    if (g.cap <= 0) return hipSuccess;
    const long nx = (a.N + 63) / 64;
    const long total = (nx * g.cap + 7) / 8 * 8;
    dim3 grid((unsigned)nx, (unsigned)((total + nx - 1) / nx));
    if (bm == 128)
        hipLaunchKernelGGL((k_mfma_kq<F, 128, 64, 2, true>), grid, dim3(kMfmaThreads), 0, st, a, g, KqSplit{});
    else
        hipLaunchKernelGGL((k_mfma_kq<F, 64, 64, 4, true>), grid, dim3(kMfmaThreads), 0, st, a, g, KqSplit{});
    return hipGetLastError();
}

bool mfma_kquant_supported(int fmt, int K) {
    switch (fmt) {
        case QG_Q4_K:
        case QG_Q5_K:
        case QG_Q6_K:                              // K is a multiple of 256
        case QG_FP8: return true;                  // K is a multiple of 64
        case QG_NVFP4: return K % kMfmaKStep == 0;  // whole 64-value steps
        case QG_Q8_0: return K % kMfmaKStep == 0;  // whole 64-value steps
        default: return false;
    }
}

// Bytes per weight row in the format's first plane (and, for NVFP4, the second).
static bool kq_row_bytes(int fmt, int K, KqArgs& a) {
    switch (fmt) {
        case QG_Q4_K: a.rb = (int64_t)(K / 256) * 144; return true;
        case QG_Q5_K: a.rb = (int64_t)(K / 256) * 176; return true;
        case QG_Q6_K: a.rb = (int64_t)(K / 256) * 210; return true;
        case QG_Q8_0: a.rb = (int64_t)(K / 32) * 34; return true;
        case QG_FP8: a.rb = K; return true;
        case QG_NVFP4: a.rb = K / 2; a.rb1 = K / 16; return true;
        default: return false;
    }
}

hipError_t launch_mfma_kquant(int fmt, const uint8_t* w, const uint8_t* w1, const uint8_t* gbytes, int N, int K,
                              const uint16_t* x, int64_t ldx, int M, float* y, int64_t ldy, hipStream_t st) {
    KqArgs a = {x, ldx, w, w1, gbytes, 0, 0, y, ldy, M, N, K};
    if (!kq_row_bytes(fmt, K, a)) return hipErrorInvalidValue;
    switch (fmt) {
        case QG_Q4_K: return launch_kq<QG_Q4_K>(a, st);
        case QG_Q5_K: return launch_kq<QG_Q5_K>(a, st);
        case QG_Q6_K: return launch_kq<QG_Q6_K>(a, st);
        case QG_Q8_0: return launch_kq<QG_Q8_0>(a, st);
        case QG_FP8: return launch_kq<QG_FP8>(a, st);
        default: return launch_kq<QG_NVFP4>(a, st);
    }
}

static bool sk_plan_fmt(int fmt, int N, int M, SkPlan* p) {
    switch (fmt) {
        case QG_Q4_K: return sk_plan<QG_Q4_K>(N, M, p);
        case QG_Q5_K: return sk_plan<QG_Q5_K>(N, M, p);
        case QG_Q6_K: return sk_plan<QG_Q6_K>(N, M, p);
        case QG_Q8_0: return sk_plan<QG_Q8_0>(N, M, p);
        case QG_FP8: return sk_plan<QG_FP8>(N, M, p);
        case QG_NVFP4: return sk_plan<QG_NVFP4>(N, M, p);
        default: return false;
    }
}

size_t mfma_streamk_bytes(int fmt, int N, int K, int M) {
    SkPlan pl;
    if (M < kMfmaMinRows || !mfma_kquant_supported(fmt, K) || !sk_plan_fmt(fmt, N, M, &pl)) return 0;
    return pl.bytes;
}

hipError_t launch_mfma_kquant_streamk(int fmt, const uint8_t* w, const uint8_t* w1, const uint8_t* gbytes, int N,
                                      int K, const uint16_t* x, int64_t ldx, int M, float* y, int64_t ldy, void* ws,
                                      size_t ws_bytes, hipStream_t st) {
    SkPlan pl;
    if (!sk_plan_fmt(fmt, N, M, &pl))
        return launch_mfma_kquant(fmt, w, w1, gbytes, N, K, x, ldx, M, y, ldy, st);
    if (!ws || ws_bytes < pl.bytes) return hipErrorInvalidValue;
    KqArgs a = {x, ldx, w, w1, gbytes, 0, 0, y, ldy, M, N, K};
    if (!kq_row_bytes(fmt, K, a)) return hipErrorInvalidValue;
    switch (fmt) {
        case QG_Q4_K: return launch_kq_sk<QG_Q4_K>(a, pl, ws, st);
        case QG_Q5_K: return launch_kq_sk<QG_Q5_K>(a, pl, ws, st);
        case QG_Q6_K: return launch_kq_sk<QG_Q6_K>(a, pl, ws, st);
        case QG_Q8_0: return launch_kq_sk<QG_Q8_0>(a, pl, ws, st);
        case QG_FP8: return launch_kq_sk<QG_FP8>(a, pl, ws, st);
        default: return launch_kq_sk<QG_NVFP4>(a, pl, ws, st);
    }
}

hipError_t launch_mfma_kquant_grouped(int fmt, const uint8_t* w, const uint8_t* w1, const uint8_t* gbytes, int N,
                                      int K, const uint16_t* x, int64_t ldx, float* y, int64_t ldy, const KqGroup& g,
                                      int bm, hipStream_t st) {
    KqArgs a = {x, ldx, w, w1, gbytes, 0, 0, y, ldy, 0, N, K};
    if (!kq_row_bytes(fmt, K, a)) return hipErrorInvalidValue;
    switch (fmt) {
        case QG_Q4_K: return launch_kq_grouped<QG_Q4_K>(a, g, bm, st);
        case QG_Q5_K: return launch_kq_grouped<QG_Q5_K>(a, g, bm, st);
        case QG_Q6_K: return launch_kq_grouped<QG_Q6_K>(a, g, bm, st);
        case QG_Q8_0: return launch_kq_grouped<QG_Q8_0>(a, g, bm, st);
        case QG_FP8: return launch_kq_grouped<QG_FP8>(a, g, bm, st);
        default: return launch_kq_grouped<QG_NVFP4>(a, g, bm, st);
    }
}

}  // namespace qg
