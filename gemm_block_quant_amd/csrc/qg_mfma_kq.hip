// qg_mfma_kq.hip -- Q4_K and Q5_K products for M >= 32 activation rows on the
// bf16 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// Prefill must read each packed weight slab once for all rows rather than once
// per few rows ("Qwen3.8-27B on one Tenstorrent P150", section "3. Porting the
// 9B stack to 27B geometry": re-streaming the weights per 32 rows was the
// prefill bug).  A dequantized K-quant weight d*sc*q - dmin*m is not exact in
// bf16, but its code is: the tile holds bf16(128 + q) (q <= 31, exact), the
// matrix cores form D = sum (128 + q) x over each 32-value sub-block in fp32,
// and the sub-block's scale and min enter in fp32 afterwards:
//   sum_k w x = s * D + t * X,  s = d * sc,  t = -(128 s + dmin * m),
// X = sum of the sub-block's 32 activations (the factorisation of the decode
// path, applied per 32 x 32 output block).
//
// Tiling as the NVFP4 tile kernel: a 256-thread workgroup computes a BM x BN
// tile of y, four waves own (BM/2) x (BN/2) quarters as 32x32 accumulators; a
// K step is 64 values (two sub-blocks, one quarter of a super-block) staged in
// one of two LDS buffers: activations, their two sub-block sums per row, the
// decoded codes, and per weight row (s, t) of both sub-blocks.  The loads of the
// next steps run in a register ring several steps ahead.
#include "qg_mfma.h"

namespace qg {


struct KqArgs {
    const uint16_t* x;  // bf16 [M, K], row stride ldx
    int64_t ldx;
    const uint8_t* w;  // packed rows of K/256 super-blocks
    int64_t rb;        // bytes per weight row
    float* y;          // fp32 [M, N], row stride ldy
    int64_t ldy;
    int M, N, K;
};

template <int F> struct KqGeom;
template <> struct KqGeom<QG_Q4_K> {
    static constexpr int BB = 144, CODES = 16, HIGH = -1;
};
template <> struct KqGeom<QG_Q5_K> {
    static constexpr int BB = 176, CODES = 48, HIGH = 16;  // fifth bits at [16, 48)
};

// D: K steps of loads in flight in the register ring (an even number).
template <int F, int BM, int BN, int D>
__global__ __launch_bounds__(kMfmaThreads, 2) void k_mfma_kq(const KqArgs a) {
    using G = KqGeom<F>;
    constexpr int FM = BM / 64, FN = BN / 64;     // 32x32 fragments per wave
    constexpr int XCH = BM * 8 / kMfmaThreads;    // 16-byte activation chunks per thread per step
    constexpr int TILE_X = BM * kMfmaRowBytes;    // activations (bf16, padded rows)
    constexpr int TILE_W = BN * kMfmaRowBytes;    // codes as bf16(128 + q)
    constexpr int TILE_S = BN * 16;               // per weight row: s0, s1, t0, t1
    constexpr int TILE_XS = 2 * BM * 4;           // per sub-block and activation row: X
    constexpr int BUF = TILE_X + TILE_W + TILE_S + TILE_XS;
    __shared__ __attribute__((aligned(16))) uint8_t smem_generic[2 * BUF];
    lds_u8* smem = (lds_u8*)smem_generic;

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const int wm = (wid >> 1) * (BM / 2), wn = (wid & 1) * (BN / 2);
    const int K = a.K, M = a.M, N = a.N;
    const int nsteps = K / kMfmaKStep;  // K is a multiple of 256

    // Register ring: activation chunks and this thread's weight piece (a
    // quarter of one row's 32 code bytes for the step, the row's 16-byte
    // header and, for Q5_K, the 8 fifth-bit bytes of the same positions).
    static_assert(BN * 4 == kMfmaThreads, "four threads per weight row");
    u32x4 xr[D][XCH];
    u32x4 wh[D];
    u32x2 wq[D], wf[D];
    const int wr = tid >> 2, wpart = tid & 3;  // weight tile row and quarter owned by this thread

    // Per-thread row pointers, fixed for the whole K loop.  Rows past M or N
    // read row M - 1 or row 0 instead: such rows feed only outputs that are
    // never written, so no select is needed.
    const uint16_t* xp[XCH];
#pragma unroll
    for (int c = 0; c < XCH; ++c) {
        const int i = tid + c * kMfmaThreads;
        xp[c] = a.x + (size_t)min(m0 + (i >> 3), M - 1) * a.ldx + (i & 7) * 8;
    }
    const uint8_t* wrow = a.w + (size_t)(n0 + wr < N ? n0 + wr : 0) * a.rb;
    const uint8_t* wcode = wrow + G::CODES + 8 * wpart;
    const uint8_t* whigh = wrow + (G::HIGH >= 0 ? G::HIGH : 0) + 8 * wpart;

    // Loads without branches: a load under a branch makes the compiler wait
    // for every outstanding load.
    auto load = [&](int s, auto stage_tag) {
        constexpr int j = decltype(stage_tag)::value;
        const int k0 = s * kMfmaKStep;
#pragma unroll
        for (int c = 0; c < XCH; ++c) xr[j][c] = ld_global128(xp[c] + k0);
        const size_t bo = (size_t)(s >> 2) * G::BB;
        wq[j] = ld_global64(wcode + bo + 32 * (s & 3));
        wh[j] = ld_global128(wrow + bo);
        if constexpr (G::HIGH >= 0) wf[j] = ld_global64(whigh + bo);
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
            // sum of this chunk's 8 values (pairs dotted with (1, 1)), then over
            // the 4 chunks of the sub-block: lanes xor 1, then xor 2 of a quad
            // (element copies first: a bit cast of a vector element reads element 0)
            const uint32_t e0 = xr[j][c].x, e1 = xr[j][c].y, e2 = xr[j][c].z, e3 = xr[j][c].w;
            float p = dot2bf(e0, kBf16Ones, 0.f);
            p = dot2bf(e1, kBf16Ones, p);
            p = dot2bf(e2, kBf16Ones, p);
            p = dot2bf(e3, kBf16Ones, p);
            p += __builtin_amdgcn_update_dpp(0.f, p, kDppQuadXor1, 0xF, 0xF, false);
            p += __builtin_amdgcn_update_dpp(0.f, p, kDppQuadXor2, 0xF, 0xF, false);
            if ((q & 3) == 0) txs[(q >> 2) * BM + r] = p;
        }
        // codes: bytes [8 part, 8 part + 8) of quarter g; low nibbles are
        // positions 8 part .. + 7 of sub-block 2g, high nibbles of 2g + 1
        const int g = s & 3;
        uint32_t l0 = wq[j].x & 0x0F0F0F0Fu, l1 = wq[j].y & 0x0F0F0F0Fu;
        uint32_t h0 = (wq[j].x >> 4) & 0x0F0F0F0Fu, h1 = (wq[j].y >> 4) & 0x0F0F0F0Fu;
        if constexpr (G::HIGH >= 0) {
            // fifth bit of sub-block 2g + t at bit 2g + t of each H byte
            const uint32_t f0 = wf[j].x >> (2 * g), f1 = wf[j].y >> (2 * g);
            l0 |= (f0 << 4) & 0x10101010u;
            l1 |= (f1 << 4) & 0x10101010u;
            h0 |= (f0 << 3) & 0x10101010u;
            h1 |= (f1 << 3) & 0x10101010u;
        }
        lds_u8* pw = tw + wr * kMfmaRowBytes;
        *(lds_u32x4*)(pw + 16 * wpart) =
            u32x4{bias128_pair(l0, kSelB0B1), bias128_pair(l0, kSelB2B3), bias128_pair(l1, kSelB0B1),
                  bias128_pair(l1, kSelB2B3)};
        *(lds_u32x4*)(pw + 64 + 16 * wpart) =
            u32x4{bias128_pair(h0, kSelB0B1), bias128_pair(h0, kSelB2B3), bias128_pair(h1, kSelB0B1),
                  bias128_pair(h1, kSelB2B3)};
        if (wpart < 2) {
            // 6-bit scale and min of sub-block jb = 2g + part (Q4_K packing over
            // S[0..3], S[4..7], S[8..11]: jb < 4 whole in S[jb], S[jb + 4];
            // jb >= 4 low bits in S[jb + 4], top bits in S[jb - 4] and S[jb])
            const uint32_t S0 = wh[j].y, S1 = wh[j].z, S2 = wh[j].w;
            const uint32_t o = 8u * (uint32_t)((2 * g + wpart) & 3);
            uint32_t sc, m;
            if (g < 2) {
                sc = __builtin_amdgcn_ubfe(S0, o, 6);
                m = __builtin_amdgcn_ubfe(S1, o, 6);
            } else {
                sc = __builtin_amdgcn_ubfe(S2, o, 4) | (__builtin_amdgcn_ubfe(S0, o + 6, 2) << 4);
                m = __builtin_amdgcn_ubfe(S2, o + 4, 4) | (__builtin_amdgcn_ubfe(S1, o + 6, 2) << 4);
            }
            const float d = f16_to_f32(wh[j].x), dmin = f16_to_f32(wh[j].x >> 16);
            const float sv = d * (float)sc;
            ts[wr * 4 + wpart] = sv;
            ts[wr * 4 + 2 + wpart] = -fmaf(dmin, (float)m, 128.f * sv);
        }
    };

    // One fp32 accumulator per fragment takes both terms: t * X from the
    // matrix cores, s * D from the vector unit.  (At most 256 registers per
    // lane, two waves per SIMD: the compiler then keeps matrix-core results in
    // ordinary VGPRs, which the vector unit can read without copies.)
    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    const int frow = lane & 31, fcol = (lane >> 5) * 16, half = lane >> 5;
    auto mma = [&](int buf) {
        const lds_u8* tx = smem + buf * BUF;
        const lds_u8* tw = tx + TILE_X;
        const lds_f32* ts = (const lds_f32*)(tw + TILE_W);
        const lds_f32* txs = (const lds_f32*)((const lds_u8*)ts + TILE_S);
        // t * X of both sub-blocks in one 32x32x2 fp32 product per fragment:
        // A[m][k] = X(row m, sub-block k), lane l holds m = l % 32, k = l / 32;
        // B[k][n] = t(row n, sub-block k), same lane mapping.
        float xa[FM], tb[FN], sv[FN][2];
#pragma unroll
        for (int i = 0; i < FM; ++i) xa[i] = txs[half * BM + wm + 32 * i + frow];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int row = (wn + 32 * j + frow) * 4;
            tb[j] = ts[row + 2 + half];
            sv[j][0] = ts[row];
            sv[j][1] = ts[row + 1];
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(xa[i], tb[j], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            bf16x8_t fa[FM][2], fb[FN][2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int kk = 2 * sb + h;
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    fa[i][h] = __builtin_bit_cast(
                        bf16x8_t, lds_ld128(tx + (wm + 32 * i + frow) * kMfmaRowBytes + kk * 32 + fcol));
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    fb[j][h] = __builtin_bit_cast(
                        bf16x8_t, lds_ld128(tw + (wn + 32 * j + frow) * kMfmaRowBytes + kk * 32 + fcol));
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    // D = sum (128 + q) x over the sub-block, then acc += s * D
                    f32x16 dsum = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i][0], fb[j][0], f32x16{}, 0, 0, 0);
                    dsum = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i][1], fb[j][1], dsum, 0, 0, 0);
                    const float s = sv[j][sb];
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][j][r] = fmaf(s, dsum[r], acc[i][j][r]);
                }
        }
    };

    // prologue: steps 0 .. D-1 in flight, step 0 in LDS, step D into the freed stage
    static_for<D>([&](auto j) { load(min((int)decltype(j)::value, nsteps - 1), j); });
    store(0, 0, std::integral_constant<int, 0>{});
    load(min(D, nsteps - 1), std::integral_constant<int, 0>{});
    __syncthreads();
    // main loop over whole groups of D steps: no branches, so the compiler
    // waits only for the loads each store needs
    int s0 = 0;
    for (; s0 + D < nsteps; s0 += D) {
        static_for<D>([&](auto jt) {
            constexpr int j = decltype(jt)::value;
            constexpr int nj = (j + 1) % D;
            const int s = s0 + j;
            mma(j & 1);  // s0 is a multiple of D (even), so s & 1 == j & 1
            __builtin_amdgcn_sched_barrier(0);
            store((j + 1) & 1, s + 1, std::integral_constant<int, nj>{});
            __builtin_amdgcn_sched_barrier(0);
            load(min(s + 1 + D, nsteps - 1), std::integral_constant<int, nj>{});  // (past the end: a harmless reload)
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
        });
    }
    // the last (up to D) steps
    static_for<D>([&](auto jt) {
        constexpr int j = decltype(jt)::value;
        constexpr int nj = (j + 1) % D;
        const int s = s0 + j;
        if (s < nsteps) {
            mma(j & 1);
            if (s + 1 < nsteps) store((j + 1) & 1, s + 1, std::integral_constant<int, nj>{});
            __syncthreads();
        }
    });

#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const int n = n0 + wn + 32 * j + (lane & 31);
                if (m < M && n < N) st_global_f32(a.y + (size_t)m * a.ldy + n, acc[i][j][r]);
            }
}

// Tile shape: 128 x 64 when its tile count covers every CU, else 64 x 64.
// (A 128 x 128 tile needs more than the 256 registers per lane that keep the
// matrix-core results in VGPRs.)
template <int F>
static hipError_t launch_kq(const KqArgs& a, hipStream_t st) {
    const long cus = num_cus();
    const long tiles = (long)((a.N + 63) / 64) * ((a.M + 127) / 128);
    if (tiles >= cus) {
        dim3 grid((a.N + 63) / 64, (a.M + 127) / 128);
        hipLaunchKernelGGL((k_mfma_kq<F, 128, 64, 2>), grid, dim3(kMfmaThreads), 0, st, a);
    } else {
        dim3 grid((a.N + 63) / 64, (a.M + 63) / 64);
        hipLaunchKernelGGL((k_mfma_kq<F, 64, 64, 4>), grid, dim3(kMfmaThreads), 0, st, a);
    }
    return hipGetLastError();
}

hipError_t launch_mfma_kquant(int fmt, const uint8_t* w, int N, int K, const uint16_t* x, int64_t ldx, int M,
                              float* y, int64_t ldy, hipStream_t st) {
    KqArgs a = {x, ldx, w, 0, y, ldy, M, N, K};
    if (fmt == QG_Q4_K) {
        a.rb = (int64_t)(K / 256) * KqGeom<QG_Q4_K>::BB;
        return launch_kq<QG_Q4_K>(a, st);
    }
    if (fmt == QG_Q5_K) {
        a.rb = (int64_t)(K / 256) * KqGeom<QG_Q5_K>::BB;
        return launch_kq<QG_Q5_K>(a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace qg
