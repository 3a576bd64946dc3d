// qg_mfma.hip -- NVFP4 product for M >= 32 activation rows on the bf16 matrix
// cores (v_mfma_f32_32x32x16_bf16).
//
// With many activation rows the product is a dense contraction, so weights are
// decoded once per workgroup tile and used by every activation row of the tile
// ("I Built a Custom Blackwell Kernel for Qwen3.8-27B", section "What the
// custom path actually does": E2M1 codes, one E4M3 scale per 16 values, one
// fp32 scale per tensor).  An E2M1 value has at most 2 significant bits and an
// E4M3 scale at most 4, so their product is exact in bf16 (8 bits): the tile
// holds bf16(c * s) with no rounding, the matrix cores form exact fp32
// products with the bf16 activations and accumulate in fp32, and the tensor
// scale g multiplies the fp32 sum once per output.
//
// Tiling: a 256-thread workgroup computes a BM x BN tile of y (activation rows
// x weight rows); its four waves each own a (BM/2) x (BN/2) quarter as
// (BM/64) x (BN/64) 32x32 accumulators.  K advances 64 values (four NVFP4
// blocks) per step through two LDS buffers: while the matrix cores work on
// one, the next step is decoded into the other, and the loads of the steps
// after it are already in flight in a register ring several steps deep.
#include "qg_mfma.h"

namespace qg {

constexpr int kMfmaStages = 4;  // K steps of loads in flight (an even number)


struct MfmaArgs {
    const uint16_t* x;  // bf16 [M, K], row stride ldx
    int64_t ldx;
    const uint8_t* codes;   // E2M1 plane, K/2 bytes per row
    const uint8_t* scales;  // E4M3 plane, K/16 bytes per row
    const uint8_t* gbytes;  // fp32 tensor scale (any alignment)
    float* y;               // fp32 [M, N], row stride ldy
    int64_t ldy;
    int M, N, K;
};

template <int BM, int BN>
__global__ __launch_bounds__(kMfmaThreads) void k_mfma_nvfp4(const MfmaArgs a) {
    constexpr int FM = BM / 64, FN = BN / 64;          // 32x32 fragments per wave
    constexpr int XCH = BM * 8 / kMfmaThreads;         // 16-byte activation chunks per thread per step
    constexpr int TILE_X = BM * kMfmaRowBytes, TILE_W = BN * kMfmaRowBytes;
    __shared__ __attribute__((aligned(16))) uint8_t smem_generic[2 * (TILE_X + TILE_W)];
    lds_u8* smem = (lds_u8*)smem_generic;

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const int wm = (wid >> 1) * (BM / 2), wn = (wid & 1) * (BN / 2);
    const int K = a.K, M = a.M, N = a.N;
    const int nsteps = (K + kMfmaKStep - 1) / kMfmaKStep;
    const int64_t crow = K / 2, srow = K / 16;

    // Per-thread register staging of one K step (activation chunks and one
    // NVFP4 block), in a ring of kMfmaStages steps: the loads of step s + 1 +
    // kMfmaStages - 1 are issued while step s is on the matrix cores, so the
    // memory latency is covered by several steps of work.
    constexpr int D = kMfmaStages;
    u32x4 xr[D][XCH];
    u32x4 wc[D];
    uint32_t wsb[D];
    const int wr = tid >> 1, wh = tid & 1;  // weight tile row and block half owned by this thread
    const bool w_owner = tid < BN * 2;

    // Loads are branch-free (clamped addresses, results selected afterwards):
    // a load under a branch makes the compiler wait for every outstanding load
    // before the next use, which would void the prefetch.
    auto load = [&](int s, auto stage_tag) {
        constexpr int j = decltype(stage_tag)::value;
        const int k0 = s * kMfmaKStep;
#pragma unroll
        for (int c = 0; c < XCH; ++c) {
            const int i = tid + c * kMfmaThreads;
            const int r = i >> 3, q = i & 7;
            const int m = m0 + r, k = k0 + q * 8;
            const bool ok = m < M && k < K;
            const u32x4 v = ld_global128(a.x + (ok ? (size_t)m * a.ldx + k : 0));
            xr[j][c] = ok ? v : u32x4{0u, 0u, 0u, 0u};
        }
        // 32 values = two NVFP4 blocks of row n; a row whose K % 32 == 16 ends
        // with a single block, whose neighbour bytes (inside the tensor) are
        // read and dropped
        const int n = n0 + wr, kb = k0 + wh * 32;
        const bool ok = w_owner && n < N && kb < K;
        const bool two = kb + 16 < K;
        const size_t nn = ok ? (size_t)n : 0, kk = ok ? (size_t)kb : 0;
        const u32x4 cw = ld_global128(a.codes + nn * crow + kk / 2);
        const uint32_t sw = *(const QG_GLOBAL uint16_t*)(uintptr_t)(a.scales + nn * srow + kk / 16);
        wc[j] = ok ? (two ? cw : u32x4{cw.x, cw.y, 0u, 0u}) : u32x4{0u, 0u, 0u, 0u};
        wsb[j] = ok ? (two ? sw : (sw & 0xffu)) : 0u;
    };
    auto store = [&](int buf, auto stage_tag) {
        constexpr int j = decltype(stage_tag)::value;
        lds_u8* tx = smem + buf * (TILE_X + TILE_W);
        lds_u8* tw = tx + TILE_X;
#pragma unroll
        for (int c = 0; c < XCH; ++c) {
            const int i = tid + c * kMfmaThreads;
            *(lds_u32x4*)(tx + (i >> 3) * kMfmaRowBytes + (i & 7) * 16) = xr[j][c];
        }
        if (w_owner) {
            uint32_t o[8], o2[8];
            decode_nvfp4_block_bf16(wc[j].x, wc[j].y, e4m3_to_f32<0>(wsb[j]), o);
            decode_nvfp4_block_bf16(wc[j].z, wc[j].w, e4m3_to_f32<1>(wsb[j]), o2);
            lds_u8* p = tw + wr * kMfmaRowBytes + wh * 64;
            *(lds_u32x4*)p = u32x4{o[0], o[1], o[2], o[3]};
            *(lds_u32x4*)(p + 16) = u32x4{o[4], o[5], o[6], o[7]};
            *(lds_u32x4*)(p + 32) = u32x4{o2[0], o2[1], o2[2], o2[3]};
            *(lds_u32x4*)(p + 48) = u32x4{o2[4], o2[5], o2[6], o2[7]};
        }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    const int frow = lane & 31, fcol = (lane >> 5) * 16;
    auto mma = [&](int buf) {
        const lds_u8* tx = smem + buf * (TILE_X + TILE_W);
        const lds_u8* tw = tx + TILE_X;
#pragma unroll
        for (int kk = 0; kk < kMfmaKStep / 16; ++kk) {
            bf16x8_t fa[FM], fb[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                fa[i] = __builtin_bit_cast(bf16x8_t, lds_ld128(tx + (wm + 32 * i + frow) * kMfmaRowBytes + kk * 32 + fcol));
#pragma unroll
            for (int j = 0; j < FN; ++j)
                fb[j] = __builtin_bit_cast(bf16x8_t, lds_ld128(tw + (wn + 32 * j + frow) * kMfmaRowBytes + kk * 32 + fcol));
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
    };

    // prologue: steps 0 .. D-1 in flight, step 0 in LDS, step D into the freed stage
    static_for<D>([&](auto j) { load(min((int)decltype(j)::value, nsteps - 1), j); });
    store(0, std::integral_constant<int, 0>{});
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
            store((j + 1) & 1, std::integral_constant<int, nj>{});
            load(min(s + 1 + D, nsteps - 1), std::integral_constant<int, nj>{});  // (past the end: a harmless reload)
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
            if (s + 1 < nsteps) store((j + 1) & 1, std::integral_constant<int, nj>{});
            __syncthreads();
        }
    });

    const uint8_t* gb = a.gbytes;
    const uint32_t gbits = (uint32_t)gb[0] | ((uint32_t)gb[1] << 8) | ((uint32_t)gb[2] << 16) | ((uint32_t)gb[3] << 24);
    const float g = __builtin_bit_cast(float, gbits);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const int n = n0 + wn + 32 * j + (lane & 31);
                if (m < M && n < N) st_global_f32(a.y + (size_t)m * a.ldy + n, g * acc[i][j][r]);
            }
}

// Tile shape: the largest whose tile count still gives every CU at least two
// workgroups, else the smallest.
hipError_t launch_mfma_nvfp4(const uint8_t* codes, const uint8_t* scales, const uint8_t* gbytes, int N, int K,
                             const uint16_t* x, int64_t ldx, int M, float* y, int64_t ldy, hipStream_t st) {
    MfmaArgs a = {x, ldx, codes, scales, gbytes, y, ldy, M, N, K};
    const long cus = num_cus();
    auto tiles = [&](int bm, int bn) { return (long)((N + bn - 1) / bn) * ((M + bm - 1) / bm); };
    if (tiles(128, 128) >= 2 * cus) {
        dim3 grid((N + 127) / 128, (M + 127) / 128);
        hipLaunchKernelGGL((k_mfma_nvfp4<128, 128>), grid, dim3(kMfmaThreads), 0, st, a);
    } else if (tiles(128, 64) >= cus) {
        dim3 grid((N + 63) / 64, (M + 127) / 128);
        hipLaunchKernelGGL((k_mfma_nvfp4<128, 64>), grid, dim3(kMfmaThreads), 0, st, a);
    } else {
        dim3 grid((N + 63) / 64, (M + 63) / 64);
        hipLaunchKernelGGL((k_mfma_nvfp4<64, 64>), grid, dim3(kMfmaThreads), 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace qg
