// qg_gemv.hip -- dense decode GEMV (M = 1) and skinny product (M <= 16 rows
// per pass) over one packed weight matrix: persistent workgroups, the grid's
// waves taking rows n = gw, gw + GW, ...  The streaming core is qg_stream.h.
#include "qg_stream.h"

namespace qg {

// LDS layout: [x bf16: MT*K][x sums fp32: MT*K/16][per-wave row buffers]
template <int F, int MT, int CPL, int CPLS, int PF>
__global__ __launch_bounds__(256) void k_stream_gemm(const StreamArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem_generic[];
    lds_u8* smem = (lds_u8*)smem_generic;
    constexpr bool kSums = (F == QG_Q4_K || F == QG_Q6_K);
    const int K = a.K;
    lds_u8* xl = smem;
    lds_f32* xs = (lds_f32*)(smem + (size_t)MT * K * 2);
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    lds_u8* rowbuf = smem + rowbuf_offset(MT, K) + (size_t)wid * rowbuf_bytes(CPL, CPLS);
    lds_u8* rowbuf_s = rowbuf + CPL * 1024 + 32;

    stage_x<MT, kSums>(xl, xs, a.x, a.ldx, a.M, K, [&](int m) { return a.xrow[m]; });

    const int lane = threadIdx.x & 63;
    const int GW = gridDim.x * kWavesPerBlock;
    const int gw = blockIdx.x * kWavesPerBlock + wid;
    MatView mv = {a.w0, a.rb0, a.w1, a.rb1, a.gbytes};
    const int64_t yrow = a.yrow[lane < a.M ? lane : 0];
    wave_stream<F, MT, CPL, CPLS, PF>(mv, K, a.seg_blocks, a.nseg, xl, xs, rowbuf, rowbuf_s, gw, GW, a.N, a.y,
                                      a.ldy, yrow, a.M);
}

template <int F, int MT, int CPL, int CPLS, int PF>
static hipError_t launch_one(const StreamArgs& a, int per_cu, hipStream_t st) {
    const size_t lds = gemv_lds_bytes(MT, a.K, CPL, CPLS);
    auto kern = k_stream_gemm<F, MT, CPL, CPLS, PF>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    // persistent grid: as many 4-wave workgroups as fit at once, never more waves than rows
    int fit = (int)(kLdsBytes / lds);
    if (fit > per_cu) fit = per_cu;
    if (fit < 1) fit = 1;
    long waves = (long)num_cus() * fit * kWavesPerBlock;
    if (waves > a.N) waves = a.N;
    const int grid = (int)((waves + kWavesPerBlock - 1) / kWavesPerBlock);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, st, a);
    return hipGetLastError();
}

template <int F, int MT>
static hipError_t dispatch_cpl(StreamArgs a, hipStream_t st) {
    const int cpl = choose_cpl(F, a.K);
    a.seg_blocks = segment_blocks(F, a.K, cpl);
    const int nb = a.K / BlockGeom<F>::QK;
    a.nseg = (nb + a.seg_blocks - 1) / a.seg_blocks;
    constexpr int S = (F == QG_NVFP4) ? 1 : 0;
    switch (cpl) {
        case 1: return launch_one<F, MT, 1, S, 4>(a, 4, st);
        case 2: return launch_one<F, MT, 2, S, 4>(a, 4, st);
        case 3: return launch_one<F, MT, 3, S, 4>(a, 4, st);
        case 4: return launch_one<F, MT, 4, S, 3>(a, 4, st);
        default: return launch_one<F, MT, 6, S, 2>(a, 4, st);
    }
}

template <int F>
static hipError_t dispatch_mt(const StreamArgs& a, int mt, hipStream_t st) {
    switch (mt) {
        case 1: return dispatch_cpl<F, 1>(a, st);
        case 2: return dispatch_cpl<F, 2>(a, st);
        case 4: return dispatch_cpl<F, 4>(a, st);
        case 8: return dispatch_cpl<F, 8>(a, st);
        default: return dispatch_cpl<F, 16>(a, st);
    }
}

static int mt_for(int m) { return m <= 1 ? 1 : m <= 2 ? 2 : m <= 4 ? 4 : m <= 8 ? 8 : 16; }

// Activation rows one pass of the streaming kernel can take: the largest of
// 16, 8, 4, 2, 1 (capped by M) whose activations, activation sums and row
// buffers fit in the 160 KB of LDS.  0 when not even one row fits.
int stream_rows_per_pass(int fmt, int K, int M) {
    const int cands[5] = {16, 8, 4, 2, 1};
    const int cpl = choose_cpl(fmt, K);
    for (int i = 0; i < 5; ++i) {
        const int mt = cands[i];
        if (mt > 1 && mt / 2 >= M) continue;  // a smaller instantiation already covers M
        if (gemv_lds_bytes(mt, K, cpl, fmt == QG_NVFP4 ? 1 : 0) <= (size_t)kLdsBytes) return mt < M ? mt : M;
    }
    return 0;
}

hipError_t launch_stream_gemm(int fmt, StreamArgs a, hipStream_t st) {
    const int mt = mt_for(a.M);
    switch (fmt) {
        case QG_Q8_0: return dispatch_mt<QG_Q8_0>(a, mt, st);
        case QG_Q4_K: return dispatch_mt<QG_Q4_K>(a, mt, st);
        case QG_Q6_K: return dispatch_mt<QG_Q6_K>(a, mt, st);
        default: return dispatch_mt<QG_NVFP4>(a, mt, st);
    }
}

}  // namespace qg
