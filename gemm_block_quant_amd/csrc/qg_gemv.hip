// qg_gemv.hip -- dense decode GEMV (M = 1) and skinny product (M <= 16 rows
// per pass) over one packed weight matrix.  Q4_K, Q6_K and NVFP4 (K % 64 ==
// 0) stream straight into registers and multiply on the matrix cores
// (qg_direct.h); Q8_0 and NVFP4 with K % 64 == 32 go through a wave-private
// LDS row buffer (qg_stream.h).
#include "qg_direct.h"

namespace qg {

// The direct kernel's LDS starts with its row-group counter.
constexpr int kDirectCounterBytes = 64;  // item counters of up to 16 K phases

// LDS one launch needs for `mt` activation rows.
// Direct path: LDS of one launch with K staged in `nph` phases, for a share of
// `rgs` row groups.
static size_t direct_launch_lds(int fmt, int K, int mt, Segments sg, int nph, int64_t rgs) {
    const int seg_per_ph = (sg.S + nph - 1) / nph;
    const int U = K / 64;
    const int KLmax = (U < seg_per_ph * sg.PS * kDirectSlots ? U : seg_per_ph * sg.PS * kDirectSlots) * 64;
    return kDirectCounterBytes + direct_lds_bytes(fmt, mt, KLmax) + direct_seg_lds_bytes(sg.S, (int)rgs, mt);
}

// Fewest K phases (at most 16, each a whole number of segments) whose staged
// activations fit in LDS; 0 when none does.
static int direct_phases(int fmt, int64_t N, int K, int mt) {
    const int cus = num_cus();
    const Segments sg = direct_segments(fmt, N, K, cus);
    const int64_t groups = (N + kDirectRows - 1) / kDirectRows;
    // largest share of row groups a workgroup gets (the grid holds at least
    // min(cus, groups) workgroups)
    const int64_t rgs = groups > cus ? (groups + cus - 1) / cus : 1;
    for (int nph = 1; nph <= sg.S && nph <= kDirectCounterBytes / 4; ++nph)
        if (direct_launch_lds(fmt, K, mt, sg, nph, rgs) <= (size_t)kLdsBytes) return nph;
    return 0;
}

size_t stream_lds_bytes(int fmt, int K, int mt) {
    if (direct_eligible(fmt, K))
        return kDirectCounterBytes + direct_lds_bytes(fmt, mt, K) + direct_seg_lds_bytes(2, kDirectSegRgsMax, mt);  // (worst case)
    return gemv_lds_bytes(mt, K, choose_cpl(fmt, K), fmt == QG_NVFP4 ? 1 : 0);
}

template <int F, int MT, int CPL, int CPLS, int PF>
__global__ __launch_bounds__(256) void k_stream_gemm(const StreamArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem_generic[];
    lds_u8* smem = (lds_u8*)smem_generic;
    const int K = a.K;
    lds_u8* xl = smem;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    lds_u8* rowbuf = smem + rowbuf_offset(MT, K) + (size_t)wid * rowbuf_bytes(CPL, CPLS);
    lds_u8* rowbuf_s = rowbuf + CPL * 1024 + 32;
    const int lane = threadIdx.x & 63;
    const int GW = gridDim.x * kWavesPerBlock;
    const int gw = blockIdx.x * kWavesPerBlock + wid;
    MatView mv = {a.w0, a.rb0, a.w1, a.rb1, a.gbytes};
    const int64_t yrow = a.yrow[lane < a.M ? lane : 0];
    auto stage = [&] { stage_x<MT>(xl, a.x, a.ldx, a.M, K, [&](int m) { return a.xrow[m]; }); };
    wave_stream<F, MT, CPL, CPLS, PF>(mv, K, a.seg_blocks, a.nseg, xl, rowbuf, rowbuf_s, gw, GW, a.N, a.y, a.ldy,
                                      yrow, a.M, stage);
}

// Direct path: workgroups of the wave counts below, as many per CU as the
// registers allow (one at one activation row).  Workgroup b owns an equal
// contiguous share of the row groups; its waves take (row group, K segment)
// items one at a time from a counter in LDS, so every CU finishes within
// about one item of the others.  The order in which waves take items does not
// change any row's arithmetic.
// 16 waves per workgroup; 8 where the accumulators of many activation rows
// need more registers than 4 waves per SIMD allow, and for one activation row
// (measured 5 % faster than 16 on the Q6_K LM head and down projection, 1-2 %
// on Q4_K and FP8, 1 % slower on NVFP4, which keeps 16).  At one row the
// unsegmented launch puts one workgroup of direct_row1_waves on each CU (see
// dispatch_direct); the Q6_K kernels (132-176 VGPRs) fit only one anyway.
// More waves per CU were slower: Q6_K capped at 128 VGPRs to fit two
// workgroups spilled and ran 6 % (LM head) and 59 % (down projection)
// slower, 4-wave workgroups at five waves per SIMD 6 % slower on Q4_K and 2 %
// on FP8, 8-wave NVFP4 workgroups 25 % slower on the down projection.
template <int F, int MT> constexpr int direct_waves() {
    return MT >= 16 || ((F == QG_Q6_K || F == QG_Q5_K) && MT >= 8) || (MT == 1 && F != QG_NVFP4) ? 8 : 16;
}
// Waves of the one workgroup per CU that the unsegmented kernel runs at one
// activation row.  Swept per format (waves per CU, Q4_K gate+up matrix:
// 6 22.3, 7 21.9, 8 21.3, 9 20.9, 10 20.7, 12 21.8 us; NVFP4 17408 rows: 7-9
// 12.5, 10 12.3, 12-16 12.4-12.6 us; FP8 gate+up: 4 33.7, 5 32.1, 6 33.1,
// 7 32.3, 8 36.2, 9-10 32.3 us, and its LM head 5-6 214 us against 237 at
// 8; Q6_K LM head: 6 227, 8 201, 10 194.5, 12 195 us; Q5_K keeps 8: 6, 7, 9
// and 10 were slower; on another box 9 and 11 waves against 10: Q4_K +2 %
// and +4 %, NVFP4 +2 % and +1 %, the Q6_K LM head +1.5 % and -0.6 %).
template <int F> constexpr int direct_row1_waves() {
    return F == QG_Q4_K || F == QG_NVFP4 || F == QG_Q6_K ? 10 : F == QG_FP8 ? 5 : 8;
}
// Waves per workgroup of the unsegmented launch: the one-row table above;
// 12 for the 8-row Q6_K and Q5_K kernels, whose 146-165 registers allow
// three waves per SIMD (Q6_K LM head at eight rows 256 -> 242 us, 10 waves
// 249 us; Q5_K gate+up 41.2 -> 39.9 us); otherwise direct_waves.
template <int F, int MT> constexpr int direct_plain_waves() {
    return MT == 1 ? direct_row1_waves<F>() : (F == QG_Q6_K || F == QG_Q5_K) && MT == 8 ? 12 : direct_waves<F, MT>();
}
// The kernel's block-size bound covers the launches of its instantiation
// (the segmented one keeps direct_waves: a larger bound would cap its
// registers below what the Q6_K segmented kernels hold).
template <int F, int MT, bool SEG> constexpr int direct_bound() {
    return !SEG && direct_plain_waves<F, MT>() > direct_waves<F, MT>() ? direct_plain_waves<F, MT>()
                                                                       : direct_waves<F, MT>();
}

// Eager activation staging (see XStage) for the 8-wave Q5_K and Q6_K kernels,
// with up to five vectors per thread loaded before the weight loads (one row
// of K <= 20,480 values; two at 16 rows, where more would spill): measured
// 1-2 % faster on the Q6_K down projection at one and eight activation rows,
// on the Q6_K LM head and on Q5_K.  The other kernels keep two vectors and the waiting form
// (eager staging measured 1 % slower on Q4_K, 8 % on FP8 and up to 17 % on
// NVFP4 at eight rows).
// Waves per workgroup of the segment-per-workgroup launch (XS, eight rows):
// 12 for Q6_K, whose 165 registers allow three waves per SIMD (the down
// projection at eight rows 31.0 -> 29.1 us); direct_waves otherwise.
template <int F, int MT> constexpr int direct_xs_waves() { return F == QG_Q6_K ? 12 : direct_waves<F, MT>(); }

template <int F, int MT> constexpr bool direct_eager() {
    return direct_waves<F, MT>() == 8 && (F == QG_Q5_K || F == QG_Q6_K);
}
template <int F, int MT> constexpr int direct_xv() { return direct_eager<F, MT>() && MT < 16 ? 5 : 2; }

// SEG false: one K segment and one phase (the launch guarantees it).
// XS: each workgroup takes one K segment (workgroup b: segment b % S, the
// (b / S)-th share of the row groups), stages only that segment's activations
// and adds its sums to the other segments' through a.xs_part / a.xs_cnt.
template <int F, int MT, int SP, int PF, bool SEG, bool XS = false>
__global__ __launch_bounds__(((XS ? direct_xs_waves<F, MT>() : direct_bound<F, MT, SEG>()) * 64)) void k_direct_gemm(
    const StreamArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem_generic[];
    lds_u8* smem = (lds_u8*)smem_generic;
    constexpr int RW = kDirectRows;
    const int K = a.K;
    const int U = K / 64;
    const Segments sg = SEG ? Segments{a.seg_S > 0 ? a.seg_S : 1, a.seg_PS > 0 ? a.seg_PS : 1}
                            : Segments{1, (U + kDirectSlots - 1) / kDirectSlots};
    const int nph = XS ? 1 : SEG && a.phases > 0 ? a.phases : 1;
    const int seg_per_ph = XS ? 1 : (sg.S + nph - 1) / nph;
    // LDS: one item counter per phase, then the activations of the longest
    // phase and their sums, then the segment sums
    const int KLmax = min(U, seg_per_ph * sg.PS * kDirectSlots) * 64;
    QG_LDS int* counters = (QG_LDS int*)smem;
    lds_u8* xl = smem + kDirectCounterBytes;
    lds_f32* xs = (lds_f32*)(xl + (size_t)direct_mg(MT) * direct_mg_bytes(F, KLmax));
    const int lane = threadIdx.x & 63;
    const int li = direct_out_slot(lane);
    const int groups = (a.N + RW - 1) / RW;
    // (XS: the grid is a whole number of workgroups per segment)
    const int shares = XS ? (int)gridDim.x / sg.S : (int)gridDim.x;
    const int share = XS ? (int)blockIdx.x / sg.S : (int)blockIdx.x;
    const int per = (groups + shares - 1) / shares;
    const int g0 = share * per, g1 = min(groups, g0 + per);
    const int rgs = g1 > g0 ? g1 - g0 : 0;
    // segment sums after the activations: progress[per], then total[per][4][MT]
    SegLds sl;
    sl.progress = (QG_LDS int*)(xl + direct_lds_bytes(F, MT, KLmax));
    sl.total = (lds_f32*)((lds_u8*)sl.progress + ((size_t)per * 4 + 15) / 16 * 16);
    sl.mtmax = MT;
    sl.gpart = a.xs_part;
    sl.gcnt = a.xs_cnt;
    if (threadIdx.x < kDirectCounterBytes / 4) counters[threadIdx.x] = 0;
    if (SEG && !XS && sg.S > 1)
        for (int i = threadIdx.x; i < per; i += blockDim.x) sl.progress[i] = 0;
    MatView mv = {a.w0, a.rb0, a.w1, a.rb1, a.gbytes};
    // activation and output rows of the pass: resolved once into registers for
    // eager staging, read from the arguments otherwise
    constexpr bool EAGER = direct_eager<F, MT>();
    RowTable<MT> rows;
    if constexpr (EAGER) {
#pragma unroll
        for (int m = 0; m < MT; ++m) rows.set(m, a.xrow[m]);
    }
    auto row_of = [&](int m) {
        if constexpr (EAGER) return rows(m);
        else return a.xrow[m];
    };
    int64_t yrow;
    if constexpr (EAGER) {
        RowTable<MT> yrows;
#pragma unroll
        for (int m = 0; m < MT; ++m) yrows.set(m, a.yrow[m]);
        yrow = yrows(li < a.M ? li : 0);
    } else {
        yrow = a.yrow[li < a.M ? li : 0];
    }
    for (int p = 0; p < nph; ++p) {
        Phase ph;
        ph.s_lo = XS ? (int)blockIdx.x % sg.S : p * seg_per_ph;
        ph.ns = min(sg.S, ph.s_lo + seg_per_ph) - ph.s_lo;
        ph.u0 = ph.s_lo * sg.PS * kDirectSlots;
        ph.KL = (min(U, (ph.s_lo + ph.ns) * sg.PS * kDirectSlots) - ph.u0) * 64;
        const int items = rgs * ph.ns;
        QG_LDS int* counter = counters + p;
        auto next_item = [&]() {
            int t = 0;
            if (lane == 0) t = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            t = __builtin_amdgcn_readfirstlane(t);
            return t < items ? t : -1;
        };
        const uint16_t* xp = a.x + (size_t)ph.u0 * 64;
        XStage<F, MT, direct_xv<F, MT>(), EAGER> xst;
        xst.issue(xp, a.ldx, a.M, ph.KL, row_of);
        // the counters and progress are initialised, and every wave is done with
        // the previous phase's activations, before any wave goes on
        __syncthreads();
        auto between = [&] { xst.commit(xl, xs, xp, a.ldx, a.M, ph.KL, row_of); };
        wave_stream_direct<F, MT, SP, PF, SEG, XS>(mv, a.N, K, xl, xs, next_item, g0, sg, ph, sl, a.y, a.ldy, yrow,
                                                   a.M, between);
    }
    if constexpr (XS) {
        // This workgroup's segment sums (LDS, [row group][4][MT]) to the
        // workspace, every store complete before any row group counts in; the
        // last of a row group's S segments to count in adds the S sums in
        // segment order -- the running sum of the single-workgroup path -- and
        // writes the row group's outputs.  Nothing waits on another workgroup.
        const int S = sg.S, s = (int)blockIdx.x % S;
        constexpr int V = RW * MT;  // values per row group and segment
        __syncthreads();
        for (int i = threadIdx.x; i < rgs * V; i += blockDim.x)
            __hip_atomic_store(a.xs_part + ((size_t)(g0 + i / V) * S + s) * V + i % V, sl.total[i],
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        float gscale = 1.f;
        if (F == QG_NVFP4) {
            const uint8_t* gb = a.gbytes;
            gscale = __builtin_bit_cast(float, (uint32_t)gb[0] | ((uint32_t)gb[1] << 8) | ((uint32_t)gb[2] << 16) |
                                                   ((uint32_t)gb[3] << 24));
        }
        // row groups whose last segment this is, then one output per thread
        QG_LDS int* last = sl.progress;
        for (int t = threadIdx.x; t < rgs; t += blockDim.x)
            last[t] = __hip_atomic_fetch_add(a.xs_cnt + g0 + t, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
        __syncthreads();
        for (int i = threadIdx.x; i < rgs * V; i += blockDim.x) {
            const int t = i / V, e = i % V, gi = e / MT, m = e % MT;
            const int n = RW * (g0 + t) + gi;
            if (!last[t] || m >= a.M || n >= a.N) continue;
            const float* part = a.xs_part + (size_t)(g0 + t) * S * V + e;
            float tot = 0.f;
            for (int q = 0; q < S; ++q) {
                const float v = __hip_atomic_load(part + (size_t)q * V, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                tot = q == 0 ? v : tot + v;
            }
            if (F == QG_NVFP4) tot *= gscale;
            st_global_f32(a.y + (int64_t)a.yrow[m] * a.ldy + n, tot);
        }
    }
}

// Persistent grid: as many 4-wave workgroups as can be resident at once (by
// registers and LDS), never more waves than work items (rows / rows per wave).
template <class Kern>
static hipError_t launch_persistent(Kern kern, const StreamArgs& a, size_t lds, int rows_per_wave, hipStream_t st) {
    int fit = 0;
    hipError_t e = kernel_residency((const void*)kern, lds, &fit, 256);
    if (e != hipSuccess) return e;
    long waves = (long)num_cus() * fit * kWavesPerBlock;
    const long need = (a.N + rows_per_wave - 1) / rows_per_wave;
    if (waves > need) waves = need;
    const int grid = (int)((waves + kWavesPerBlock - 1) / kWavesPerBlock);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, st, a);
    return hipGetLastError();
}

template <int F, int MT>
static hipError_t dispatch_rlt(StreamArgs a, hipStream_t st) {
    const int cpl = choose_cpl(F, a.K);
    a.seg_blocks = segment_blocks(F, a.K, cpl);
    const int nb = a.K / BlockGeom<F>::QK;
    a.nseg = (nb + a.seg_blocks - 1) / a.seg_blocks;
    constexpr int S = (F == QG_NVFP4) ? 1 : 0;
    const size_t lds = gemv_lds_bytes(MT, a.K, cpl, S);
    switch (cpl) {
        case 1: return launch_persistent(k_stream_gemm<F, MT, 1, S, 4>, a, lds, 1, st);
        case 2: return launch_persistent(k_stream_gemm<F, MT, 2, S, 4>, a, lds, 1, st);
        case 3: return launch_persistent(k_stream_gemm<F, MT, 3, S, 4>, a, lds, 1, st);
        case 4: return launch_persistent(k_stream_gemm<F, MT, 4, S, 3>, a, lds, 1, st);
        default: return launch_persistent(k_stream_gemm<F, MT, 6, S, 2>, a, lds, 1, st);
    }
}

// Direct path: SP passes per ring slot, PF slots (pure tuning: the per-row
// arithmetic does not depend on them).
template <int F, int MT> struct DirectTune;
template <int MT> struct DirectTune<QG_Q4_K, MT> { static constexpr int SP = 1, PF = 2; };
template <int MT> struct DirectTune<QG_Q5_K, MT> { static constexpr int SP = 1, PF = 2; };
template <int MT> struct DirectTune<QG_NVFP4, MT> { static constexpr int SP = 1, PF = 2; };
template <int MT> struct DirectTune<QG_Q6_K, MT> { static constexpr int SP = 1, PF = 2; };
template <int MT> struct DirectTune<QG_FP8, MT> { static constexpr int SP = 1, PF = 2; };

template <int F, int MT>
static hipError_t dispatch_direct(StreamArgs a, hipStream_t st) {
    const Segments sg = direct_segments(F, a.N, a.K, num_cus());
    a.seg_S = sg.S;
    a.seg_PS = sg.PS;
    a.phases = direct_phases(F, a.N, a.K, MT);
    if (a.phases <= 0) return hipErrorInvalidValue;
    // one ring slot for NVFP4's K-segmented rows at one activation row (2 %
    // faster on the 5120-row down projection; Q6_K 5 % slower that way)
    constexpr int PFS = F == QG_NVFP4 && MT == 1 ? 1 : DirectTune<F, MT>::PF;
    const bool seg = sg.S > 1 || a.phases > 1;
    auto kern = seg ? k_direct_gemm<F, MT, DirectTune<F, MT>::SP, PFS, true>
                    : k_direct_gemm<F, MT, DirectTune<F, MT>::SP, DirectTune<F, MT>::PF, false>;
    // One activation row on the unsegmented kernel: one workgroup of
    // direct_row1_waves per CU, even where the registers fit more (two 8-wave
    // workgroups per CU measured 1.5-2 % slower on Q4_K, 2-5 % on Q5_K).  The
    // K-segmented kernels keep the residency their segment count is cut for.
    const bool one_per_cu = !seg && MT == 1;
    const int waves = seg ? direct_waves<F, MT>() : direct_plain_waves<F, MT>();
    constexpr int RW = kDirectRows;
    const long groups = (a.N + RW - 1) / RW;
    // grid from the residency, then the LDS for the resulting share of row
    // groups (and the residency again)
    size_t lds = direct_launch_lds(F, a.K, MT, sg, a.phases, 1);
    long grid = 0;
    for (int pass = 0; pass < 2; ++pass) {
        int fit = 0;
        hipError_t e = kernel_residency((const void*)kern, lds, &fit, waves * 64);
        if (e != hipSuccess) return e;
        grid = (long)num_cus() * (one_per_cu ? 1 : fit);
        if (grid > groups) grid = groups;
        const long per = (groups + grid - 1) / grid;
        lds = direct_launch_lds(F, a.K, MT, sg, a.phases, per);
    }
    if (lds > (size_t)kLdsBytes) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(waves * 64), lds, st, a);
    return hipGetLastError();
}

// Segment-per-workgroup launch (XS): taken where the plain launch would stage
// the activations in several K phases (eight rows of K = 17,408), each phase
// then giving a CU only its few row groups' items of one segment.  Workgroups
// of one segment share the row groups in equal contiguous shares.
constexpr int kXsegMT = kXsegRows;

static size_t xseg_counter_bytes(int64_t groups) { return ((size_t)groups * 4 + 255) / 256 * 256; }

template <int F, int MT>
static bool xseg_plan(int64_t N, int K, Segments* sg_out, size_t* lds_out, long* grid_out, long* per_out) {
    const Segments sg = direct_segments(F, N, K, num_cus());
    if (sg.S < 2 || direct_phases(F, N, K, MT) < 2) return false;
    constexpr int RW = kDirectRows;
    const long groups = (N + RW - 1) / RW;
    auto kern = k_direct_gemm<F, MT, DirectTune<F, MT>::SP, DirectTune<F, MT>::PF, true, true>;
    size_t lds = direct_launch_lds(F, K, MT, sg, sg.S, 1);
    long grid = 0, per = 0;
    for (int pass = 0; pass < 2; ++pass) {
        int fit = 0;
        if (kernel_residency((const void*)kern, lds, &fit, direct_xs_waves<F, MT>() * 64) != hipSuccess) return false;
        long shares = (long)num_cus() * fit / sg.S;
        if (shares < 1) shares = 1;
        if (shares > groups) shares = groups;
        per = (groups + shares - 1) / shares;
        grid = shares * sg.S;
        lds = direct_launch_lds(F, K, MT, sg, sg.S, per);
    }
    if (lds > (size_t)kLdsBytes) return false;
    *sg_out = sg;
    *lds_out = lds;
    *grid_out = grid;
    *per_out = per;
    return true;
}

__global__ void k_zero_counters(int32_t* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

template <int F>
static size_t xseg_bytes_fmt(int64_t N, int K) {
    if constexpr (F == QG_Q4_K || F == QG_Q5_K || F == QG_Q6_K || F == QG_NVFP4 || F == QG_FP8) {
        Segments sg;
        size_t lds;
        long grid, per;
        if (!direct_eligible(F, K) || !xseg_plan<F, kXsegMT>(N, K, &sg, &lds, &grid, &per)) return 0;
        const int64_t groups = (N + kDirectRows - 1) / kDirectRows;
        return xseg_counter_bytes(groups) + (size_t)groups * sg.S * kDirectRows * kXsegMT * sizeof(float);
    }
    return 0;
}

size_t direct_xseg_bytes(int fmt, int64_t N, int K, int M) {
    // 5..16 rows, in passes of up to 8 (fewer rows fit one phase on the plain launch)
    if (M < 5 || M > kMaxPassRows) return 0;
    switch (fmt) {
        case QG_Q4_K: return xseg_bytes_fmt<QG_Q4_K>(N, K);
        case QG_Q5_K: return xseg_bytes_fmt<QG_Q5_K>(N, K);
        case QG_Q6_K: return xseg_bytes_fmt<QG_Q6_K>(N, K);
        case QG_NVFP4: return xseg_bytes_fmt<QG_NVFP4>(N, K);
        case QG_FP8: return xseg_bytes_fmt<QG_FP8>(N, K);
        default: return 0;
    }
}

template <int F>
static hipError_t launch_xseg_fmt(StreamArgs a, void* ws, hipStream_t st) {
    if constexpr (F == QG_Q4_K || F == QG_Q5_K || F == QG_Q6_K || F == QG_NVFP4 || F == QG_FP8) {
        constexpr int MT = kXsegMT;
        Segments sg;
        size_t lds;
        long grid, per;
        if (!xseg_plan<F, MT>(a.N, a.K, &sg, &lds, &grid, &per)) return hipErrorInvalidValue;
        const int64_t groups = (a.N + kDirectRows - 1) / kDirectRows;
        a.seg_S = sg.S;
        a.seg_PS = sg.PS;
        a.phases = 1;
        a.xs_cnt = (int32_t*)ws;
        a.xs_part = (float*)((uint8_t*)ws + xseg_counter_bytes(groups));
        // the counters start at zero in every call (a fill kernel, not a
        // memset: the call may be captured into a graph)
        hipLaunchKernelGGL(k_zero_counters, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, st, a.xs_cnt,
                           (int)groups);
        hipLaunchKernelGGL((k_direct_gemm<F, MT, DirectTune<F, MT>::SP, DirectTune<F, MT>::PF, true, true>),
                           dim3((unsigned)grid), dim3(direct_xs_waves<F, MT>() * 64), lds, st, a);
        return hipGetLastError();
    }
    return hipErrorInvalidValue;
}

hipError_t launch_direct_xseg(int fmt, StreamArgs a, void* ws, hipStream_t st) {
    if (a.M < 1 || a.M > kXsegMT) return hipErrorInvalidValue;
    switch (fmt) {
        case QG_Q4_K: return launch_xseg_fmt<QG_Q4_K>(a, ws, st);
        case QG_Q5_K: return launch_xseg_fmt<QG_Q5_K>(a, ws, st);
        case QG_Q6_K: return launch_xseg_fmt<QG_Q6_K>(a, ws, st);
        case QG_NVFP4: return launch_xseg_fmt<QG_NVFP4>(a, ws, st);
        case QG_FP8: return launch_xseg_fmt<QG_FP8>(a, ws, st);
        default: return hipErrorInvalidValue;
    }
}

template <int F>
static hipError_t dispatch_mt(const StreamArgs& a, int mt, hipStream_t st) {
    if constexpr (F == QG_Q4_K || F == QG_Q5_K || F == QG_Q6_K || F == QG_NVFP4 || F == QG_FP8) {
        if (direct_eligible(F, a.K)) {
            switch (mt) {
                case 1: return dispatch_direct<F, 1>(a, st);
                case 2: return dispatch_direct<F, 2>(a, st);
                case 4: return dispatch_direct<F, 4>(a, st);
                case 8: return dispatch_direct<F, 8>(a, st);
                default: return dispatch_direct<F, 16>(a, st);
            }
        }
    }
    if constexpr (F == QG_Q8_0 || F == QG_NVFP4) {
        switch (mt) {
            case 1: return dispatch_rlt<F, 1>(a, st);
            case 2: return dispatch_rlt<F, 2>(a, st);
            case 4: return dispatch_rlt<F, 4>(a, st);
            case 8: return dispatch_rlt<F, 8>(a, st);
            default: return dispatch_rlt<F, 16>(a, st);
        }
    }
    return hipErrorInvalidValue;
}

static int mt_for(int m) { return m <= 1 ? 1 : m <= 2 ? 2 : m <= 4 ? 4 : m <= 8 ? 8 : 16; }

// Activation rows one pass of the streaming kernel can take: the largest of
// 16, 8, 4, 2, 1 (capped by M) whose LDS needs fit in 160 KB.  0 when not
// even one row fits.
int stream_rows_per_pass(int fmt, int64_t N, int K, int M) {
    const int cands[5] = {16, 8, 4, 2, 1};
    for (int i = 0; i < 5; ++i) {
        const int mt = cands[i];
        if (mt > 1 && mt / 2 >= M) continue;  // a smaller instantiation already covers M
        const bool fits = direct_eligible(fmt, K) ? direct_phases(fmt, N, K, mt) > 0
                                                  : stream_lds_bytes(fmt, K, mt) <= (size_t)kLdsBytes;
        if (fits) return mt < M ? mt : M;
    }
    return 0;
}

hipError_t launch_stream_gemm(int fmt, StreamArgs a, hipStream_t st) {
    const int mt = mt_for(a.M);
    switch (fmt) {
        case QG_Q8_0: return dispatch_mt<QG_Q8_0>(a, mt, st);
        case QG_Q4_K: return dispatch_mt<QG_Q4_K>(a, mt, st);
        case QG_Q5_K: return dispatch_mt<QG_Q5_K>(a, mt, st);
        case QG_Q6_K: return dispatch_mt<QG_Q6_K>(a, mt, st);
        case QG_FP8: return dispatch_mt<QG_FP8>(a, mt, st);
        default: return dispatch_mt<QG_NVFP4>(a, mt, st);
    }
}

}  // namespace qg
