// qg_grouped.hip -- grouped-expert product over a stacked weight[E*N, K]:
//     y[i, :] = W_{ids[i]} x[i, :],  W_e = rows [e*N, (e+1)*N)
// (the operator seam of vllm.cpp issue #3030 "BACKEND-TENSTORRENT-KEEPQUANT",
// section "Second falsification": E = 1 is the dense case, E = N the stacked
// expert tower).
//
// Rows are bucketed by expert on the device first, so that each DISTINCT
// expert's weights stream from HBM once per call however many rows route to
// it.  "A 320B MoE on a free Kaggle TPU" (section "The decode kernel's cost is
// not distinct experts") shows a decode path that runs one grid step per
// (token, expert) pair instead, re-reading and re-decoding an expert for every
// pair that selects it; its prefill path sorts slots by expert, which is what
// the bucketing kernel below does.
//
//  1. k_bucket (one workgroup): group the rows by expert id -- a counting sort
//     for calls of more than 128 rows, else a bitonic sort of the keys
//     (id << 32 | row) -- with invalid ids last, and write slot -> (expert,
//     first sorted row) and the sorted row list.  Rows whose id is outside
//     [0, E) get NaN in every element of y.
//     When the call has at least 4 rows per possible distinct expert it also
//     lists the row tiles of the experts with at least kMfmaMinRows rows, for
//     64- and for 128-row tiles.
//  2. k_grouped: workgroup (slot, chunk) stages the slot's activation rows
//     (16 at most per pass) in LDS and its 4 waves stream rows [chunk*RPC,
//     ...) of the slot's expert through the same core as the dense product,
//     writing y rows at the original row indices.  Workgroups whose slot is
//     past the number of distinct experts exit at once, and so do those of a
//     slot that the matrix-core tiles take.
//  3. Experts with at least kMfmaMinRows rows (where the format has a tile
//     path): the dense product's matrix-core tile kernel over the listed row
//     tiles, each reading its expert's weights once per tile of rows, not once
//     per 16 rows ("Qwen3.8-27B on one Tenstorrent P150", section "3. Porting
//     the 9B stack to 27B geometry").
// The per-row arithmetic is the dense kernel's, so E = 1 with ids = NULL
// reproduces quant_gemm bit for bit.
#include <climits>
#include <type_traits>

#include "qg_direct.h"

namespace qg {

constexpr int kBucketThreads = 1024;

// Workspace (int32): [0] slot count, [1] and [2] the number of 64- and of
// 128-row tiles listed, [4 .. 4+S) slot expert, [4+S .. 5+2S) slot start, then
// M sorted rows, then the two tile lists (64-row tiles first), each entry the
// pair (first sorted row, slot).  S = min(E, M).  A slot of c >= kMfmaMinRows
// rows has ceil(c / 64) <= c / kMfmaMinRows tiles, so a list holds at most
// M / kMfmaMinRows entries.
__host__ __device__ inline int64_t ws_slots(int64_t E, int64_t M) { return E < M ? E : M; }
__host__ __device__ inline int64_t ws_tile_cap(int64_t M) { return M / kMfmaMinRows; }
// int offset of the list of bm-row tiles (bm 64 or 128)
__host__ __device__ inline int64_t ws_tile_list(int64_t E, int64_t M, int bm) {
    return 5 + 2 * ws_slots(E, M) + M + (bm == 128 ? 2 * ws_tile_cap(M) : 0);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int d) {
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, d, 64);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), d, 64);
    return ((uint64_t)hi << 32) | lo;
}

// Counting sort by expert id (calls with E <= kCountMaxExperts):
// one LDS counter per id (and one for invalid ids, bin E); each row takes its
// rank inside its bin from an LDS atomic, the bins' exclusive scan gives the
// slots and their starts, and each row lands at start + rank.  The order of the
// rows inside a bin follows the atomics and can differ from call to call; no
// result depends on it (every row's arithmetic is independent of which rows
// share its pass or tile).  Rows with invalid ids sort last and get NaN rows.
// Writes ws[0], the slots and the permutation; part: 16 ints of LDS.
constexpr int kCountMaxExperts = 16384;
__device__ __forceinline__ void bucket_by_counting(const int32_t* __restrict__ ids, int E, int M,
                                                   int32_t* __restrict__ ws, float* __restrict__ y, int N,
                                                   int64_t ldy, QG_LDS int32_t* hist, QG_LDS int32_t* part) {
    constexpr int R = kGroupedMaxRows / kBucketThreads;  // rows per thread at most
    const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wv = tid >> 6;
    const int64_t S = ws_slots(E, M);
    int32_t* slot_expert = ws + 4;
    int32_t* slot_start = ws + 4 + S;
    int32_t* perm = ws + 5 + 2 * S;
    for (int b = tid; b <= E; b += nt) hist[b] = 0;
    __syncthreads();
    int key[R], rank[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = tid + r * nt;
        key[r] = E;
        rank[r] = 0;
        if (i < M) {
            const int id = ids ? ids[i] : 0;
            key[r] = (id >= 0 && id < E) ? id : E;
            rank[r] = __hip_atomic_fetch_add(hist + key[r], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
    }
    __syncthreads();
    // exclusive scan over the E + 1 bins of (rows, non-empty valid bins), packed
    // as rows | bins << 16 (each total at most 16384)
    const int per = (E + 1 + nt - 1) / nt;
    const int b0 = tid * per, b1 = min(E + 1, b0 + per);
    int cnt = 0;
    for (int b = b0; b < b1; ++b) {
        const int c = hist[b];
        cnt += c | ((b < E && c > 0) ? 1 << 16 : 0);
    }
    int inc = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(inc, d, 64);
        if (lane >= d) inc += v;
    }
    if (lane == 63) part[wv] = inc;
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int t = 0; t < nt / 64; ++t) {
            const int c = part[t];
            part[t] = run;
            run += c;
        }
        ws[0] = run >> 16;
    }
    __syncthreads();
    int off = (part[wv] + inc - cnt) & 0xFFFF, slot = (part[wv] + inc - cnt) >> 16;
    for (int b = b0; b < b1; ++b) {
        const int c = hist[b];
        hist[b] = off;
        if (b < E && c > 0) {
            slot_expert[slot] = b;
            slot_start[slot] = off;
            ++slot;
        }
        if (b == E) slot_start[slot] = off;  // the last slot ends where the invalid rows start
        off += c;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = tid + r * nt;
        if (i < M) perm[hist[key[r]] + rank[r]] = i;
    }
    // NaN rows for ids outside [0, E): the last sorted positions
    __syncthreads();
    const int valid = hist[E];
    for (int p = valid; p < M; ++p) {
        const int row = perm[p];
        for (int n = tid; n < N; n += nt) y[(int64_t)row * ldy + n] = __builtin_nanf("");
    }
}

// P: sort keys, a power of two >= max(M, 128); P == 128 sorts in one wave's
// registers; P == 0: counting sort (bucket_by_counting).
// lists: also list the row tiles of the slots with at least kMfmaMinRows rows
// (else their counts are 0).
__global__ __launch_bounds__(kBucketThreads) void k_bucket(const int32_t* __restrict__ ids, int E, int M, int P,
                                                           int32_t* __restrict__ ws, float* __restrict__ y, int N,
                                                           int64_t ldy, int lists) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem_generic[];
    const int tid = threadIdx.x, nt = blockDim.x;  // nt: a multiple of 64, at most kBucketThreads
    const int lane = tid & 63, wv = tid >> 6;
    const int64_t S = ws_slots(E, M);
    int32_t* slot_start = ws + 4 + S;
    int32_t* perm = ws + 5 + 2 * S;
    QG_LDS int32_t* part;
    if (P == 0) {
        QG_LDS int32_t* hist = (QG_LDS int32_t*)smem_generic;  // E + 1 bins
        part = hist + ((E + 1 + 3) & ~3);
        bucket_by_counting(ids, E, M, ws, y, N, ldy, hist, part);
    } else {
        QG_LDS uint64_t* keys = (QG_LDS uint64_t*)smem_generic;  // P keys
        part = (QG_LDS int32_t*)(smem_generic + (size_t)P * 8);  // per-wave partial counts
        int32_t* slot_expert = ws + 4;

        for (int i = tid; i < P; i += nt) {
            uint64_t k = ~0ull;
            if (i < M) {
                const int id = ids ? ids[i] : 0;
                const uint32_t hi = (id >= 0 && id < E) ? (uint32_t)id : 0x7fffffffu;
                k = ((uint64_t)hi << 32) | (uint32_t)i;
            }
            keys[i] = k;
        }
        __syncthreads();
        if (P == 128) {
            // one wave (nt == 64): keys 2 t and 2 t + 1 in lane t's registers and
            // the same bitonic network by lane shuffles (no barriers)
            uint64_t k0 = keys[2 * tid], k1 = keys[2 * tid + 1];
            for (int size = 2; size <= P; size <<= 1) {
                for (int stride = size >> 1; stride > 0; stride >>= 1) {
                    const bool up = ((2 * tid) & size) == 0;
                    if (stride == 1) {
                        if ((k0 > k1) == up) {
                            const uint64_t t = k0;
                            k0 = k1;
                            k1 = t;
                        }
                    } else {
                        // partner of position 2 t + e is 2 (t ^ d) + e, d = stride / 2
                        const int d = stride >> 1;
                        const uint64_t p0 = shfl_xor_u64(k0, d), p1 = shfl_xor_u64(k1, d);
                        const bool keep_min = ((tid & d) == 0) == up;  // lower position of an ascending pair, or upper of a descending one
                        k0 = keep_min ? (k0 < p0 ? k0 : p0) : (k0 > p0 ? k0 : p0);
                        k1 = keep_min ? (k1 < p1 ? k1 : p1) : (k1 > p1 ? k1 : p1);
                    }
                }
            }
            keys[2 * tid] = k0;
            keys[2 * tid + 1] = k1;
            __syncthreads();
        } else {
            // bitonic sort in LDS, ascending
            for (int size = 2; size <= P; size <<= 1) {
                for (int stride = size >> 1; stride > 0; stride >>= 1) {
                    for (int i = tid; i < P / 2; i += nt) {
                        const int lo = 2 * i - (i & (stride - 1));
                        const int hi = lo + stride;
                        const bool up = (lo & size) == 0;
                        const uint64_t a = keys[lo], b = keys[hi];
                        if ((a > b) == up) {
                            keys[lo] = b;
                            keys[hi] = a;
                        }
                    }
                    __syncthreads();
                }
            }
        }
        // heads of runs of equal valid ids -> slots (block scan over contiguous chunks)
        const int per = (M + nt - 1) / nt;
        const int b0 = tid * per, b1 = min(M, b0 + per);
        int cnt = 0;
        for (int i = b0; i < b1; ++i) {
            const uint32_t id = (uint32_t)(keys[i] >> 32);
            const bool valid = id != 0x7fffffffu;
            const bool head = valid && (i == 0 || (uint32_t)(keys[i - 1] >> 32) != id);
            cnt += head;
        }
        // exclusive scan of the counts: inclusive within each wave (shuffles),
        // then the waves' totals in order
        int inc = cnt;
    #pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(inc, d, 64);
            if (lane >= d) inc += v;
        }
        if (lane == 63) part[wv] = inc;
        __syncthreads();
        if (tid == 0) {
            int run = 0;
            for (int t = 0; t < nt / 64; ++t) {
                const int c = part[t];
                part[t] = run;
                run += c;
            }
            ws[0] = run;
        }
        __syncthreads();
        int slot = part[wv] + inc - cnt;
        for (int i = b0; i < b1; ++i) {
            const uint64_t k = keys[i];
            const uint32_t id = (uint32_t)(k >> 32);
            const bool valid = id != 0x7fffffffu;
            const bool head = valid && (i == 0 || (uint32_t)(keys[i - 1] >> 32) != id);
            perm[i] = (int32_t)(uint32_t)k;
            if (head) {
                slot_expert[slot] = (int32_t)id;
                slot_start[slot] = i;
                ++slot;
            }
        }
        if (tid == 0) {
            // the last slot ends at the first invalid sorted position (or M)
            int lo = 0, hi = M;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if ((uint32_t)(keys[mid] >> 32) == 0x7fffffffu) hi = mid;
                else lo = mid + 1;
            }
            slot_start[ws[0]] = lo;
        }
        // NaN rows for ids outside [0, E)
        for (int i = M - 1; i >= 0; --i) {
            if ((uint32_t)(keys[i] >> 32) != 0x7fffffffu) break;
            const int row = (int)(uint32_t)keys[i];
            for (int n = tid; n < N; n += nt) y[(int64_t)row * ldy + n] = __builtin_nanf("");
        }
    }  // bitonic
    // row tiles of the slots with at least kMfmaMinRows rows: per thread a
    // contiguous run of slots; 64-row counts in the low and 128-row counts in
    // the high half of one scanned word (each total is at most M / 32)
    __syncthreads();  // every slot start (and ws[0]) is written
    const int nslots = lists ? ws[0] : 0;
    const int sper = (nslots + nt - 1) / nt;
    const int s0 = tid * sper, s1 = min(nslots, s0 + sper);
    int tcnt = 0;
    for (int q = s0; q < s1; ++q) {
        const int c = slot_start[q + 1] - slot_start[q];
        if (c >= kMfmaMinRows) tcnt += ((c + 63) >> 6) | (((c + 127) >> 7) << 16);
    }
    int tinc = tcnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(tinc, d, 64);
        if (lane >= d) tinc += v;
    }
    if (lane == 63) part[wv] = tinc;
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int t = 0; t < nt / 64; ++t) {
            const int c = part[t];
            part[t] = run;
            run += c;
        }
        ws[1] = run & 0xFFFF;
        ws[2] = run >> 16;
    }
    __syncthreads();
    {
        const int first = part[wv] + tinc - tcnt;
        int o64 = first & 0xFFFF, o128 = first >> 16;
        int32_t* list64 = perm + M;
        int32_t* list128 = list64 + 2 * ws_tile_cap(M);
        for (int q = s0; q < s1; ++q) {
            const int r0 = slot_start[q], c = slot_start[q + 1] - r0;
            if (c < kMfmaMinRows) continue;
            for (int r = 0; r < c; r += 64, ++o64) {
                list64[2 * o64] = r0 + r;
                list64[2 * o64 + 1] = q;
            }
            for (int r = 0; r < c; r += 128, ++o128) {
                list128[2 * o128] = r0 + r;
                list128[2 * o128 + 1] = q;
            }
        }
    }
}

// Grouped streaming kernel.  MTMAX: activation rows per pass (LDS sized for
// it); DIRECT: register-direct streaming (Q4_K, Q5_K, Q6_K, NVFP4 with K % 64 == 0) with SP
// passes per ring slot, else the LDS row-buffer path with CPL/CPLS chunks.
// Slots of tile_min rows or more are left to the matrix-core tiles.
template <int F, int MTMAX, bool DIRECT, int CPL, int CPLS, int SP, int PF>
__global__ __launch_bounds__(256) void k_grouped(const StreamArgs a, const int32_t* __restrict__ ws, int64_t E,
                                                 int64_t M, int rpc, int nchunks, int64_t estride0,
                                                 int64_t estride1, int tile_min) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem_generic[];
    lds_u8* smem = (lds_u8*)smem_generic;
    const int K = a.K;
    const int slot = blockIdx.x / nchunks, chunk = blockIdx.x % nchunks;
    const int nslots = ws[0];
    if (slot >= nslots) return;  // uniform across the workgroup: no barrier is skipped by part of it
    const int64_t S = ws_slots(E, M);
    const int e = ws[4 + slot];
    const int r0 = ws[4 + S + slot], r1 = ws[4 + S + slot + 1];
    if (r1 - r0 >= tile_min) return;  // uniform: the tile kernel takes this slot
    const int32_t* perm = ws + 5 + 2 * S;

    lds_u8* xl = smem;
    lds_f32* xs = (lds_f32*)(smem + (DIRECT ? (size_t)direct_mg(MTMAX) * direct_mg_bytes(F, K) : (size_t)MTMAX * K * 2));
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    lds_u8* rowbuf = smem + rowbuf_offset(MTMAX, K) + (size_t)wid * rowbuf_bytes(CPL, CPLS);
    lds_u8* rowbuf_s = rowbuf + CPL * 1024 + 32;

    MatView mv;
    mv.w0 = a.w0 + (size_t)e * estride0;
    mv.rb0 = a.rb0;
    mv.w1 = a.w1 ? a.w1 + (size_t)e * estride1 : nullptr;
    mv.rb1 = a.rb1;
    mv.gbytes = a.gbytes ? a.gbytes + 4 * (size_t)e : nullptr;
    const int n_begin = chunk * rpc;
    const int n_end = min(a.N, n_begin + rpc);

    for (int p0 = r0; p0 < r1; p0 += MTMAX) {
        const int cnt = min(MTMAX, r1 - p0);
        if (p0 != r0) __syncthreads();  // every wave is done with the previous pass's activations
        const int li = DIRECT ? direct_out_slot(lane) : lane;
        const int64_t yrow = perm[p0 + (li < cnt ? li : 0)];
        const int xdiv = a.xdiv > 1 ? a.xdiv : 1;
        auto row_of = [&](int m) { return perm[p0 + m] / xdiv; };
        auto run = [&](auto mt_tag) {
            constexpr int MT = decltype(mt_tag)::value;
            if constexpr (DIRECT) {
                constexpr int RW = kDirectRows;
                // rpc is a multiple of RW, so row groups never straddle chunks; the
                // workgroup's waves take its (row group, K segment) items round robin
                const Segments sg{a.seg_S > 0 ? a.seg_S : 1, a.seg_PS > 0 ? a.seg_PS : 1};
                const int rg0 = n_begin / RW, rgs = (n_end - n_begin + RW - 1) / RW;
                SegLds sl{};
                sl.progress = (QG_LDS int*)(xl + direct_lds_bytes(F, MTMAX, K));
                sl.total = (lds_f32*)((lds_u8*)sl.progress + ((size_t)rgs * 4 + 15) / 16 * 16);
                sl.mtmax = MT;
                if (sg.S > 1)
                    for (int i = threadIdx.x; i < rgs; i += blockDim.x) sl.progress[i] = 0;
                XStage<F, MT, 1> xst;
                xst.issue(a.x, a.ldx, cnt, K, row_of);
                auto between = [&] { xst.commit(xl, xs, a.x, a.ldx, cnt, K, row_of); };
                const int items = rgs * sg.S;  // one phase: the whole row
                int next = wid;
                auto next_item = [&]() {
                    const int t = next;
                    next += kWavesPerBlock;
                    return t < items ? t : -1;
                };
                const Phase ph{0, sg.S, 0, K};
                wave_stream_direct<F, MT, SP, PF, true>(mv, n_end, K, xl, xs, next_item, rg0, sg, ph, sl, a.y, a.ldy,
                                                  yrow, cnt, between);
            } else {
                auto stage = [&] { stage_x<MT>(xl, a.x, a.ldx, cnt, K, row_of); };
                wave_stream<F, MT, CPL, CPLS, PF>(mv, K, a.seg_blocks, a.nseg, xl, rowbuf, rowbuf_s, n_begin + wid,
                                                  kWavesPerBlock, n_end, a.y, a.ldy, yrow, cnt, stage);
            }
        };
        if (cnt <= 1 || MTMAX == 1) run(std::integral_constant<int, 1>{});
        else if (cnt <= 2 || MTMAX == 2) run(std::integral_constant<int, (MTMAX < 2 ? MTMAX : 2)>{});
        else if (cnt <= 4 || MTMAX == 4) run(std::integral_constant<int, (MTMAX < 4 ? MTMAX : 4)>{});
        else if (cnt <= 8 || MTMAX == 8) run(std::integral_constant<int, (MTMAX < 8 ? MTMAX : 8)>{});
        else run(std::integral_constant<int, MTMAX>{});
    }
}

size_t grouped_workspace_bytes(int64_t E, int64_t M) {
    const int64_t ints = ws_tile_list(E, M, 128) + 2 * ws_tile_cap(M);
    return (size_t)((ints * 4 + 15) / 16 * 16);
}

// lds: the kernel's LDS; seg_mt > 0: the register-direct path, whose chunks
// are kept short (many workgroups keep the CUs evenly busy over the live
// experts), with LDS for the K-segment sums of a chunk when rows are cut into
// segments.
template <class Kern>
static hipError_t launch_grouped_one(Kern kern, size_t lds, const StreamArgs& a, const int32_t* ws, int64_t E,
                                     int64_t M, int64_t estride0, int64_t estride1, int tile_min, hipStream_t st,
                                     int seg_mt = 0) {
    int fit = 0;
    hipError_t e = kernel_residency((const void*)kern, lds, &fit);
    if (e != hipSuccess) return e;
    // enough (slot, chunk) workgroups to fill the chip even when only a few slots are live
    const int64_t S = ws_slots(E, M);
    const int64_t target = (int64_t)num_cus() * fit;
    int64_t nchunks = (target + S - 1) / S;
    const int64_t max_chunks = (a.N + 63) / 64;  // at least 16 rows per wave
    if (nchunks > max_chunks) nchunks = max_chunks;
    if (nchunks < 1) nchunks = 1;
    int rpc = (int)((a.N + nchunks - 1) / nchunks);
    rpc = (rpc + 3) & ~3;  // a multiple of every rows-per-wave (1, 2, 4)
    const bool split = seg_mt > 0 && a.seg_S > 1;
    // register-direct path: chunks of at most 32 row groups when rows are
    // whole (measured against 8, 16 and 64 on the 288-expert layers), 16 when
    // they are cut into K segments (their sums take LDS per row group)
    const int rpc_max = split ? 4 * kDirectSegRgsMax : 128;
    if (seg_mt > 0 && rpc > rpc_max) rpc = rpc_max;
    nchunks = (a.N + rpc - 1) / rpc;
    if (split) lds += direct_seg_lds_bytes(a.seg_S, rpc / 4, seg_mt);
    hipLaunchKernelGGL(kern, dim3((unsigned)(S * nchunks)), dim3(256), lds, st, a, ws, E, M, rpc, (int)nchunks,
                       estride0, estride1, tile_min);
    return hipGetLastError();
}

template <int F, int MTMAX>
static hipError_t grouped_paths(StreamArgs a, const int32_t* ws, int64_t E, int64_t M, int64_t es0, int64_t es1,
                                int tm, hipStream_t st) {
    if constexpr (F == QG_Q4_K || F == QG_Q5_K || F == QG_Q6_K || F == QG_NVFP4 || F == QG_FP8) {
        if (direct_eligible(F, a.K)) {
            // E = 1 splits rows exactly as the dense product does (so the two
            // agree bit for bit); stacked experts give enough row groups to
            // fill the CUs without cutting rows along K (8 % faster on the
            // 288-expert layers than with one expert's split)
            const int P = (a.K / 64 + kDirectSlots - 1) / kDirectSlots;
            const Segments sg = E > 1 ? Segments{1, P} : direct_segments(F, a.N, a.K, num_cus());
            a.seg_S = sg.S;
            a.seg_PS = sg.PS;
            const size_t lds = direct_lds_bytes(F, MTMAX, a.K);
            constexpr int SP = 1, PF = 3;
            return launch_grouped_one(k_grouped<F, MTMAX, true, 1, 0, SP, PF>, lds, a, ws, E, M, es0, es1, tm, st,
                                      MTMAX);
        }
    }
    if constexpr (F == QG_Q8_0 || F == QG_NVFP4) {
        const int cpl = choose_cpl(F, a.K);
        a.seg_blocks = segment_blocks(F, a.K, cpl);
        const int nb = a.K / BlockGeom<F>::QK;
        a.nseg = (nb + a.seg_blocks - 1) / a.seg_blocks;
        constexpr int S = (F == QG_NVFP4) ? 1 : 0;
        const size_t lds = gemv_lds_bytes(MTMAX, a.K, cpl, S);
        switch (cpl) {
            case 1: return launch_grouped_one(k_grouped<F, MTMAX, false, 1, S, 1, 4>, lds, a, ws, E, M, es0, es1, tm, st);
            case 2: return launch_grouped_one(k_grouped<F, MTMAX, false, 2, S, 1, 4>, lds, a, ws, E, M, es0, es1, tm, st);
            case 3: return launch_grouped_one(k_grouped<F, MTMAX, false, 3, S, 1, 4>, lds, a, ws, E, M, es0, es1, tm, st);
            case 4: return launch_grouped_one(k_grouped<F, MTMAX, false, 4, S, 1, 3>, lds, a, ws, E, M, es0, es1, tm, st);
            default: return launch_grouped_one(k_grouped<F, MTMAX, false, 6, S, 1, 2>, lds, a, ws, E, M, es0, es1, tm, st);
        }
    }
    return hipErrorInvalidValue;
}

template <int F>
static hipError_t grouped_mt(const StreamArgs& a, int mtmax, const int32_t* ws, int64_t E, int64_t M, int64_t es0,
                             int64_t es1, int tm, hipStream_t st) {
    switch (mtmax) {
        case 1: return grouped_paths<F, 1>(a, ws, E, M, es0, es1, tm, st);
        case 2: return grouped_paths<F, 2>(a, ws, E, M, es0, es1, tm, st);
        case 4: return grouped_paths<F, 4>(a, ws, E, M, es0, es1, tm, st);
        case 8: return grouped_paths<F, 8>(a, ws, E, M, es0, es1, tm, st);
        default: return grouped_paths<F, 16>(a, ws, E, M, es0, es1, tm, st);
    }
}

hipError_t launch_grouped(int fmt, const StreamArgs& a, const int32_t* ids, int64_t E, int64_t M, int32_t* ws,
                          int64_t estride0, int64_t estride1, hipStream_t st, bool bucket) {
    // 1. bucketing: a counting sort by id (a bitonic sort of 16,384 keys took
    // 176 us; at 128 rows the counting sort also measured 1.5 % faster per
    // grouped call), or for more than kCountMaxExperts experts a bitonic sort
    // of (id, row) keys (one wave up to 128 rows)
    int P = 128;
    while (P < M) P <<= 1;
    // one thread per compare-exchange of the sort (P / 2), whole waves, 64..1024
    int nt = P / 2 < 64 ? 64 : (P / 2 > kBucketThreads ? kBucketThreads : P / 2);
    size_t lds = (size_t)P * 8 + (kBucketThreads / 64) * 4;
    if (E <= kCountMaxExperts) {
        P = 0;
        // one thread per row, whole waves (1024 threads at 128 rows: 1.5 % slower)
        nt = M <= 64 ? 64 : M >= kBucketThreads ? kBucketThreads : (int)((M + 63) / 64 * 64);
        lds = (size_t)((E + 1 + 3) & ~3) * 4 + (kBucketThreads / 64) * 4;
    }
    {
        hipError_t e = allow_full_lds((const void*)k_bucket);
        if (e != hipSuccess) return e;
    }
    // Row-tile lists only where an expert may plausibly reach kMfmaMinRows rows:
    // at least 4 rows per possible distinct expert on average (a decode batch,
    // 128 rows over 288 experts, skips the lists and the tile launch; any expert
    // that still has that many rows then streams in passes of 16).  The choice
    // depends on (E, M) only, so a bucketing reused by a later call (bucket ==
    // false, same ids) matches that call's choice.
    const int64_t S = ws_slots(E, M);
    const bool lists = M >= kMfmaMinRows && M >= 4 * S;
    if (bucket) {
        hipLaunchKernelGGL(k_bucket, dim3(1), dim3(nt), lds, st, ids, (int)E, (int)M, P, ws, a.y, a.N, a.ldy,
                           (int)lists);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // 2. the matrix-core tiles take the experts with at least kMfmaMinRows rows
    const bool tiles = lists && mfma_kquant_supported(fmt, a.K);
    const int tm = tiles ? kMfmaMinRows : INT_MAX;
    if (tiles) {
        // tile height from the mean rows per distinct expert
        const int bm = M / S >= 128 ? 128 : 64;
        KqGroup g;
        g.ws = ws;
        g.S = (int)S;
        g.list = (int)ws_tile_list(E, M, bm);
        g.count = bm == 128 ? 2 : 1;
        g.cap = (int)ws_tile_cap(M);
        g.es0 = estride0;
        g.es1 = estride1;
        g.xdiv = a.xdiv > 1 ? a.xdiv : 1;
        hipError_t e = launch_mfma_kquant_grouped(fmt, a.w0, a.w1, a.gbytes, a.N, a.K, a.x, a.ldx, a.y, a.ldy, g,
                                                  bm, st);
        if (e != hipSuccess) return e;
    }
    // 3. rows per pass of the streaming kernel: room for the expected rows per
    // distinct expert (twice the mean, at least 4, below the tiles' threshold),
    // as LDS allows.  At least 4: a decode batch (128 rows over 288 experts)
    // has a few experts with 3 or 4 rows, each read twice in passes of 2 (the
    // MoE layer 328 -> 318 us with passes of up to 4)
    int64_t want = 2 * ((M + S - 1) / S);
    int mtmax = want <= 4 ? 4 : want <= 8 ? 8 : 16;
    while (mtmax > 1 && stream_lds_bytes(fmt, a.K, mtmax) > (size_t)kLdsBytes) mtmax >>= 1;
    switch (fmt) {
        case QG_Q8_0: return grouped_mt<QG_Q8_0>(a, mtmax, ws, E, M, estride0, estride1, tm, st);
        case QG_Q4_K: return grouped_mt<QG_Q4_K>(a, mtmax, ws, E, M, estride0, estride1, tm, st);
        case QG_Q5_K: return grouped_mt<QG_Q5_K>(a, mtmax, ws, E, M, estride0, estride1, tm, st);
        case QG_Q6_K: return grouped_mt<QG_Q6_K>(a, mtmax, ws, E, M, estride0, estride1, tm, st);
        case QG_FP8: return grouped_mt<QG_FP8>(a, mtmax, ws, E, M, estride0, estride1, tm, st);
        default: return grouped_mt<QG_NVFP4>(a, mtmax, ws, E, M, estride0, estride1, tm, st);
    }
}

}  // namespace qg
