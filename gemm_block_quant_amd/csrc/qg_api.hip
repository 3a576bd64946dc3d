// qg_api.hip -- the C ABI of libquantgemm: host-side validation and dispatch.
// Nothing here allocates device memory or synchronizes a stream.
#include <limits.h>

#include <atomic>
#include <mutex>
#include <unordered_map>

#include "qg_stream.h"

using namespace qg;

namespace {

int64_t block_values(int fmt) {
    switch (fmt) {
        case QG_Q8_0: return 32;
        case QG_Q4_K: return 256;
        case QG_Q5_K: return 256;
        case QG_Q6_K: return 256;
        case QG_NVFP4: return 16;
        case QG_FP8: return 64;
        default: return 0;
    }
}

int64_t block_bytes(int fmt) {
    switch (fmt) {
        case QG_Q8_0: return 34;
        case QG_Q4_K: return 144;
        case QG_Q5_K: return 176;
        case QG_Q6_K: return 210;
        default: return 0;
    }
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Shape checks common to every product entry point.  K is capped at
// kMaxK so that every LDS size and offset the kernels derive from it fits in
// an int.
constexpr int64_t kMaxK = (int64_t)1 << 24;
qg_status check_shape(int fmt, int64_t E, int64_t N, int64_t K, int64_t M) {
    if (block_values(fmt) == 0) return QG_EFORMAT;
    if (E < 1 || N < 0 || M < 0 || K <= 0 || K % block_values(fmt)) return QG_ESHAPE;
    if (N > INT_MAX / 2 || K > kMaxK || M > INT_MAX / 2) return QG_ESHAPE;
    if (E > 0 && N > 0 && E > (int64_t)INT_MAX / N) return QG_ESHAPE;
    return QG_OK;
}

// The grouped product stages one activation row of the whole K in LDS.
qg_status check_grouped_k(int fmt, int64_t K) {
    return stream_lds_bytes(fmt, (int)K, 1) <= (size_t)kLdsBytes ? QG_OK : QG_ESHAPE;
}

// Streaming-kernel arguments for matrix e of a stacked weight[E*N, K].
StreamArgs stream_args(const void* w, int fmt, int64_t E, int64_t e, int64_t N, int64_t K) {
    StreamArgs a = {};
    const uint8_t* base = (const uint8_t*)w;
    const int64_t R = E * N;
    if (fmt == QG_NVFP4) {
        a.rb0 = K / 2;
        a.rb1 = K / 16;
        a.w0 = base + e * N * a.rb0;
        a.w1 = base + R * a.rb0 + e * N * a.rb1;
        a.gbytes = base + R * a.rb0 + R * a.rb1 + 4 * e;
    } else if (fmt == QG_FP8) {
        a.rb0 = K;  // codes
        a.rb1 = 4;  // one fp32 row scale
        a.w0 = base + e * N * a.rb0;
        a.w1 = base + R * a.rb0 + e * N * a.rb1;
    } else {
        a.rb0 = (K / block_values(fmt)) * block_bytes(fmt);
        a.w0 = base + e * N * a.rb0;
    }
    a.N = (int)N;
    a.K = (int)K;
    return a;
}

qg_status from_hip(hipError_t e) { return e == hipSuccess ? QG_OK : QG_EHIP; }

// Workspace regions of the mixture-of-experts block (256-byte aligned offsets).
struct MoeLayout {
    size_t gu, h, yd, gws, total;
};
MoeLayout moe_layout(int64_t E, int64_t P, int64_t D, int64_t F) {
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    MoeLayout L;
    size_t o = 0;
    L.gu = o;
    o += up((size_t)P * (size_t)F * 8);  // fp32 gate|up per pair
    L.h = o;
    o += up((size_t)P * (size_t)F * 2);  // bf16 SwiGLU per pair
    L.yd = o;
    o += up((size_t)P * (size_t)D * 4);  // fp32 down product per pair
    L.gws = o;
    o += up(grouped_workspace_bytes(E, P));
    L.total = o;
    return L;
}

// Shape checks of the block; P = T * topk pairs.
qg_status check_moe(int fmt_gu, int fmt_dn, int64_t E, int64_t D, int64_t F, int64_t T, int64_t topk) {
    if (block_values(fmt_gu) == 0 || block_values(fmt_dn) == 0) return QG_EFORMAT;
    if (E < 1 || D <= 0 || F <= 0 || T < 0 || topk < 1 || topk > kGroupedMaxRows) return QG_ESHAPE;
    if (T > kGroupedMaxRows / topk) return QG_ESHAPE;
    if (F > INT_MAX / 4) return QG_ESHAPE;
    qg_status s = check_shape(fmt_gu, E, 2 * F, D, T * topk);
    if (s != QG_OK) return s;
    s = check_shape(fmt_dn, E, D, F, T * topk);
    if (s != QG_OK) return s;
    s = check_grouped_k(fmt_gu, D);
    if (s != QG_OK) return s;
    return check_grouped_k(fmt_dn, F);
}

// Validation shared by the grouped entry points (everything but the workspace).
qg_status check_grouped(const void* w, int fmt, int64_t E, int64_t N, int64_t K, int64_t M, const uint16_t* x,
                        const int32_t* ids, float* y) {
    qg_status s = check_shape(fmt, E, N, K, M);
    if (s != QG_OK) return s;
    if (M > kGroupedMaxRows) return QG_ESHAPE;
    s = check_grouped_k(fmt, K);
    if (s != QG_OK) return s;
    if (M == 0 || N == 0) return QG_OK;
    if (!w || !x || !y) return QG_EINVAL;
    if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 4) || (ids && !aligned(ids, 4))) return QG_EALIGN;
    return QG_OK;
}

// The grouped product of a validated call with its bucketing workspace ws.
qg_status run_grouped(const void* w, int fmt, int64_t E, int64_t N, int64_t K, int64_t M, const uint16_t* x,
                      const int32_t* ids, float* y, void* ws, void* stream) {
    StreamArgs a = stream_args(w, fmt, E, 0, N, K);
    a.x = x;
    a.ldx = K;
    a.y = y;
    a.ldy = N;
    const int64_t es0 = N * a.rb0, es1 = N * a.rb1;
    return from_hip(launch_grouped(fmt, a, ids, E, M, (int32_t*)ws, es0, es1, (hipStream_t)stream));
}

}  // namespace

// Scratch of quant_grouped_gemm_noalloc: the bucketing workspace of the
// largest grouped call (16384 rows and as many slots: 5 + 2 * 16384 + 16384
// int32, then two tile lists of 2 * 16384 / 32 int32 each: 204,820 bytes),
// one copy per GPU for the life of the process.  In host code this name is
// only a handle for hipGetSymbolAddress: the device address of each GPU's copy
// is resolved once per device and used everywhere else.
static constexpr size_t kScratchBytes = 204832;
static_assert(kScratchBytes >= ((5 + 3 * kGroupedMaxRows + 4 * (kGroupedMaxRows / kMfmaMinRows)) * 4 + 15) / 16 * 16,
              "holds the largest bucketing");
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace qg {

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];  // CU count per device, 0 until queried

int current_device() {
    int dev = 0;
    return hipGetDevice(&dev) == hipSuccess ? dev : 0;
}

// Launch attributes and residencies per (device, kernel): the opt-in to the
// whole LDS is set once per kernel on each device, and residencies are cached
// per dynamic LDS size.
std::mutex g_fn_mu;
std::unordered_map<uint64_t, std::unordered_map<const void*, std::unordered_map<size_t, int>>> g_fn_cache;

// Looks up (creating it on first use) the residency map of fn on the current
// device; the caller holds g_fn_mu.
hipError_t fn_entry(const void* fn, std::unordered_map<size_t, int>** out) {
    auto& per_dev = g_fn_cache[(uint64_t)current_device()];
    auto it = per_dev.find(fn);
    if (it == per_dev.end()) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
        if (e != hipSuccess) return e;
        it = per_dev.emplace(fn, std::unordered_map<size_t, int>()).first;
    }
    *out = &it->second;
    return hipSuccess;
}
}  // namespace

int num_cus() {
    const int dev = current_device();
    if (dev >= 0 && dev < kMaxDevices) {
        const int n = g_cus[dev].load(std::memory_order_relaxed);
        if (n > 0) return n;
    }
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
        return 256;  // not cached: the next call asks again
    if (dev >= 0 && dev < kMaxDevices) g_cus[dev].store(v, std::memory_order_relaxed);
    return v;
}

hipError_t allow_full_lds(const void* fn) {
    std::lock_guard<std::mutex> lock(g_fn_mu);
    std::unordered_map<size_t, int>* m = nullptr;
    return fn_entry(fn, &m);
}

hipError_t kernel_residency(const void* fn, size_t lds, int* per_cu, int block) {
    std::lock_guard<std::mutex> lock(g_fn_mu);
    std::unordered_map<size_t, int>* m = nullptr;
    hipError_t e = fn_entry(fn, &m);
    if (e != hipSuccess) return e;
    // a kernel is always launched with the same block size, so LDS is the key
    auto jt = m->find(lds);
    if (jt != m->end()) {
        *per_cu = jt->second;
        return hipSuccess;
    }
    int fit = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&fit, fn, block, lds);
    if (e != hipSuccess) return e;
    if (fit < 1) fit = 1;
    m->emplace(lds, fit);
    *per_cu = fit;
    return hipSuccess;
}

namespace {
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];  // device address of `scratch` per device (null until resolved)
}  // namespace

}  // namespace qg

// Device address of the current device's copy of `scratch`, resolved on the
// first call for that device (with the device current) and kept.
static qg_status scratch_on_current_device(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= qg::kMaxDevices) return QG_EHIP;
    std::lock_guard<std::mutex> lock(qg::g_scratch_mu);
    if (!qg::g_scratch_dev[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return QG_EHIP;
        qg::g_scratch_dev[dev] = p;
    }
    *out = qg::g_scratch_dev[dev];
    return QG_OK;
}

namespace qg {

// Plain streaming read (measurement reference): 256-thread workgroups, eight
// per CU, striding over the buffer in blocks of eight 16-byte granules per
// thread, every granule once, non-temporal loads (the fastest of the shapes
// measured on MI355X: 100 MB in 16.4 us, 1 GiB at 7.0 TB/s; one 1024-thread
// workgroup per CU over a contiguous chunk took 17.1 us and 6.9 TB/s, and the
// same reads without the non-temporal hint top out at 6.15 TB/s).
constexpr int kProbeThreads = 256, kProbeUnroll = 8, kProbeWgsPerCu = 8;
__global__ __launch_bounds__(kProbeThreads) void k_read_probe(const u32x4* __restrict__ p, size_t n16,
                                                              uint32_t* sink) {
    constexpr size_t T = kProbeThreads, U = kProbeUnroll;
    const size_t stride = (size_t)gridDim.x * T * U;
    uint32_t acc = 0;
    size_t i = (size_t)blockIdx.x * T * U + threadIdx.x;
    for (; i + (U - 1) * T < n16; i += stride) {
        u32x4 v[U];
#pragma unroll
        for (size_t u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load((const QG_GLOBAL u32x4*)(p + i + u * T));
#pragma unroll
        for (size_t u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    // the one block that straddles the end (its workgroup's threads step by T)
    for (; i < n16; i += T) {
        const u32x4 v = __builtin_nontemporal_load((const QG_GLOBAL u32x4*)(p + i));
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x9E3779B9u) *sink = acc;  // keeps the loads; practically never taken
}

}  // namespace qg

extern "C" {

int64_t quant_block_values(qg_format fmt) { return block_values(fmt); }

size_t quant_packed_bytes(qg_format fmt, int64_t E, int64_t N, int64_t K) {
    const int64_t qk = block_values(fmt);
    if (qk == 0 || E < 0 || N < 0 || K < 0 || K % qk) return 0;
    const int64_t rows = E * N, blocks = rows * (K / qk);
    if (fmt == QG_NVFP4) return (size_t)(blocks * 9 + 4 * E);
    if (fmt == QG_FP8) return (size_t)(rows * K + 4 * rows);
    return (size_t)(blocks * block_bytes(fmt));
}

const char* quant_status_string(qg_status s) {
    switch (s) {
        case QG_OK: return "ok";
        case QG_EINVAL: return "null pointer argument";
        case QG_EFORMAT: return "unknown weight format tag";
        case QG_EALIGN: return "pointer not aligned as required (w, x, workspace: 16 bytes; y, ids: 4 bytes)";
        case QG_ESHAPE: return "invalid shape: negative size, K not a positive multiple of the block, or a limit exceeded";
        case QG_EHIP: return "HIP runtime error on launch";
        case QG_ENOTIMPL: return "not implemented for this combination";
        case QG_EWORKSPACE: return "workspace missing or too small";
        default: return "unknown status";
    }
}

qg_status quant_gemm(const void* w, qg_format fmt, int64_t N, int64_t K, int64_t M, const uint16_t* x, float* y,
                     void* stream) {
    qg_status s = check_shape(fmt, 1, N, K, M);
    if (s != QG_OK) return s;
    if (M == 0 || N == 0) return QG_OK;
    if (!w || !x || !y) return QG_EINVAL;
    if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 4)) return QG_EALIGN;
    StreamArgs a = stream_args(w, fmt, 1, 0, N, K);
    if (M >= kMfmaMinRows && (fmt == QG_NVFP4 || mfma_kquant_supported(fmt, (int)K))) {
        const bool tile = mfma_kquant_supported(fmt, (int)K);  // NVFP4 with K % 64 != 0: its own kernel
        // matrix-core tiles; rows in chunks that keep the grid's row-tile
        // count within its 65,535 limit (each row's result does not depend on
        // the other rows)
        constexpr int64_t kChunk = (int64_t)1 << 21;
        for (int64_t m0 = 0; m0 < M; m0 += kChunk) {
            const int cnt = (int)(M - m0 < kChunk ? M - m0 : kChunk);
            const uint16_t* xc = x + m0 * K;
            float* yc = y + m0 * N;
            const hipError_t e =
                !tile ? launch_mfma_nvfp4(a.w0, a.w1, a.gbytes, (int)N, (int)K, xc, K, cnt, yc, N, (hipStream_t)stream)
                      : launch_mfma_kquant(fmt, a.w0, a.w1, a.gbytes, (int)N, (int)K, xc, K, cnt, yc, N,
                                           (hipStream_t)stream);
            if (e != hipSuccess) return QG_EHIP;
        }
        return QG_OK;
    }
    const int rows = stream_rows_per_pass(fmt, N, (int)K, (int)(M < 16 ? M : 16));
    if (rows <= 0) return QG_ESHAPE;
    a.x = x;
    a.ldx = K;
    a.y = y;
    a.ldy = N;
    for (int64_t m0 = 0; m0 < M; m0 += rows) {
        const int cnt = (int)(M - m0 < rows ? M - m0 : rows);
        a.M = cnt;
        for (int i = 0; i < kMaxPassRows; ++i) {
            a.xrow[i] = (int)(m0 + (i < cnt ? i : 0));
            a.yrow[i] = a.xrow[i];
        }
        hipError_t e = launch_stream_gemm(fmt, a, (hipStream_t)stream);
        if (e != hipSuccess) return QG_EHIP;
    }
    return QG_OK;
}

qg_status quant_gemv(const void* w, qg_format fmt, int64_t N, int64_t K, const uint16_t* x, float* y, void* stream) {
    return quant_gemm(w, fmt, N, K, 1, x, y, stream);
}

// Workspace variant of quant_gemm: the workspace it needs (0 where quant_gemm's
// schedule is kept).  Up to 16 rows: the direct path with one K segment per
// workgroup where the plain launch would stage the activations in several K
// phases; from 32 rows: stream-K tiles where the plain grid is under-filled.
static size_t streamk_bytes(qg_format fmt, int64_t N, int64_t K, int64_t M) {
    if (check_shape(fmt, 1, N, K, M) != QG_OK || N == 0 || M < 2 || M > ((int64_t)1 << 21)) return 0;
    if (M <= kMaxPassRows) return direct_xseg_bytes(fmt, N, (int)K, (int)M);
    if (M < kMfmaMinRows) return 0;
    return mfma_streamk_bytes(fmt, (int)N, (int)K, (int)M);
}

size_t quant_gemm_streamk_workspace_bytes(qg_format fmt, int64_t N, int64_t K, int64_t M) {
    return streamk_bytes(fmt, N, K, M);
}

qg_status quant_gemm_streamk(const void* w, qg_format fmt, int64_t N, int64_t K, int64_t M, const uint16_t* x,
                             float* y, void* workspace, size_t workspace_bytes, void* stream) {
    const size_t need = streamk_bytes(fmt, N, K, M);
    if (need == 0) return quant_gemm(w, fmt, N, K, M, x, y, stream);
    if (!w || !x || !y) return QG_EINVAL;
    if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 4)) return QG_EALIGN;
    if (!workspace || workspace_bytes < need) return QG_EWORKSPACE;
    if (!aligned(workspace, 16)) return QG_EALIGN;
    if (M <= kMaxPassRows) {
        // passes of up to 8 rows (every row keeps its arithmetic whatever the pass)
        StreamArgs a = stream_args(w, fmt, 1, 0, N, K);
        a.x = x;
        a.ldx = K;
        a.y = y;
        a.ldy = N;
        for (int64_t m0 = 0; m0 < M; m0 += kXsegRows) {
            const int cnt = (int)(M - m0 < kXsegRows ? M - m0 : kXsegRows);
            a.M = cnt;
            for (int i = 0; i < kMaxPassRows; ++i) a.xrow[i] = a.yrow[i] = (int)(m0 + (i < cnt ? i : 0));
            if (launch_direct_xseg(fmt, a, workspace, (hipStream_t)stream) != hipSuccess) return QG_EHIP;
        }
        return QG_OK;
    }
    const StreamArgs a = stream_args(w, fmt, 1, 0, N, K);
    const hipError_t e = launch_mfma_kquant_streamk(fmt, a.w0, a.w1, a.gbytes, (int)N, (int)K, x, K, (int)M, y, N,
                                                    workspace, workspace_bytes, (hipStream_t)stream);
    return e == hipSuccess ? QG_OK : QG_EHIP;
}

size_t quant_grouped_workspace_bytes(int64_t E, int64_t M) {
    if (E < 1 || M < 0) return 0;
    return grouped_workspace_bytes(E, M);
}

qg_status quant_grouped_gemm(const void* w, qg_format fmt, int64_t E, int64_t N, int64_t K, int64_t M,
                             const uint16_t* x, const int32_t* ids, float* y, void* workspace, size_t workspace_bytes,
                             void* stream) {
    qg_status s = check_grouped(w, fmt, E, N, K, M, x, ids, y);
    if (s != QG_OK || M == 0 || N == 0) return s;
    if (!workspace || workspace_bytes < grouped_workspace_bytes(E, M)) return QG_EWORKSPACE;
    if (!aligned(workspace, 16)) return QG_EALIGN;
    return run_grouped(w, fmt, E, N, K, M, x, ids, y, workspace, stream);
}

qg_status quant_grouped_gemm_noalloc(const void* w, qg_format fmt, int64_t E, int64_t N, int64_t K, int64_t M,
                                     const uint16_t* x, const int32_t* ids, float* y, void* stream) {
    qg_status s = check_grouped(w, fmt, E, N, K, M, x, ids, y);
    if (s != QG_OK || M == 0 || N == 0) return s;
    if (grouped_workspace_bytes(E, M) > kScratchBytes) return QG_EWORKSPACE;
    void* ws = nullptr;
    s = scratch_on_current_device(&ws);
    if (s != QG_OK) return s;
    return run_grouped(w, fmt, E, N, K, M, x, ids, y, ws, stream);
}

size_t quant_moe_workspace_bytes(qg_format fmt_gate_up, qg_format fmt_down, int64_t E, int64_t D, int64_t F,
                                 int64_t T, int64_t topk) {
    if (check_moe(fmt_gate_up, fmt_down, E, D, F, T, topk) != QG_OK) return 0;
    return moe_layout(E, T * topk, D, F).total;
}

qg_status quant_moe_block(const void* w_gate_up, qg_format fmt_gate_up, const void* w_down, qg_format fmt_down,
                          int64_t E, int64_t D, int64_t F, int64_t T, int64_t topk, const uint16_t* x,
                          const int32_t* idx, const float* wts, float* y, void* workspace, size_t workspace_bytes,
                          void* stream) {
    qg_status s = check_moe(fmt_gate_up, fmt_down, E, D, F, T, topk);
    if (s != QG_OK) return s;
    if (T == 0) return QG_OK;
    if (!w_gate_up || !w_down || !x || !idx || !wts || !y) return QG_EINVAL;
    const int64_t P = T * topk;
    const MoeLayout L = moe_layout(E, P, D, F);
    if (!workspace || workspace_bytes < L.total) return QG_EWORKSPACE;
    if (!aligned(w_gate_up, 16) || !aligned(w_down, 16) || !aligned(x, 16) || !aligned(idx, 4) ||
        !aligned(wts, 4) || !aligned(y, 4) || !aligned(workspace, 16))
        return QG_EALIGN;
    hipStream_t st = (hipStream_t)stream;
    uint8_t* ws = (uint8_t*)workspace;
    float* gu = (float*)(ws + L.gu);
    uint16_t* h = (uint16_t*)(ws + L.h);
    float* yd = (float*)(ws + L.yd);
    int32_t* gws = (int32_t*)(ws + L.gws);
    // 1. gate|up of every (token, expert) pair p, reading token p / topk's
    // activations; each distinct expert's weights read once
    StreamArgs a = stream_args(w_gate_up, fmt_gate_up, E, 0, 2 * F, D);
    a.x = x;
    a.ldx = D;
    a.xdiv = (int)topk;
    a.y = gu;
    a.ldy = 2 * F;
    if (launch_grouped(fmt_gate_up, a, idx, E, P, gws, 2 * F * a.rb0, 2 * F * a.rb1, st) != hipSuccess)
        return QG_EHIP;
    // 2. SwiGLU, rounded to bf16
    if (launch_moe_swiglu(gu, h, (int)P, (int)F, st) != hipSuccess) return QG_EHIP;
    // 3. down products
    StreamArgs b = stream_args(w_down, fmt_down, E, 0, D, F);
    b.x = h;
    b.ldx = F;
    b.y = yd;
    b.ldy = D;
    // (the same ids: the bucketing of step 1 is reused)
    if (launch_grouped(fmt_down, b, idx, E, P, gws, D * b.rb0, D * b.rb1, st, false) != hipSuccess) return QG_EHIP;
    // 4. routing-weighted sum over each token's experts
    return from_hip(launch_moe_combine(yd, wts, idx, (int)E, y, (int)T, (int)topk, (int)D, st));
}

qg_status quant_dequantize_stacked(const void* w, qg_format fmt, int64_t E, int64_t N, int64_t K, float* out,
                                   void* stream) {
    qg_status s = check_shape(fmt, E, N, K, 0);
    if (s != QG_OK) return s;
    if (N == 0) return QG_OK;
    if (!w || !out) return QG_EINVAL;
    if (!aligned(w, 16) || !aligned(out, 4)) return QG_EALIGN;
    return from_hip(launch_dequant(fmt, (const uint8_t*)w, E, N, K, out, (hipStream_t)stream));
}

qg_status quant_dequantize(const void* w, qg_format fmt, int64_t rows, int64_t K, float* out, void* stream) {
    return quant_dequantize_stacked(w, fmt, 1, rows, K, out, stream);
}

qg_status quant_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    if (!buf || !sink) return QG_EINVAL;
    if (!aligned(buf, 16) || !aligned(sink, 4)) return QG_EALIGN;
    if (bytes % 16) return QG_ESHAPE;
    if (bytes == 0) return QG_OK;
    const size_t n16 = bytes / 16;
    size_t grid = (size_t)qg::num_cus() * qg::kProbeWgsPerCu;
    const size_t blocks = (n16 + qg::kProbeThreads * qg::kProbeUnroll - 1) / (qg::kProbeThreads * qg::kProbeUnroll);
    if (grid > blocks) grid = blocks;
    hipLaunchKernelGGL(qg::k_read_probe, dim3((unsigned)grid), dim3(qg::kProbeThreads), 0, (hipStream_t)stream,
                       (const qg::u32x4*)buf, n16, sink);
    return from_hip(hipGetLastError());
}

}  // extern "C"
