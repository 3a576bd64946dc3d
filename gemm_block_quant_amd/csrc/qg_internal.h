// qg_internal.h -- declarations shared by the kernel files and the C-ABI layer.
#pragma once

#include "../../include/quantgemm.h"
#include "qg_common.h"

namespace qg {

constexpr int kMaxPassRows = 16;

// One launch of the weight-streaming kernel: rows [0, N) of one weight matrix
// times up to 16 activation rows.
struct StreamArgs {
    const uint8_t* w0;   // row 0 of the matrix: blocks (Q8_0/Q4_K/Q6_K) or E2M1 codes (NVFP4)
    int64_t rb0;         // bytes per row in that plane
    const uint8_t* w1;   // NVFP4: row 0 of the E4M3 scale plane
    int64_t rb1;         // NVFP4: scale bytes per row
    const uint8_t* gbytes;  // NVFP4: device address of the matrix's fp32 tensor scale (any alignment)
    int N, K;
    int seg_blocks, nseg;  // row-buffer path: filled by the dispatcher
    int seg_S, seg_PS;     // direct path: K segments per row and passes per segment
    int phases;            // direct path: K phases of staged activations (1: the whole row)
    const uint16_t* x;   // activations (bf16 bits); row m of this pass is x + xrow[m] * ldx
    int64_t ldx;
    float* y;            // output; row m of this pass is y + yrow[m] * ldy
    int64_t ldy;
    int M;               // activation rows in this pass (1..16)
    int xdiv;            // grouped product: row i of the call reads activation row i / xdiv (0 or 1: i)
    int xrow[kMaxPassRows];
    int yrow[kMaxPassRows];
    // direct path with each workgroup on one K segment: per (row group,
    // segment) sums and per-row-group counters (zero on entry); null otherwise
    float* xs_part;
    int32_t* xs_cnt;
};

hipError_t launch_stream_gemm(int fmt, StreamArgs a, hipStream_t st);
// The direct path with each workgroup on one K segment, for calls of 5..16
// rows whose activations would otherwise be staged in several K phases: the
// workspace it needs (0: not taken), and the launch of one pass of up to
// kXsegRows rows (ws of at least that many bytes, 16-byte aligned).
constexpr int kXsegRows = 8;
size_t direct_xseg_bytes(int fmt, int64_t N, int K, int M);
hipError_t launch_direct_xseg(int fmt, StreamArgs a, void* ws, hipStream_t st);
int stream_rows_per_pass(int fmt, int64_t N, int K, int M);
size_t stream_lds_bytes(int fmt, int K, int mt);

// Grouped-expert product: bucketing + streaming over the distinct experts.
constexpr int64_t kGroupedMaxRows = 16384;
size_t grouped_workspace_bytes(int64_t E, int64_t M);
// bucket == false: ws already holds the bucketing of these ids (an earlier call
// on the same stream); rows with invalid ids are then left unwritten.
hipError_t launch_grouped(int fmt, const StreamArgs& a, const int32_t* ids, int64_t E, int64_t M, int32_t* ws,
                          int64_t estride0, int64_t estride1, hipStream_t st, bool bucket = true);

// NVFP4 product for M >= kMfmaMinRows on the bf16 matrix cores.
constexpr int kMfmaMinRows = 32;
hipError_t launch_mfma_nvfp4(const uint8_t* codes, const uint8_t* scales, const uint8_t* gbytes, int N, int K,
                             const uint16_t* x, int64_t ldx, int M, float* y, int64_t ldy, hipStream_t st);
// Q4_K / Q5_K / Q6_K / Q8_0 product for M >= kMfmaMinRows on the bf16 matrix
// cores (codes as exact bf16, sub-block scales and offsets in fp32), for the
// formats and K that mfma_kquant_supported accepts.
bool mfma_kquant_supported(int fmt, int K);
// w1: the row scales of QG_FP8, the scale plane of QG_NVFP4; gbytes: the NVFP4
// tensor scale (unused otherwise).
hipError_t launch_mfma_kquant(int fmt, const uint8_t* w, const uint8_t* w1, const uint8_t* gbytes, int N, int K,
                              const uint16_t* x, int64_t ldx, int M, float* y, int64_t ldy, hipStream_t st);
// The same product with the (tile, K step) iterations dealt evenly over one
// workgroup per resident slot (stream-K), where the tile count is not a whole
// number of rounds; ws holds per-tile counters and partial tiles
// (mfma_streamk_bytes; 0: the plain launch is taken and ws is not used).
size_t mfma_streamk_bytes(int fmt, int N, int K, int M);
hipError_t launch_mfma_kquant_streamk(int fmt, const uint8_t* w, const uint8_t* w1, const uint8_t* gbytes, int N,
                                      int K, const uint16_t* x, int64_t ldx, int M, float* y, int64_t ldy, void* ws,
                                      size_t ws_bytes, hipStream_t st);
// The same tiles over the row tiles of a grouped product's bucketing
// workspace: tile t of the list at ws[list ..] (count at ws[count], at most
// cap entries) is rows [p, p + bm) of the sorted rows of slot q, (p, q) =
// ws[list + 2 t], ws[list + 2 t + 1], cut at the slot's end; x row perm / xdiv
// in, y row perm out, the weights of the slot's expert (es0 and es1 bytes per
// expert in the two planes; NVFP4: 4 bytes of tensor scale per expert).
struct KqGroup {
    const int32_t* ws;
    int S;             // slots of the layout
    int list, count, cap;
    int64_t es0, es1;
    int xdiv;          // 1: x row = sorted row's original index
};
hipError_t launch_mfma_kquant_grouped(int fmt, const uint8_t* w, const uint8_t* w1, const uint8_t* gbytes, int N,
                                      int K, const uint16_t* x, int64_t ldx, float* y, int64_t ldy, const KqGroup& g,
                                      int bm, hipStream_t st);
int num_cus();

// Element-wise steps of the mixture-of-experts block (qg_moe.hip).
hipError_t launch_moe_swiglu(const float* gu, uint16_t* h, int P, int F, hipStream_t st);
hipError_t launch_moe_combine(const float* yd, const float* wts, const int32_t* idx, int E, float* y, int T, int topk,
                              int D, hipStream_t st);

// Dequantization of rows [0, rows) to fp32.
hipError_t launch_dequant(int fmt, const uint8_t* w, int64_t E, int64_t N, int64_t K, float* out, hipStream_t st);

}  // namespace qg
