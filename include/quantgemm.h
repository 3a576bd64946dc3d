/*
 * quantgemm.h -- C ABI of the MI355X (gfx950) block-quantized weight x bf16
 * activation library (libquantgemm.so).
 *
 * The library multiplies a packed low-bit weight matrix W[N, K] ("BT" layout:
 * one output per stored row, blocks running along K) by bf16 activations
 * x[M, K] and writes fp32 y[M, N]:
 *
 *     y[m, n] = sum_k W[n, k] * x[m, k]
 *
 * Each packed weight block is read from device memory once per call and
 * dequantized in registers; the dequantized matrix never exists in memory.
 * This is the fused dequant-matvec of "A 320B MoE on a free Kaggle TPU"
 * (section "The kernel, and why 64 tok/s is not a bandwidth number"), and the
 * decode weight stream whose bytes / bandwidth set the token rate in
 * "Qwen3.8-27B on one Tenstorrent P150" (section "4. Measuring the ceiling").
 * The grouped entry point follows the operator seam weight[E*N, K] of vllm.cpp
 * issue #3030 ("BACKEND-TENSTORRENT-KEEPQUANT", section "Second
 * falsification"): E stacked matrices, E = 1 being the dense case.
 *
 * Conventions shared by every entry point:
 *  - Pointers named w*, x, y, ids, idx, wts, out and workspace are DEVICE pointers owned by
 *    the caller; the library allocates nothing, keeps no per-call state and
 *    never synchronizes.  `stream` is a hipStream_t (NULL = the null stream);
 *    work is enqueued on it and the call returns immediately.
 *  - Arguments are validated on the host before anything is launched.  On
 *    failure a non-zero qg_status is returned and nothing is enqueued.  A
 *    failed launch returns QG_EHIP.  No C++ exception crosses this ABI.
 *  - Alignment: w 16 bytes, x 16 bytes, y / out 4 bytes, ids 4 bytes,
 *    workspace 16 bytes (QG_EALIGN otherwise).
 *  - Weight reads are whole aligned 16-byte granules: the last granule of a
 *    weight plane may be read past the plane's final byte (never past the
 *    granule, so never onto another page); those bytes are not used.
 *  - Shapes: N, M, E >= 0; 0 < K <= 2^24 and a multiple of the format's
 *    block (QG_ESHAPE otherwise).  M == 0 or N == 0 is a valid no-op.
 *
 * Packed layouts (all multi-byte fields little endian; rows contiguous, row r
 * of weight[R, K] holding K / QK blocks in K order):
 *  - QG_Q8_0 (QK = 32, 34 bytes): fp16 d, then 32 int8 q.  w = d * q.
 *  - QG_Q4_K (QK = 256, 144 bytes): fp16 d, fp16 dmin, 12 bytes of packed
 *    6-bit sub-block scales sc[8] and mins m[8], 128 bytes of 4-bit codes.
 *    w = d * sc_j * q - dmin * m_j for sub-block j of 32 values.
 *  - QG_Q5_K (QK = 256, 176 bytes): fp16 d, fp16 dmin, the 12 scale bytes of
 *    Q4_K, 32 bytes H of fifth bits, 128 bytes of 4-bit codes laid out as in
 *    Q4_K; the code of sub-block j at position l gets bit j of H[l] as its
 *    fifth bit (q in 0..31).  w = d * sc_j * q - dmin * m_j.  (The 27B
 *    artefact carries Q5_K tensors that the packed-word kernels still owe:
 *    vllm.cpp issue #3030, paragraph "Re-anchor (scope item 1 replaced)".)
 *  - QG_Q6_K (QK = 256, 210 bytes): 128 bytes low nibbles, 64 bytes high
 *    2-bit pairs, 16 int8 sub-scales (one per 16 values), fp16 d.
 *    w = d * s * (q - 32).
 *    (Q8_0 = 34 B and Q6_K = 210 B blocks: vllm.cpp issue #3030, issue body,
 *    residency budget.  Bit positions inside the K-quant blocks follow the
 *    GGUF convention.)
 *  - QG_NVFP4 (QK = 16): three planes over R = E*N rows:
 *      codes  [R][K/2]   E2M1 nibbles, value k in the low nibble of byte k/2
 *                        when k is even, the high nibble when odd;
 *      scales [R][K/16]  one E4M3 (fn) scale per 16 values;
 *      g      [E]        one fp32 scale per stacked matrix.
 *    w = (e2m1 * e4m3) * g  ("I Built a Custom Blackwell Kernel for
 *    Qwen3.8-27B", section "What the custom path actually does": E2M1 codes,
 *    block scales and a per-site weight scale kept in the artefact).
 *  - QG_FP8 (row-scaled FP8; K a multiple of 64): two planes over R = E*N rows:
 *      codes  [R][K]  one E4M3 (fn) byte per value;
 *      scales [R]     one fp32 scale per row.
 *    w = e4m3 * s  (same page and section: attention and GDN projections, the
 *    output head and the last eight MLPs stay row-scaled FP8).
 *  quant_packed_bytes() is the single source of truth for buffer sizes.
 *
 * Numerics: the dequantized weights of quant_dequantize are bit-exact fp32
 * (one rounding at most, round to nearest even).  The products take each
 * block's integer codes at their own value (never shifted by a constant that
 * is subtracted again later), so a row whose weights are all zero gives
 * exactly 0, and apply the block scales and mins in fp32 to per-block sums.
 * The FP8 row scale and the NVFP4 tensor scale multiply finished fp32 sums,
 * which matches summing the fp32 weights of quant_dequantize (to fp32
 * rounding) while every product e4m3 * s, or e2m1 * e4m3 * g, lies in fp32's
 * normal range: FP8 row scales in [2^-117, 2^119], NVFP4 g in [2^-116, 2^115].
 * Products accumulate in fp32 in a fixed order: results are deterministic run
 * to run, row m of any quant_gemm call with M <= 16 is bitwise equal to
 * quant_gemv on x[m], and
 * such a call is bitwise equal to quant_grouped_gemm with E = 1 and ids =
 * NULL.  Calls with M >= 32 that run on the matrix cores (below) accumulate
 * in another (still fixed) order: their rows do not depend on M or on the
 * other rows, and they too equal quant_grouped_gemm with E = 1 and ids = NULL
 * bit for bit (QG_NVFP4 with K % 64 != 0 aside).
 */
#ifndef QUANTGEMM_H
#define QUANTGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The *_MAX_ENUM members give both enums the full 32-bit int range: a caller
 * may pass any int, and an unknown value is rejected (QG_EFORMAT, "unknown
 * status") rather than being out of the enum's range. */
typedef enum {
    QG_Q8_0 = 1,
    QG_Q4_K = 2,
    QG_Q6_K = 3,
    QG_NVFP4 = 4,
    QG_Q5_K = 5,
    QG_FP8 = 6,
    QG_FORMAT_MAX_ENUM = 0x7FFFFFFF
} qg_format;

typedef enum {
    QG_OK = 0,
    QG_EINVAL = 1,   /* null pointer where one is required */
    QG_EFORMAT = 2,  /* unknown format tag */
    QG_EALIGN = 3,   /* a pointer violates the alignment above */
    QG_ESHAPE = 4,   /* negative size, K not a positive multiple of the block, size overflow, limits */
    QG_EHIP = 5,     /* the HIP runtime reported an error on launch */
    QG_ENOTIMPL = 6, /* combination not implemented by this build */
    QG_EWORKSPACE = 7, /* workspace missing or smaller than quant_grouped_workspace_bytes() */
    QG_STATUS_MAX_ENUM = 0x7FFFFFFF
} qg_status;

/* Values per block (Q8_0 32, Q4_K / Q5_K / Q6_K 256, NVFP4 16; FP8 64, the
 * granularity of K) for a tag, 0 for an unknown tag.  Host only. */
int64_t quant_block_values(qg_format fmt);

/* Bytes of a packed weight[E*N, K] tensor in the layout above; 0 when the tag
 * is unknown, a size is negative or K is not a multiple of the block.  Host
 * only, touches no device.  The count a residency budget is made of: packed
 * bytes per tensor (vllm.cpp issue #3030, issue body: the packed-versus-bf16
 * byte inventory of the 27B artefact, 34- and 210-byte blocks), and the bytes
 * a decode step must stream ("Qwen3.8-27B on one Tenstorrent P150", section
 * "4. Measuring the ceiling"). */
size_t quant_packed_bytes(qg_format fmt, int64_t E, int64_t N, int64_t K);

/* Decode GEMV (M = 1): y[n] = sum_k W[n, k] * x[k].
 * w: packed weight[N, K]; x: bf16 bit patterns [K]; y: fp32 [N] (overwritten). */
qg_status quant_gemv(const void* w, qg_format fmt, int64_t N, int64_t K, const uint16_t* x, float* y,
                     void* stream);

/* Skinny / prefill product: y[m, n] = sum_k W[n, k] * x[m, k] for m < M.
 * x: bf16 [M, K] row-major; y: fp32 [M, N] row-major (overwritten).
 * Each weight block is read once per call for M <= 16 (speculative-verify
 * blocks of 8 positions: "Qwen3.8-27B on one Tenstorrent P150", section "5.
 * DFlash2 on Blackhole").  With M >= 32 every format runs a bf16 matrix-core
 * tile path that reads each weight block once per tile of 64 or 128
 * activation rows ("Qwen3.8-27B on one Tenstorrent P150", section "3. Porting
 * the 9B stack to 27B geometry": prefill must not re-stream the weights per
 * few rows); QG_Q8_0 does so when K is a multiple of 64.  Other calls with
 * M > 16 take passes of 16 rows. */
qg_status quant_gemm(const void* w, qg_format fmt, int64_t N, int64_t K, int64_t M, const uint16_t* x, float* y,
                     void* stream);

/* Bytes of workspace quant_gemm_streamk needs for this call (0 where it
 * needs none: quant_gemm_streamk is then quant_gemm and ignores the
 * workspace).  Depends on the current device (its compute-unit count and
 * the kernels' residency on it).  Host only; 0 for invalid shapes. */
size_t quant_gemm_streamk_workspace_bytes(qg_format fmt, int64_t N, int64_t K, int64_t M);

/* quant_gemm (same operation, arguments and limits: the product of the
 * passage cited there) with a workspace that lets two schedules spread the
 * work evenly over the GPU:
 *  - 5..16 rows, where quant_gemm would stage the activations in several K
 *    phases (rows of K = 17,408 cut into K segments, e.g. the 5120-row down
 *    projections): passes of up to 8 rows in which each workgroup takes one
 *    K segment and the segments' fp32 sums meet in the workspace, added in
 *    segment order by the last to finish.  The arithmetic is quant_gemm's:
 *    each row equals the M = 1 result bit for bit.
 *  - 32 <= M <= 2^21 rows, where the matrix-core tiles would leave resident
 *    workgroups (two per compute unit) idle: the (tile, 64-value K step)
 *    iterations are dealt to them in equal contiguous ranges, and a tile
 *    split between workgroups is finished by the last part to arrive, which
 *    adds the parts' fp32 partial sums in a fixed order.  Results are
 *    deterministic and within quant_gemm's error bound, but not bit for bit
 *    quant_gemm's where a tile is split.
 * Each weight block is still read once per call (per tile of rows at M >= 32).
 * workspace: device scratch of at least
 * quant_gemm_streamk_workspace_bytes(fmt, N, K, M) bytes (16-byte aligned;
 * NULL allowed when that is 0), contents undefined between calls; calls
 * sharing a workspace must be ordered on one stream.  QG_EWORKSPACE if it is
 * missing or too small.  Captures into a HIP graph (no memset, no allocation). */
qg_status quant_gemm_streamk(const void* w, qg_format fmt, int64_t N, int64_t K, int64_t M, const uint16_t* x,
                             float* y, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace quant_grouped_gemm needs for E experts and M rows: the
 * device-side bucketing of rows by expert (per-expert counts and offsets, the
 * row permutation), which is how each distinct expert is read once per call
 * ("A 320B MoE on a free Kaggle TPU", section "Three things the README gets
 * wrong": prefill groups the routed pairs by expert before the matvec).
 * Host only; 0 for a negative size. */
size_t quant_grouped_workspace_bytes(int64_t E, int64_t M);

/* Grouped-expert product over stacked weights:
 *     y[i, n] = sum_k W_{ids[i]}[n, k] * x[i, k],  W_e = rows [e*N, (e+1)*N) of weight[E*N, K].
 * w: packed weight[E*N, K] (for QG_NVFP4 the planes span all E*N rows and g
 * holds E scales); x: bf16 [M, K]; ids: int32 [M] expert ids, or NULL meaning
 * expert 0 for every row; y: fp32 [M, N].
 * Rows are bucketed by expert on the device so that each distinct expert's
 * weights are read once per call, whatever the number of rows routed to it
 * ("A 320B MoE on a free Kaggle TPU", section "The decode kernel's cost is not
 * distinct experts").  When the call has at least 4 rows per possible
 * distinct expert (M >= 32 and M >= 4 * min(E, M)), an expert with 32 or more
 * rows runs on the matrix-core tiles of quant_gemm over its rows (64- or
 * 128-row tiles; its weights are read once per tile of rows, the repeats from
 * cache), except for QG_NVFP4 with K % 64 != 0 and QG_Q8_0 with K % 64 == 32.
 * Every other expert streams its weights for up to 16 of its rows per pass
 * (once for all its rows when it has at most 16).
 * An id outside [0, E) cannot be reported without a synchronization: every
 * element of that row of y is set to NaN.
 * workspace: device scratch of at least quant_grouped_workspace_bytes(E, M)
 * bytes, contents undefined between calls; calls sharing a workspace must be
 * ordered on one stream.  Limits (QG_ESHAPE beyond, before anything is
 * launched): M <= 16384; one activation row of K values must fit in the 160 KB
 * of LDS with the kernel's other state: K <= 19200 for Q4_K and Q5_K, 20224
 * for Q6_K, 20416 for NVFP4 and FP8 with K % 64 == 0. */
qg_status quant_grouped_gemm(const void* w, qg_format fmt, int64_t E, int64_t N, int64_t K, int64_t M,
                             const uint16_t* x, const int32_t* ids, float* y, void* workspace,
                             size_t workspace_bytes, void* stream);

/* quant_grouped_gemm without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments, results (bit for bit),
 * limits and errors as quant_grouped_gemm; it allocates nothing and calls no
 * allocating routine.  Its bucketing scratch is a static device array of
 * 204,832 bytes inside the library (enough for the largest call, M = 16384;
 * QG_EWORKSPACE if a call ever needed more), one copy per GPU, held until the
 * process ends.  The first call on each device resolves that copy's address
 * (a host-side query; make it outside graph capture).  Every call on one GPU
 * shares the array and leaves its last contents there (each call writes all
 * it reads first), so calls on one GPU must be ordered on one stream: calls
 * that overlap on one GPU race. */
qg_status quant_grouped_gemm_noalloc(const void* w, qg_format fmt, int64_t E, int64_t N, int64_t K, int64_t M,
                                     const uint16_t* x, const int32_t* ids, float* y, void* stream);

/* Bytes of workspace quant_moe_block needs (0 when the arguments would be
 * rejected by quant_moe_block's shape checks).  Host only. */
size_t quant_moe_workspace_bytes(qg_format fmt_gate_up, qg_format fmt_down, int64_t E, int64_t D, int64_t F,
                                 int64_t T, int64_t topk);

/* Mixture-of-experts block over T tokens, each routed to topk experts:
 *     y[t, :] = sum_j wts[t, j] * W_down_e . h_{t,j},   e = idx[t, j],
 *     h_{t,j} = bf16( silu(g) * u ),  g = W_gate_e . x[t, :],  u = W_up_e . x[t, :],
 *     silu(g) = g / (1 + exp(-g)),
 * the dispatch interface x [T, D], idx [T, topk] int32, wts [T, topk] fp32 ->
 * [T, D] of "A 320B MoE on a free Kaggle TPU" (section "The decode kernel's
 * cost is not distinct experts"), with gate and up joined into one parent
 * because they share the input ("I Built a Custom Blackwell Kernel for
 * Qwen3.8-27B", section "What the custom path actually does").
 * w_gate_up: packed weight[E * 2F, D] of fmt_gate_up; rows [e*2F, e*2F + F) of
 *   expert e are its gate, rows [e*2F + F, (e+1)*2F) its up (NVFP4: E tensor
 *   scales, one per expert's 2F rows).
 * w_down: packed weight[E * D, F] of fmt_down.
 * x: bf16 [T, D]; idx: int32 [T, topk]; wts: fp32 [T, topk]; y: fp32 [T, D]
 * (overwritten).  The intermediate h is rounded once to bf16 (round to
 * nearest even) from fp32; the sum over j runs in ascending order in fp32.
 * Each distinct expert's weights are read once per product.
 * A token with an id outside [0, E) gets NaN in every element of its row.
 * workspace: device scratch of at least quant_moe_workspace_bytes(...) bytes,
 * contents undefined between calls; calls sharing it must be ordered on one
 * stream.  Limits: T * topk <= 16384; D and F multiples of the formats'
 * blocks and within quant_grouped_gemm's K limits (QG_ESHAPE otherwise).
 * T == 0 is a valid no-op.
 * Alignment: w_gate_up, w_down, x, workspace 16 bytes; idx, wts, y 4 bytes. */
qg_status quant_moe_block(const void* w_gate_up, qg_format fmt_gate_up, const void* w_down, qg_format fmt_down,
                          int64_t E, int64_t D, int64_t F, int64_t T, int64_t topk, const uint16_t* x,
                          const int32_t* idx, const float* wts, float* y, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Dequantize rows [0, rows) of a packed weight[rows, K] to fp32 out[rows, K]
 * (bit-exact; a test and debugging aid, the products never call it).  It
 * writes out the per-format block decode that the products do in registers,
 * so that it can be compared with a dequantizer taken as the reference
 * (vllm.cpp issue #3030, issue body: keep-quant matmuls gated against
 * llama.cpp's own dequantization; "A 320B MoE on a free Kaggle TPU", section
 * "What I actually ran": the kernel checked against gguf's dequantize).
 * For QG_NVFP4, `rows` is E*N of the tensor and all rows use g[0]; use
 * quant_dequantize_stacked for several stacked matrices. */
qg_status quant_dequantize(const void* w, qg_format fmt, int64_t rows, int64_t K, float* out, void* stream);

/* As quant_dequantize for a stacked weight[E*N, K]: out is [E*N, K]. */
qg_status quant_dequantize_stacked(const void* w, qg_format fmt, int64_t E, int64_t N, int64_t K, float* out,
                                   void* stream);

/* Static description of a status code, "unknown status" for any other value;
 * never NULL.  Host only.  (A convenience of this ABI; the pages define no
 * error codes.) */
const char* quant_status_string(qg_status s);

/* Measurement reference, not part of the product path: a plain streaming read
 * of `bytes` bytes at `buf` (each 16-byte granule once, non-temporal loads,
 * eight 256-thread workgroups per CU striding over the buffer with eight
 * loads in flight per thread: the fastest read shape measured),
 * the achievable-bandwidth ceiling the streaming kernels are compared with
 * ("Qwen3.8-27B on one Tenstorrent P150", section "4. Measuring the ceiling,
 * and lots of dead ends": a validated read microbenchmark as the ceiling).
 * buf: device, 16-byte aligned; bytes: a multiple of 16 (0 is a no-op);
 * sink: one device uint32, written only in the (practically impossible) case
 * that the xor of all words equals 0x9E3779B9.  Asynchronous on `stream`.
 * Errors: QG_EINVAL (null), QG_EALIGN, QG_ESHAPE (bytes % 16), QG_EHIP. */
qg_status quant_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QUANTGEMM_H */
