// qg_dequant.hip -- packed weight[E*N, K] -> fp32, one thread per block.
//
// A test and debugging aid: the products never materialize dequantized
// weights.  Every value is produced with the operation order that makes it
// exact up to a single rounding to nearest even:
//   Q8_0  w = d * q                         (exact)
//   Q4_K  w = (d * sc) * q - dmin * m       (both products exact, one rounding)
//   Q5_K  the same, with 5-bit codes
//   Q6_K  w = (d * s) * (q - 32)            (exact)
//   NVFP4 w = (e2m1 * e4m3) * g             (first product exact, one rounding)
//   FP8   w = e4m3 * s                      (one rounding; a thread per 64 values)
// Block sizes: Q8_0 34 bytes and Q6_K 210 bytes (vllm.cpp issue #3030,
// "BACKEND-TENSTORRENT-KEEPQUANT", issue body); NVFP4 ingredients: E2M1 codes,
// block scales and a per-tensor scale ("I Built a Custom Blackwell Kernel for
// Qwen3.8-27B", section "What the custom path actually does").
#include "qg_internal.h"

namespace qg {

__device__ __forceinline__ uint32_t ld_u16(const uint8_t* p) { return (uint32_t)p[0] | ((uint32_t)p[1] << 8); }

// E2M1 code (4 bits) -> fp32: sign, 2-bit exponent with bias 1, 1-bit mantissa.
__device__ __forceinline__ float e2m1_value(uint32_t c) {
    const uint32_t e = (c >> 1) & 3u, m = c & 1u;
    const float mag = e == 0 ? 0.5f * (float)m : (1.0f + 0.5f * (float)m) * (float)(1u << e) * 0.5f;
    return (c & 8u) ? -mag : mag;
}

__global__ __launch_bounds__(256) void k_dequant_block(int fmt, const uint8_t* __restrict__ w, int64_t rows, int64_t K,
                                                      int64_t N, float* __restrict__ out) {
    const int qk = fmt == QG_Q8_0 ? 32 : fmt == QG_NVFP4 ? 16 : fmt == QG_FP8 ? 64 : 256;
    const int64_t nb = K / qk;
    const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (blk >= rows * nb) return;
    const int64_t r = blk / nb, b = blk % nb;
    float* o = out + r * K + b * qk;
    if (fmt == QG_Q8_0) {
        const uint8_t* p = w + blk * 34;
        const float d = f16_to_f32(ld_u16(p));
        for (int i = 0; i < 32; ++i) o[i] = d * (float)(int8_t)p[2 + i];
    } else if (fmt == QG_Q4_K) {
        const uint8_t* p = w + blk * 144;
        const float d = f16_to_f32(ld_u16(p)), dmin = f16_to_f32(ld_u16(p + 2));
        const uint8_t* S = p + 4;
        const uint8_t* Q = p + 16;
        for (int j = 0; j < 8; ++j) {
            uint32_t sc, m;
            if (j < 4) {
                sc = S[j] & 63u;
                m = S[j + 4] & 63u;
            } else {
                sc = (S[j + 4] & 15u) | ((uint32_t)(S[j - 4] >> 6) << 4);
                m = (S[j + 4] >> 4) | ((uint32_t)(S[j] >> 6) << 4);
            }
            const float ds = d * (float)sc, mm = dmin * (float)m;
            const int g = j >> 1, hi = j & 1;
            for (int l = 0; l < 32; ++l) {
                const uint32_t byte = Q[32 * g + l];
                const uint32_t q = hi ? (byte >> 4) : (byte & 15u);
                o[32 * j + l] = ds * (float)q - mm;
            }
        }
    } else if (fmt == QG_Q5_K) {
        const uint8_t* p = w + blk * 176;
        const float d = f16_to_f32(ld_u16(p)), dmin = f16_to_f32(ld_u16(p + 2));
        const uint8_t* S = p + 4;
        const uint8_t* H = p + 16;
        const uint8_t* Q = p + 48;
        for (int j = 0; j < 8; ++j) {
            uint32_t sc, m;
            if (j < 4) {
                sc = S[j] & 63u;
                m = S[j + 4] & 63u;
            } else {
                sc = (S[j + 4] & 15u) | ((uint32_t)(S[j - 4] >> 6) << 4);
                m = (S[j + 4] >> 4) | ((uint32_t)(S[j] >> 6) << 4);
            }
            const float ds = d * (float)sc, mm = dmin * (float)m;
            const int g = j >> 1, hi = j & 1;
            for (int l = 0; l < 32; ++l) {
                const uint32_t byte = Q[32 * g + l];
                const uint32_t q = (hi ? (byte >> 4) : (byte & 15u)) | ((((uint32_t)H[l] >> j) & 1u) << 4);
                o[32 * j + l] = ds * (float)q - mm;
            }
        }
    } else if (fmt == QG_Q6_K) {
        const uint8_t* p = w + blk * 210;
        const float d = f16_to_f32(ld_u16(p + 208));
        const int8_t* s = (const int8_t*)(p + 192);
        for (int h = 0; h < 2; ++h) {
            const uint8_t* L = p + 64 * h;
            const uint8_t* H = p + 128 + 32 * h;
            for (int l = 0; l < 32; ++l) {
                uint32_t q[4];
                q[0] = (L[l] & 15u) | (((uint32_t)(H[l] >> 0) & 3u) << 4);
                q[1] = (L[l + 32] & 15u) | (((uint32_t)(H[l] >> 2) & 3u) << 4);
                q[2] = (L[l] >> 4) | (((uint32_t)(H[l] >> 4) & 3u) << 4);
                q[3] = (L[l + 32] >> 4) | (((uint32_t)(H[l] >> 6) & 3u) << 4);
                for (int t = 0; t < 4; ++t) {
                    const int v = 128 * h + 32 * t + l;
                    o[v] = (d * (float)s[v >> 4]) * (float)((int)q[t] - 32);
                }
            }
        }
    } else if (fmt == QG_FP8) {  // planes over R = rows: codes [R][K], fp32 row scales [R]
        const uint8_t* codes = w + r * K + b * 64;
        const uint8_t* sp = w + rows * K + 4 * r;
        const uint32_t sb = (uint32_t)sp[0] | ((uint32_t)sp[1] << 8) | ((uint32_t)sp[2] << 16) | ((uint32_t)sp[3] << 24);
        const float s = __builtin_bit_cast(float, sb);
        for (int i = 0; i < 64; ++i) o[i] = e4m3_to_f32<0>(codes[i]) * s;
    } else {  // NVFP4 planes over R = rows: codes [R][K/2], scales [R][K/16], g [rows / N]
        const uint8_t* codes = w + r * (K / 2) + b * 8;
        const uint8_t sb = w[rows * (K / 2) + r * (K / 16) + b];
        const uint8_t* gp = w + rows * (K / 2) + rows * (K / 16) + 4 * (r / N);
        const uint32_t gb = (uint32_t)gp[0] | ((uint32_t)gp[1] << 8) | ((uint32_t)gp[2] << 16) | ((uint32_t)gp[3] << 24);
        const float g = __builtin_bit_cast(float, gb);
        const float s = e4m3_to_f32<0>(sb);
        for (int i = 0; i < 16; ++i) {
            const uint32_t c = (i & 1) ? (codes[i >> 1] >> 4) : (codes[i >> 1] & 15u);
            o[i] = (e2m1_value(c) * s) * g;
        }
    }
}

hipError_t launch_dequant(int fmt, const uint8_t* w, int64_t E, int64_t N, int64_t K, float* out, hipStream_t st) {
    const int qk = fmt == QG_Q8_0 ? 32 : fmt == QG_NVFP4 ? 16 : fmt == QG_FP8 ? 64 : 256;
    const int64_t rows = E * N;
    const int64_t nblk = rows * (K / qk);
    if (nblk == 0) return hipSuccess;
    const int64_t grid = (nblk + 255) / 256;
    hipLaunchKernelGGL(k_dequant_block, dim3((unsigned)grid), dim3(256), 0, st, fmt, w, rows, K, N, out);
    return hipGetLastError();
}

}  // namespace qg
