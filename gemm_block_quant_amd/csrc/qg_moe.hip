// qg_moe.hip -- the element-wise steps of the mixture-of-experts block around
// the two grouped products: SwiGLU to bf16 and the routing-weighted combine.
// Both are HBM-bound passes over a few MB; each thread produces two values or
// one output element.
#include "qg_internal.h"

namespace qg {

// fp32 -> bf16 bits, round to nearest even; NaN -> 0x7FC0; overflow -> infinity.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float v) {
    const uint32_t b = __builtin_bit_cast(uint32_t, v);
    if ((b & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// h[p, f] = bf16(silu(g) * u), g = gu[p, f], u = gu[p, F + f], silu(g) = g / (1 + exp(-g)).
// Two values per thread (F % 2 == 0).
__global__ __launch_bounds__(256) void k_moe_swiglu(const float* __restrict__ gu, uint16_t* __restrict__ h, int P,
                                                    int F) {
    const int half = F / 2;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)P * half) return;
    const int p = (int)(i / half), f = 2 * (int)(i % half);
    const float* row = gu + (int64_t)p * 2 * F;
    const float g0 = row[f], g1 = row[f + 1], u0 = row[F + f], u1 = row[F + f + 1];
    const float h0 = g0 / (1.f + expf(-g0)) * u0;
    const float h1 = g1 / (1.f + expf(-g1)) * u1;
    *(QG_GLOBAL uint32_t*)(uintptr_t)(h + (int64_t)p * F + f) = f32_to_bf16_rne(h0) | (f32_to_bf16_rne(h1) << 16);
}

// y[t, d] = sum_j wts[t, j] * yd[t * topk + j, d], j ascending, fp32 fused
// multiply-adds; NaN for a token with an id outside [0, E) (the down product
// does not write those pairs).
__global__ __launch_bounds__(256) void k_moe_combine(const float* __restrict__ yd, const float* __restrict__ wts,
                                                     const int32_t* __restrict__ idx, int E, float* __restrict__ y,
                                                     int T, int topk, int D) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)T * D) return;
    const int t = (int)(i / D), d = (int)(i % D);
    float acc = 0.f;
    bool bad = false;
    for (int j = 0; j < topk; ++j) {
        const int e = idx[(int64_t)t * topk + j];
        bad |= e < 0 || e >= E;
        acc = fmaf(wts[(int64_t)t * topk + j], yd[((int64_t)t * topk + j) * D + d], acc);
    }
    y[i] = bad ? __builtin_nanf("") : acc;
}

static unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }

hipError_t launch_moe_swiglu(const float* gu, uint16_t* h, int P, int F, hipStream_t st) {
    hipLaunchKernelGGL(k_moe_swiglu, dim3(blocks_for((int64_t)P * (F / 2))), dim3(256), 0, st, gu, h, P, F);
    return hipGetLastError();
}

hipError_t launch_moe_combine(const float* yd, const float* wts, const int32_t* idx, int E, float* y, int T, int topk,
                              int D, hipStream_t st) {
    hipLaunchKernelGGL(k_moe_combine, dim3(blocks_for((int64_t)T * D)), dim3(256), 0, st, yd, wts, idx, E, y, T, topk,
                       D);
    return hipGetLastError();
}

}  // namespace qg
