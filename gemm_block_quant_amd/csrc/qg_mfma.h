// qg_mfma.h -- shared pieces of the matrix-core tile kernels (M >= 32).
#pragma once

#include <type_traits>

#include "qg_internal.h"

namespace qg {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// DPP quad permutations: each lane takes the value of lane ^ 1, lane ^ 2 of its quad.
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2, 3, 0, 1]
constexpr uint32_t kBf16Ones = 0x3F803F80u;  // bf16 pair (1, 1)

constexpr int kMfmaKStep = 64;
constexpr int kMfmaRowBytes = 144;  // one tile row: 64 bf16 (128 B) + 16 B padding (conflict-free fragment reads)
constexpr int kMfmaThreads = 256;

__device__ __forceinline__ uint32_t bf16_pair_from_exact(float lo, float hi) {
    // lo, hi are exact in bf16: their top 16 bits are the bf16 encodings.
    return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, hi), __builtin_bit_cast(uint32_t, lo), 0x07060302u);
}

// 16 NVFP4 values (8 code bytes c0, c1; E4M3 scale s) -> 8 dwords of bf16
// pairs bf16(e2m1 * s), value order k = 0..15.
__device__ __forceinline__ void decode_nvfp4_block_bf16(uint32_t c0, uint32_t c1, float s, uint32_t (&o)[8]) {
    auto pair = [&](uint32_t c, int sel) -> uint32_t {
        f32x2 v;
        switch (sel) {
            case 0: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0); break;
            case 1: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 1); break;
            case 2: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 2); break;
            default: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 3); break;
        }
        const float lo = v.x * s, hi = v.y * s;
        return bf16_pair_from_exact(lo, hi);
    };
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        o[b] = pair(c0, b);
        o[4 + b] = pair(c1, b);
    }
}

// f(std::integral_constant<int, i>{}) for i = 0 .. N-1, unrolled.
template <int N, int I = 0, class Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(f);
    }
}

}  // namespace qg
