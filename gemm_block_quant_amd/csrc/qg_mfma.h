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

// f(std::integral_constant<int, i>{}) for i = 0 .. N-1, unrolled.
template <int N, int I = 0, class Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(f);
    }
}

}  // namespace qg
