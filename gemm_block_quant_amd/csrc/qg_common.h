// qg_common.h -- device helpers shared by the gfx950 kernels of libquantgemm.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
// The same vectors at only 2-byte alignment (gfx950 serves 16- and 8-byte
// global loads at any byte alignment).
typedef uint32_t u32x4_a2 __attribute__((ext_vector_type(4), aligned(2)));
typedef uint32_t u32x2_a2 __attribute__((ext_vector_type(2), aligned(2)));
typedef uint32_t u32_a2 __attribute__((aligned(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

#define QG_LDS __attribute__((address_space(3)))
#define QG_GLOBAL __attribute__((address_space(1)))
typedef QG_LDS uint8_t lds_u8;
typedef QG_LDS uint16_t lds_u16;
typedef QG_LDS uint32_t lds_u32;
typedef QG_LDS u32x4 lds_u32x4;
typedef QG_LDS u32x2 lds_u32x2;
typedef QG_LDS float lds_f32;

constexpr int kWave = 64;

// ---------------------------------------------------------------- arithmetic

// fp32 sum of a.lo*b.lo + a.hi*b.hi + c with one rounding (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2bf(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
}

__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits16 & 0xffffu));
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __builtin_bit_cast(float, (bits16 & 0xffffu) << 16);
}

// E4M3 (fn) byte `sel` (0..3) of v -> fp32, exact (v_cvt_f32_fp8).
template <int SEL>
__device__ __forceinline__ float e4m3_to_f32(uint32_t v) {
    return __builtin_amdgcn_cvt_f32_fp8(v, SEL);
}

// Two E2M1 codes in byte SEL of v -> packed bf16 pair (exact).  The scale
// operand of this conversion only contributes its exponent, so it is 1.0.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1x2_to_bf16x2(uint32_t v) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, SEL));
}

// Two E4M3 codes in half SEL of v (bytes 2 SEL, 2 SEL + 1) -> packed bf16 pair
// (exact: E4M3 values are bf16 values; scale 1.0).
template <int SEL>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t v) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, SEL != 0));
}

// Exact bf16 pair of the small integers held in bytes 2 SEL and 2 SEL + 1 of
// v, each byte an E4M3 code c of the value c * 2^-9: every byte below 16
// (E4M3's subnormals and its first normal binade share the spacing 2^-9, so
// byte b < 16 is b * 2^-9), and the codes 0x10 (16 * 2^-9), 0x90 (-16 * 2^-9),
// 0x98 (-32 * 2^-9).  The conversion scales by the exponent of its scale
// operand, 2^9, so the pair holds the integers themselves.
template <int SEL>
__device__ __forceinline__ uint32_t int_pair_bf16(uint32_t v) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 512.0f, SEL != 0));
}
// E4M3 codes of 16 (h - 2) * 2^-9 for h = 0..3, indexed by v_perm selectors 0..3.
constexpr uint32_t kQ6HighCodes = 0x10009098u;
// Each byte h (0..3) of v replaced by the E4M3 code of 16 (h - 2) * 2^-9.
__device__ __forceinline__ uint32_t q6_high_codes(uint32_t v) { return __builtin_amdgcn_perm(0u, kQ6HighCodes, v); }

// ---------------------------------------------------------------- LDS access

__device__ __forceinline__ u32x4 lds_ld128(const lds_u8* p) { return *(const lds_u32x4*)p; }
__device__ __forceinline__ u32x2 lds_ld64(const lds_u8* p) { return *(const lds_u32x2*)p; }
__device__ __forceinline__ uint32_t lds_ld32(const lds_u8* p) { return *(const lds_u32*)p; }

// 16 bytes from a 2-byte aligned LDS address (reads up to 20 bytes from the
// 4-byte aligned address below p; the buffers keep 16 bytes of slack).
__device__ __forceinline__ u32x4 lds_ld128_a2(const lds_u8* p) {
    uint32_t a = (uint32_t)(uintptr_t)p;
    const lds_u8* q = (const lds_u8*)(uintptr_t)(a & ~3u);
    uint32_t sh = (a & 3u) * 8u;
    uint32_t w0 = lds_ld32(q), w1 = lds_ld32(q + 4), w2 = lds_ld32(q + 8), w3 = lds_ld32(q + 12),
             w4 = lds_ld32(q + 16);
    u32x4 r;
    r.x = __builtin_amdgcn_alignbit(w1, w0, sh);
    r.y = __builtin_amdgcn_alignbit(w2, w1, sh);
    r.z = __builtin_amdgcn_alignbit(w3, w2, sh);
    r.w = __builtin_amdgcn_alignbit(w4, w3, sh);
    return r;
}

// 4 bytes from a 2-byte aligned LDS address.
__device__ __forceinline__ uint32_t lds_ld32_a2(const lds_u8* p) {
    uint32_t a = (uint32_t)(uintptr_t)p;
    const lds_u8* q = (const lds_u8*)(uintptr_t)(a & ~3u);
    return __builtin_amdgcn_alignbit(lds_ld32(q + 4), lds_ld32(q), (a & 3u) * 8u);
}

// ---------------------------------------------------------------- global access

// Streaming 16-byte load that should not displace cached data.  The explicit
// global address space keeps it a global_load (a flat load would also count
// against the LDS wait counter and serialize the row ring with the decode).
__device__ __forceinline__ u32x4 ld_stream128(const uint8_t* p) {
    return __builtin_nontemporal_load((const QG_GLOBAL u32x4*)(uintptr_t)p);
}

// Ordinary global 16-byte load / 4-byte store through the global address space.
__device__ __forceinline__ u32x4 ld_global128(const void* p) { return *(const QG_GLOBAL u32x4*)(uintptr_t)p; }
__device__ __forceinline__ u32x2 ld_global64(const void* p) { return *(const QG_GLOBAL u32x2*)(uintptr_t)p; }
// 16 / 8 / 2 bytes at a 2-byte aligned address.
__device__ __forceinline__ u32x4 ld_global128_a2(const void* p) {
    const u32x4_a2 v = *(const QG_GLOBAL u32x4_a2*)(uintptr_t)p;
    return u32x4{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ u32x2 ld_global64_a2(const void* p) {
    const u32x2_a2 v = *(const QG_GLOBAL u32x2_a2*)(uintptr_t)p;
    return u32x2{v.x, v.y};
}
__device__ __forceinline__ uint32_t ld_global32_a2(const void* p) { return *(const QG_GLOBAL u32_a2*)(uintptr_t)p; }
// 16 / 8 bytes at a 2-byte aligned address p, read as 4-byte aligned loads
// of the 20 / 12 bytes from p rounded down to 4 bytes and shifted into place
// (reads at most 4 bytes past p + 16 / p + 8, all inside the same 4-byte words
// as those up to p + 18 / p + 10).
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));
__device__ __forceinline__ u32x4 ld_global128_a2dw(const void* p) {
    const uintptr_t a = (uintptr_t)p, b = a & ~(uintptr_t)3;
    const uint32_t sh = (uint32_t)(a & 3);
    const u32x4_a4 v = *(const QG_GLOBAL u32x4_a4*)b;
    const uint32_t e = *(const QG_GLOBAL uint32_t*)(b + 16);
    return u32x4{__builtin_amdgcn_alignbyte(v.y, v.x, sh), __builtin_amdgcn_alignbyte(v.z, v.y, sh),
                 __builtin_amdgcn_alignbyte(v.w, v.z, sh), __builtin_amdgcn_alignbyte(e, v.w, sh)};
}
__device__ __forceinline__ u32x2 ld_global64_a2dw(const void* p) {
    const uintptr_t a = (uintptr_t)p, b = a & ~(uintptr_t)3;
    const uint32_t sh = (uint32_t)(a & 3);
    const u32x2_a4 v = *(const QG_GLOBAL u32x2_a4*)b;
    const uint32_t e = *(const QG_GLOBAL uint32_t*)(b + 8);
    return u32x2{__builtin_amdgcn_alignbyte(v.y, v.x, sh), __builtin_amdgcn_alignbyte(e, v.y, sh)};
}
__device__ __forceinline__ uint32_t ld_global16(const void* p) { return *(const QG_GLOBAL uint16_t*)(uintptr_t)p; }
__device__ __forceinline__ void st_global_f32(float* p, float v) { *(QG_GLOBAL float*)(uintptr_t)p = v; }

// 16 bytes starting at p where only [p, limit) may be read (limit - p < 16),
// one byte at a time; bytes past limit read as zero.  Only the final chunk of a
// buffer whose size is not a multiple of 16 takes this path.
__device__ __noinline__ u32x4 ld_tail128(const uint8_t* p, const uint8_t* limit) {
    uint32_t o[4] = {0u, 0u, 0u, 0u};
    uint32_t nvalid = (uint32_t)(limit - p);
    for (uint32_t i = 0; i < nvalid && i < 16u; ++i) o[i >> 2] |= (uint32_t)p[i] << ((i & 3u) * 8u);
    return u32x4{o[0], o[1], o[2], o[3]};
}

// ---------------------------------------------------------------- wave reduction

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

}  // namespace qg
