// Shared device helpers of libdit (gfx950 / CDNA4).  Nothing here computes a
// step of the method; these are types, bf16 conversions and wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// bf16 bits -> fp32 (exact)
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16 bits, round to nearest even (gfx950 v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// two fp32 -> packed bf16x2 (lo = a, hi = b), round to nearest even
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
    return __builtin_bit_cast(uint32_t, v);
}

// The adjacent-pair rotation (a, b) -> (a cos - b sin, a sin + b cos) in fp32
// with one fixed rounding order (the second product rounded, then one fused
// multiply-add each), packed to bf16: every kernel that rotates q and k gives
// the same bits for the same inputs, whatever the compiler would contract.
__device__ __forceinline__ uint32_t rotate_pack(float a, float b, float c, float s) {
    return pack_bf16x2(__builtin_fmaf(a, c, -(b * s)), __builtin_fmaf(a, s, b * c));
}

// The 32-bit value of another lane of the same 16-lane row, by a DPP row
// permutation (CTRL: a quad_perm or row mirror code); all lanes active.
template <int CTRL>
__device__ __forceinline__ float dpp_row(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over the 16 lanes of a row (lane bits 0..3), without the LDS: lane ^ 1
// and lane ^ 2 by quad permutations, then the half-row and row mirrors, which
// pair each lane with one of the other quad and half row -- whose values equal
// those of lane ^ 4 and lane ^ 8 by then, so the sums are those of the xor
// butterfly, bit for bit.
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_row<0xb1>(v);    // quad_perm(1, 0, 3, 2)
    v += dpp_row<0x4e>(v);    // quad_perm(2, 3, 0, 1)
    v += dpp_row<0x141>(v);   // row_half_mirror
    v += dpp_row<0x140>(v);   // row_mirror
    return v;
}

// silu(x) = x * sigmoid(x); hardware reciprocal (1 ulp) of 1 + e^-x.
__device__ __forceinline__ float silu_f(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// Butterfly sum over all 64 lanes of a wave.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace dit
