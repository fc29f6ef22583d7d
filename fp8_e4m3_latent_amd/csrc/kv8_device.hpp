// Device-side helpers of libkv8: the e4m3 encoder, exact e4m3 -> bf16/fp16
// conversions and wave reductions.  gfx950 only.
//
// Element format: OCP 8-bit floating point E4M3 (bias 7, no infinities,
// NaN = S.1111.111, largest finite 448, subnormal step 2^-9).
// Encoder rules: page "KV8=1: fp8 e4m3 latent KV cache (CPU + CUDA) with
// .coli_kv v2" (colibri PR #299), commit message, kv_fp8.h item -- round to
// nearest even, saturate at +-448, keep the sign of zero, store NaN as 0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kv8_internal.hpp"

namespace kv8 {

constexpr int kRowBytes = kKvLora + kRope;  // codes per token row

// ---------------------------------------------------------------------------
// Encoder: f32 -> e4m3 code with integer arithmetic on the f32 bit pattern.
//
//   |q| >= 448 (incl. inf)   -> 0x7E (saturate)
//   2^-6 <= |q| < 448       -> normal: keep 3 of the 23 mantissa bits with
//                              round-to-nearest-even by adding 0x7FFFF plus the
//                              lowest kept bit; a carry out of the mantissa
//                              moves into the exponent field, which is exactly
//                              the binade-boundary carry.  The code is the
//                              rounded pattern >> 20 minus the exponent-bias
//                              difference (127 - 7) << 3.
//   |q| < 2^-6              -> subnormal: code = RNE(|q| * 2^9), taken from the
//                              f32 addition |q|*512 + 2^23, whose result has
//                              unit spacing (|q|*512 < 8 is exact); 8 is the
//                              smallest normal code, so the carry is natural.
//   sign bit copied; NaN -> 0x00.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t encode_e4m3(float q) {
    const uint32_t u = __float_as_uint(q);
    const uint32_t a = u & 0x7FFFFFFFu;
    const uint32_t sign = (u >> 24) & 0x80u;
    // normal range: (a + 0x7FFFF + lsb - (960 << 20)) >> 20
    const uint32_t lsb = (a >> 20) & 1u;
    const uint32_t normal = (a + lsb + (0x7FFFFu - (960u << 20))) >> 20;
    // subnormal range
    const float f = __uint_as_float(a) * 512.0f;
    const uint32_t sub = __float_as_uint(f + 8388608.0f) - 0x4B000000u;
    uint32_t code = (a >= 0x3C800000u) ? normal : sub;
    code = (a >= 0x43E00000u) ? 0x7Eu : code;
    code |= sign;
    return (a > 0x7F800000u) ? 0u : code;
}

// Four codes (one 32-bit word, value k in byte k) with the gfx950 fp8
// conversion, which rounds to nearest even into OCP e4m3: NaN is replaced
// by +0 first (so NaN -> 0x00) and every value is clamped to [-448, 448]
// (so |q| >= 448 and +-inf saturate to 0x7E | sign).  Gives the same codes
// as encode_e4m3 for every f32 input.
__device__ __forceinline__ float sat_e4m3(float q) {
    q = q == q ? q : 0.0f;
    return __builtin_amdgcn_fmed3f(q, -448.0f, 448.0f);
}
__device__ __forceinline__ uint32_t encode4_e4m3_hw(float q0, float q1, float q2, float q3) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(q0), sat_e4m3(q1), 0, false);
    return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(sat_e4m3(q2), sat_e4m3(q3), lo, true));
}

// |x| bit pattern if x is finite, else 0: a max over these (as unsigned
// integers) is the largest finite magnitude.
__device__ __forceinline__ uint32_t finite_abs_bits(float x) {
    const uint32_t a = __float_as_uint(x) & 0x7FFFFFFFu;
    return a < 0x7F800000u ? a : 0u;
}

__device__ __forceinline__ uint32_t pack4(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3) {
    return c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
}

// Unsigned max over the 64 lanes of a wave (every lane gets the result).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint32_t o = static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), off, 64));
        v = v > o ? v : o;
    }
    return v;
}

// ---------------------------------------------------------------------------
// Exact decoders.  Every finite e4m3 value has at most 4 significant bits and
// an exponent in [-9, 8], so it is exactly representable in bf16 and in fp16;
// the gfx950 scaled conversions with scale 1.0 produce exactly that value.
// `hi` selects codes 2,3 (true) or 0,1 (false) of the 32-bit word.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

template <bool kHi>
__device__ __forceinline__ uint32_t dec2_bf16(uint32_t four_codes) {
    bf16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(four_codes, 1.0f, kHi);
    return __builtin_bit_cast(uint32_t, r);
}

template <bool kHi>
__device__ __forceinline__ uint32_t dec2_f16(uint32_t four_codes) {
    f16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(four_codes, 1.0f, kHi);
    return __builtin_bit_cast(uint32_t, r);
}

}  // namespace kv8
