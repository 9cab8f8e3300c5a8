// MX element arithmetic shared by the standalone quantisers and the grouped GEMM's fused
// output quantisation, so both form the same codes and scale bytes.
// [OCP-MX]: a block of 32 elements shares one E8M0 scale 2^(floor(log2 amax) - emax), emax
// being the element format's largest exponent (8 for E4M3, 2 for E2M1), stored as a byte
// (+127, clamped to 0..254); each element is divided by the scale and rounded to the nearest
// element value (ties to even), saturating at the format's largest magnitude.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// E8M0 byte for a block whose largest magnitude is `amax` (0 for an all-zero block).
__device__ __forceinline__ uint32_t mx_scale_byte(float amax) {
    if (!(amax > 0.f)) return 0u;
    int e2;
    (void)frexpf(amax, &e2);                  // amax = m * 2^e2, m in [0.5, 1)
    const int b = e2 - 1 - 8 + 127;
    return (uint32_t)min(max(b, 0), 254);
}

// 2^(127 - byte): the exact multiplier that divides by the block scale. byte <= 246 for any
// finite bf16/fp32 amax, so the result is a normal float.
__device__ __forceinline__ float mx_inv_scale(uint32_t byte) { return __uint_as_float((254u - byte) << 23); }

// Four scaled values -> four E4M3 codes (OCP "FN": bias 7, 3 mantissa bits, subnormal step
// 2^-9, max 448, no infinities), packed little-endian into one word. gfx950's v_cvt_pk_fp8_f32
// converts to OCP E4M3 with round-to-nearest-even; clamping to +-448 first gives the MX rule's
// saturation (the sign of zero passes through).
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
    a = fminf(fmaxf(a, -448.f), 448.f);
    b = fminf(fmaxf(b, -448.f), 448.f);
    c = fminf(fmaxf(c, -448.f), 448.f);
    d = fminf(fmaxf(d, -448.f), 448.f);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);   // bytes 0, 1
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);         // bytes 2, 3
    return (uint32_t)w;
}

// ---- E2M1 (bias 1, one mantissa bit: 0, 0.5, 1, 1.5, 2, 3, 4, 6)

__device__ __forceinline__ uint32_t mx4_scale_byte(float amax) {
    if (!(amax > 0.f)) return 0u;
    int e2;
    (void)frexpf(amax, &e2);                  // amax = m * 2^e2, m in [0.5, 1)
    const int b = e2 - 1 - 2 + 127;
    return (uint32_t)min(max(b, 0), 254);     // at most 252 for a finite amax
}

// E2M1 code of a scaled value: round to nearest, ties to the even mantissa (the comparisons
// against the midpoints 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5 are strict where the tie goes down
// to an even code and inclusive where it goes up to one), magnitudes above 6 saturate; the sign
// in bit 3, also for a value that rounds to zero. The magnitude index is the code's low 3 bits.
__device__ __forceinline__ uint32_t e2m1_code(float x) {
    const float m = fabsf(x);
    const uint32_t idx = (uint32_t)(m > 0.25f) + (uint32_t)(m >= 0.75f) + (uint32_t)(m > 1.25f) +
                         (uint32_t)(m >= 1.75f) + (uint32_t)(m > 2.5f) + (uint32_t)(m >= 3.5f) + (uint32_t)(m > 5.0f);
    return ((__float_as_uint(x) >> 28) & 0x8u) | idx;
}

}  // namespace moe
