// Device helpers shared by the MoE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fgs {

constexpr int kWave = 64;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

// ---------------------------------------------------------------- bfloat16

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }

// float32 -> bfloat16 bits, round to nearest even (inputs are finite)
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// dot of 2 packed bfloat16 pairs, accumulated in float32 (v_dot2_f32_bf16)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}
// 8-element bfloat16 dot product
__device__ __forceinline__ float dot8_bf16(const uint4 &a, const uint4 &b, float c) {
    c = dot2_bf16(a.x, b.x, c);
    c = dot2_bf16(a.y, b.y, c);
    c = dot2_bf16(a.z, b.z, c);
    c = dot2_bf16(a.w, b.w, c);
    return c;
}

// ---------------------------------------------------------------- FP8 E4M3FN
// OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits, subnormals at
// exponent 0, no infinities.  Exact decode from the bit fields; NaN codes are
// not produced by valid weights and decode as a large finite value.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
    uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
    float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20))
                  : float(m) * 0.001953125f;  // m * 2^-9
    return (c & 0x80u) ? -mag : mag;
}

// 8 FP8 codes (packed in a uint2) dotted with 8 bfloat16 activations (uint4)
__device__ __forceinline__ float dot8_e4m3_bf16(const uint2 &w, const uint4 &x, float c) {
    c = fmaf(e4m3_to_f32(w.x & 0xFF), bf16_lo(x.x), c);
    c = fmaf(e4m3_to_f32((w.x >> 8) & 0xFF), bf16_hi(x.x), c);
    c = fmaf(e4m3_to_f32((w.x >> 16) & 0xFF), bf16_lo(x.y), c);
    c = fmaf(e4m3_to_f32(w.x >> 24), bf16_hi(x.y), c);
    c = fmaf(e4m3_to_f32(w.y & 0xFF), bf16_lo(x.z), c);
    c = fmaf(e4m3_to_f32((w.y >> 8) & 0xFF), bf16_hi(x.z), c);
    c = fmaf(e4m3_to_f32((w.y >> 16) & 0xFF), bf16_lo(x.w), c);
    c = fmaf(e4m3_to_f32(w.y >> 24), bf16_hi(x.w), c);
    return c;
}

// ---------------------------------------------------------------- wave ops

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int s = 32; s > 0; s >>= 1) v += __shfl_xor(v, s, kWave);
    return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int s = 32; s > 0; s >>= 1) {
        uint64_t o = __shfl_xor(v, s, kWave);
        v = o > v ? o : v;
    }
    return v;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }
__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + expf(-z)); }

}  // namespace fgs
