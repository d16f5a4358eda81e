// Device helpers shared by the MoE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fgs {

constexpr int kWave = 64;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

// ---------------------------------------------------------------- loads
// Streaming (non-temporal) loads for weights that are read exactly once.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld_stream16(const void *p) {
    u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_stream8(const void *p) {
    u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p));
    return make_uint2(v.x, v.y);
}

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

// ---------------------------------------------------------------- wave ops

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int s = 32; s > 0; s >>= 1) v += __shfl_xor(v, s, kWave);
    return v;
}

// partner lane's copy of a 32-bit value across lane bit log2(S): distance 32
// and 16 by swapping a register with itself (v_permlane32_swap /
// v_permlane16_swap), below that by DPP row_mirror, row_half_mirror and quad
// permutes (the same pairings as the butterfly below)
template <int S>
__device__ __forceinline__ uint32_t partner_u32(uint32_t v) {
    if constexpr (S == 32 || S == 16) {
        auto r = (S == 32) ? __builtin_amdgcn_permlane32_swap(v, v, false, false)
                           : __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (threadIdx.x & S) ? r[0] : r[1];
    } else {
        constexpr int ctrl = S == 8 ? 0x140 : S == 4 ? 0x141 : S == 2 ? 0x4E : 0xB1;
        return __builtin_amdgcn_update_dpp(0u, v, ctrl, 0xF, 0xF, false);
    }
}

template <int S>
__device__ __forceinline__ uint64_t max_step_u64(uint64_t v) {
    const uint64_t o = ((uint64_t)partner_u32<S>((uint32_t)(v >> 32)) << 32) | partner_u32<S>((uint32_t)v);
    return o > v ? o : v;
}

// wave-wide maximum of a 64-bit key, result in every lane
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    v = max_step_u64<32>(v);
    v = max_step_u64<16>(v);
    v = max_step_u64<8>(v);
    v = max_step_u64<4>(v);
    v = max_step_u64<2>(v);
    return max_step_u64<1>(v);
}

// ---------------------------------------------------------------- butterfly
// Reduce-scatter of V partial sums (V a power of two <= 64) over a wave: at
// each halving step a lane keeps half of its values and adds its partner's
// copy of that half, so after log2(V) steps lane l holds one fully reduced
// value, index butterfly_index<V>(l); the remaining steps sum the last value.
// Lane pairing per step: distance 32 and 16 through v_permlane32_swap /
// v_permlane16_swap (one instruction exchanges the halves of two registers),
// then DPP row_mirror (lane i <-> 15-i), row_half_mirror (i <-> 7-i) and quad
// permutes (xor 2, xor 1).  Each pairing flips exactly the step's lane bit,
// and the partners' contribution sets are disjoint, so every value ends up
// summed over all 64 lanes.

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppRowMirror = 0x140, kDppHalfMirror = 0x141, kDppXor2 = 0x4E, kDppXor1 = 0xB1;

template <int S>
__device__ __forceinline__ float pair_get(float v) {  // partner's value across lane bit log2(S)
    if constexpr (S == 8) return dpp_f<kDppRowMirror>(v);
    else if constexpr (S == 4) return dpp_f<kDppHalfMirror>(v);
    else if constexpr (S == 2) return dpp_f<kDppXor2>(v);
    else return dpp_f<kDppXor1>(v);
}

template <int S, int V>
__device__ __forceinline__ void bfly_step(float (&v)[V], int &n) {
    if (n > 1) {
        const int h = n / 2;
        if constexpr (S == 32 || S == 16) {
#pragma unroll
            for (int i = 0; i < V / 2; ++i) {
                if (i < h) {
                    uint32_t a = __float_as_uint(v[i]), b = __float_as_uint(v[i + h]);
                    auto r = (S == 32) ? __builtin_amdgcn_permlane32_swap(a, b, false, false)
                                       : __builtin_amdgcn_permlane16_swap(a, b, false, false);
                    v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
                }
            }
        } else {
            const bool upper = (threadIdx.x & S) != 0;
#pragma unroll
            for (int i = 0; i < V / 2; ++i) {
                if (i < h) {
                    const float send = upper ? v[i] : v[i + h];
                    const float keep = upper ? v[i + h] : v[i];
                    v[i] = keep + pair_get<S>(send);
                }
            }
        }
        n = h;
    } else {
        if constexpr (S == 32 || S == 16) {
            uint32_t a = __float_as_uint(v[0]);
            auto r = (S == 32) ? __builtin_amdgcn_permlane32_swap(a, a, false, false)
                               : __builtin_amdgcn_permlane16_swap(a, a, false, false);
            // after swapping a register with itself each lane sees its partner's copy in one output
            const bool upper = (threadIdx.x & S) != 0;
            v[0] += __uint_as_float(upper ? r[0] : r[1]);
        } else {
            v[0] += pair_get<S>(v[0]);
        }
    }
}

template <int V>
__device__ __forceinline__ void butterfly_reduce(float (&v)[V]) {
    int n = V;
    bfly_step<32>(v, n);
    bfly_step<16>(v, n);
    bfly_step<8>(v, n);
    bfly_step<4>(v, n);
    bfly_step<2>(v, n);
    bfly_step<1>(v, n);
}

template <int V>
__device__ __forceinline__ int butterfly_index(int lane) {
    int idx = 0, n = V;
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
        if (n > 1) {
            if (lane & s) idx += n / 2;
            n /= 2;
        }
    }
    return idx;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }
__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + expf(-z)); }

}  // namespace fgs
