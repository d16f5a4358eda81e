// Dynamic FP8 quantisation of activations in 1 x 128 groups.
//
// "Inside Kolibri 1" (flozi.net), section "The FP8 path is explicitly mixed
// precision": the released checkpoint's FP8 linears take activations that are
// quantised on the fly in groups of 1 x 128.  Per group of 128 consecutive
// values of a row: scale = amax / 448 (FP32; 1 for an all-zero group), code =
// E4M3 of (v / scale), nearest-even, clamped to +-448.  Every step is an FP32
// operation with IEEE division, so codes are reproducible bit for bit.
//
// One thread handles 8 values (one 16- or 32-byte load); the 16 threads of a
// group are 16 consecutive lanes, and the group maximum is a 4-step xor
// butterfly inside them.  The kernel is bound by HBM (read v, write codes).
#include "moe_common.h"
#include "moe_plan.h"

namespace fgs {

// 8 values -> float
template <bool BF16>
__device__ __forceinline__ void load8(const void *v, size_t elem, float (&o)[8]) {
    if constexpr (BF16) {
        const uint4 u = *reinterpret_cast<const uint4 *>((const uint16_t *)v + elem);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = bf16_lo(w[i]);
            o[2 * i + 1] = bf16_hi(w[i]);
        }
    } else {
        const float4 a = *reinterpret_cast<const float4 *>((const float *)v + elem);
        const float4 b = *reinterpret_cast<const float4 *>((const float *)v + elem + 4);
        o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
        o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    }
}

// grid: ceil(rows * cols / 8 / 256); block 256.  cols is a multiple of 128.
template <bool BF16>
__global__ __launch_bounds__(256) void quant_groups_kernel(const void *__restrict__ v, int ldv, long rows, int cols,
                                                           uint8_t *__restrict__ q, int ldq, float *__restrict__ s,
                                                           int lds) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;  // 8-value chunk
    const int cpr = cols / 8;
    const long r = i / cpr;
    const int c = (int)(i % cpr) * 8;
    // threads past the end take part in the group reductions with a valid row
    const long rr = r < rows ? r : 0;
    float x[8];
    load8<BF16>(v, (size_t)rr * ldv + c, x);
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(x[j]));
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
    const float sc = m > 0.f ? m / 448.0f : 1.0f;
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = fminf(fmaxf(x[j] / sc, -448.f), 448.f);
    // v_cvt_pk_fp8_f32: two values to E4M3 (nearest even) into the low or high half-word
    uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
    uint32_t hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
    if (r >= rows) return;
    *reinterpret_cast<uint2 *>(q + (size_t)r * ldq + c) = make_uint2(lo, hi);
    if ((c & 127) == 0) s[(size_t)r * lds + c / 128] = sc;
}

hipError_t launch_quant_groups(const void *v, int v_bf16, int ldv, long rows, int cols, uint8_t *q, int ldq,
                               float *s, int lds, hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    const long chunks = rows * (long)(cols / 8);
    dim3 grid((unsigned)((chunks + 255) / 256)), block(256);
    if (v_bf16)
        hipLaunchKernelGGL((quant_groups_kernel<true>), grid, block, 0, stream, v, ldv, rows, cols, q, ldq, s, lds);
    else
        hipLaunchKernelGGL((quant_groups_kernel<false>), grid, block, 0, stream, v, ldv, rows, cols, q, ldq, s, lds);
    return hipGetLastError();
}

}  // namespace fgs
