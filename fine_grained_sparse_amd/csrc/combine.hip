// Weighted unpermute: out[t] = S(x_t) + sum_j w[t,j] * Y[row_of_pair[t*k+j]].
//
// "Kolibri 1 Deep Dive" (abrarakhunji.com), "Mathematical Routing & Load
// Balancing Formulation": the layer output is the gate-weighted sum of the
// selected experts' SwiGLU outputs; "Inside Kolibri 1" (flozi.net), section
// "The released stack": the shared expert is added for every token.  The sum
// runs in FP32 in a fixed order (shared, then slots 0..k-1) and is rounded
// once to the output type; with MOE_FLAG_ACCUMULATE the old output (the
// residual stream) is added before that rounding.
#include "moe_common.h"
#include "moe_plan.h"

namespace fgs {

template <bool YBF16>
__device__ __forceinline__ float4 load_y4(const void *Y, size_t elem) {
    if constexpr (YBF16) {
        const uint2 v = *reinterpret_cast<const uint2 *>((const uint16_t *)Y + elem);
        return make_float4(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y));
    } else {
        return *reinterpret_cast<const float4 *>((const float *)Y + elem);
    }
}

template <bool BF16OUT, bool YBF16>
__global__ __launch_bounds__(256) void combine_kernel(
    const void *__restrict__ Y, const float *__restrict__ tw, const int32_t *__restrict__ rop, void *out,
    int N, int d, int k, bool accumulate) {
    const int t = blockIdx.x;
    // the token's k <= 8 rows and weights: uniform addresses, so scalar loads
    // (slots past k repeat slot k-1 and are not added)
    int rs[8];
    float ws[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int jj = j < k ? j : k - 1;
        rs[j] = rop[(size_t)t * k + jj];
        ws[j] = tw[(size_t)t * k + jj];
    }
    const size_t shared_row = (size_t)N * k + t;
    for (int c = (blockIdx.y * blockDim.x + threadIdx.x) * 4; c < d; c += gridDim.y * blockDim.x * 4) {
        // all rows are requested at once, then added in slot order
        float4 a = load_y4<YBF16>(Y, shared_row * d + c);
        float4 y[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = load_y4<YBF16>(Y, (size_t)rs[j] * d + c);
#pragma unroll
        for (int j = 0; j < 8; ++j) {   // per-value selects, not branches: the loads stay ahead of every use
            const bool on = j < k;
            a.x = on ? fmaf(ws[j], y[j].x, a.x) : a.x;
            a.y = on ? fmaf(ws[j], y[j].y, a.y) : a.y;
            a.z = on ? fmaf(ws[j], y[j].z, a.z) : a.z;
            a.w = on ? fmaf(ws[j], y[j].w, a.w) : a.w;
        }
        if (BF16OUT) {
            uint2 *o = reinterpret_cast<uint2 *>((uint16_t *)out + (size_t)t * d + c);
            if (accumulate) {
                uint2 old = *o;
                a.x += bf16_lo(old.x); a.y += bf16_hi(old.x);
                a.z += bf16_lo(old.y); a.w += bf16_hi(old.y);
            }
            *o = make_uint2(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w));
        } else {
            float4 *o = reinterpret_cast<float4 *>((float *)out + (size_t)t * d + c);
            if (accumulate) {
                float4 old = *o;
                a.x += old.x; a.y += old.y; a.z += old.z; a.w += old.w;
            }
            *o = a;
        }
    }
}

hipError_t launch_combine(const Plan &p) {
    const bool acc = (p.flags & MOE_FLAG_ACCUMULATE) != 0;
    const bool ybf16 = !p.use_stream;  // the grouped GEMMs store Y in bfloat16
    dim3 grid(p.N, (p.d + 1023) / 1024), block(256);
#define FGS_COMBINE(OB, YB) hipLaunchKernelGGL((combine_kernel<OB, YB>), grid, block, 0, p.stream, p.Y, p.tw, p.rop, \
                                             p.out, p.N, p.d, p.k, acc)
    if (p.xdt == MOE_DTYPE_BF16) {
        if (ybf16) FGS_COMBINE(true, true); else FGS_COMBINE(true, false);
    } else {
        if (ybf16) FGS_COMBINE(false, true); else FGS_COMBINE(false, false);
    }
#undef FGS_COMBINE
    return hipGetLastError();
}

}  // namespace fgs
