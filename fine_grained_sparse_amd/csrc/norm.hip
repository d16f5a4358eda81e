// Sandwich normalisation around the MoE sublayer.
//
// "Inside Kolibri 1" (flozi.net), section "The released stack": RMSNorm
// before and after the MoE sublayer, with the residual addition after it.
//   prenorm:        x = RMSNorm(r; g_pre), rounded to the activation type; the
//                   rest of the layer reads x.
//   combine_block:  the weighted unpermute of one token's expert outputs
//                   (shared, then slots in order, FP32), its RMSNorm with
//                   g_post and the residual add, rounded once, written back
//                   over the residual row.
// RMSNorm(v; g)_i = v_i / sqrt(mean(v^2) + eps) * g_i, statistics in FP32.
#include "moe_common.h"
#include "moe_plan.h"

namespace fgs {

// sum over the 256 threads of a workgroup (4 waves); every thread gets it
__device__ __forceinline__ float block_sum_256(float v, float *red) {
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    const float s = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();
    return s;
}

template <bool XBF16>
__device__ __forceinline__ float4 load_row4(const void *p, size_t i) {
    if constexpr (XBF16) {
        const uint2 v = *reinterpret_cast<const uint2 *>((const uint16_t *)p + i);
        return make_float4(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y));
    } else {
        return *reinterpret_cast<const float4 *>((const float *)p + i);
    }
}
template <bool XBF16>
__device__ __forceinline__ void store_row4(void *p, size_t i, float4 a) {
    if constexpr (XBF16)
        *reinterpret_cast<uint2 *>((uint16_t *)p + i) = make_uint2(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w));
    else
        *reinterpret_cast<float4 *>((float *)p + i) = a;
}

// grid: N; block 256
template <bool XBF16>
__global__ __launch_bounds__(256) void prenorm_kernel(const void *__restrict__ resid, const float *__restrict__ g,
                                                      float eps, void *__restrict__ xn, int d) {
    __shared__ float red[4];
    const size_t row = (size_t)blockIdx.x * d;
    float ss = 0.f;
    for (int c = threadIdx.x * 4; c < d; c += 1024) {
        const float4 a = load_row4<XBF16>(resid, row + c);
        ss = fmaf(a.x, a.x, fmaf(a.y, a.y, fmaf(a.z, a.z, fmaf(a.w, a.w, ss))));
    }
    const float inv = 1.0f / sqrtf(block_sum_256(ss, red) / (float)d + eps);
    for (int c = threadIdx.x * 4; c < d; c += 1024) {
        const float4 a = load_row4<XBF16>(resid, row + c);
        const float4 w = *reinterpret_cast<const float4 *>(g + c);
        store_row4<XBF16>(xn, row + c, make_float4(a.x * inv * w.x, a.y * inv * w.y, a.z * inv * w.z, a.w * inv * w.w));
    }
}

// four values of Y as floats; Y is read exactly once: non-temporal loads
template <bool YBF16>
__device__ __forceinline__ float4 load_y4n(const void *Y, size_t elem) {
    if constexpr (YBF16) {
        const uint2 v = ld_stream8((const uint16_t *)Y + elem);
        return make_float4(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y));
    } else {
        const uint4 v = ld_stream16((const float *)Y + elem);
        return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
    }
}

// grid: N; block 256; dynamic LDS d floats (the token's layer output).
// KT: the top-k (6 or 8) as a constant, or 0 for any k <= 8 (slots past k
// then repeat slot k-1 and are not added)
template <bool XBF16, bool YBF16, int KT>
__global__ __launch_bounds__(256) void combine_block_kernel(const void *__restrict__ Y, const float *__restrict__ tw,
                                                            const int32_t *__restrict__ rop,
                                                            const float *__restrict__ g, float eps, void *resid,
                                                            int N, int d, int k_arg) {
    extern __shared__ float yrow[];
    __shared__ float red[4];
    constexpr int KS = KT ? KT : 8;   // slots loaded
    const int k = KT ? KT : k_arg;
    const int t = blockIdx.x;
    // the token's rows and weights: uniform addresses, so scalar loads
    int rs[KS];
    float ws[KS];
#pragma unroll
    for (int j = 0; j < KS; ++j) {
        const int jj = j < k ? j : k - 1;
        rs[j] = rop[(size_t)t * k + jj];
        ws[j] = tw[(size_t)t * k + jj];
    }
    const size_t shared_row = (size_t)N * k + t;
    float ss = 0.f;
    for (int c = threadIdx.x * 4; c < d; c += 1024) {
        // every slot's row requested at once, added in slot order
        float4 a = load_y4n<YBF16>(Y, shared_row * d + c);
        float4 y[KS];
#pragma unroll
        for (int j = 0; j < KS; ++j) y[j] = load_y4n<YBF16>(Y, (size_t)rs[j] * d + c);
#pragma unroll
        for (int j = 0; j < KS; ++j) {   // per-value selects, not branches: the loads stay ahead of every use
            const bool on = j < k;
            a.x = on ? fmaf(ws[j], y[j].x, a.x) : a.x;
            a.y = on ? fmaf(ws[j], y[j].y, a.y) : a.y;
            a.z = on ? fmaf(ws[j], y[j].z, a.z) : a.z;
            a.w = on ? fmaf(ws[j], y[j].w, a.w) : a.w;
        }
        *reinterpret_cast<float4 *>(yrow + c) = a;
        ss = fmaf(a.x, a.x, fmaf(a.y, a.y, fmaf(a.z, a.z, fmaf(a.w, a.w, ss))));
    }
    const float inv = 1.0f / sqrtf(block_sum_256(ss, red) / (float)d + eps);
    const size_t row = (size_t)t * d;
    for (int c = threadIdx.x * 4; c < d; c += 1024) {
        const float4 a = *reinterpret_cast<const float4 *>(yrow + c);
        const float4 w = *reinterpret_cast<const float4 *>(g + c);
        const float4 r = load_row4<XBF16>(resid, row + c);
        store_row4<XBF16>(resid, row + c,
                          make_float4(r.x + a.x * inv * w.x, r.y + a.y * inv * w.y, r.z + a.z * inv * w.z,
                                      r.w + a.w * inv * w.w));
    }
}

hipError_t launch_prenorm(const Plan &p, const void *resid, const float *g, float eps, void *xn) {
    if (p.xdt == MOE_DTYPE_BF16)
        hipLaunchKernelGGL((prenorm_kernel<true>), dim3(p.N), dim3(256), 0, p.stream, resid, g, eps, xn, p.d);
    else
        hipLaunchKernelGGL((prenorm_kernel<false>), dim3(p.N), dim3(256), 0, p.stream, resid, g, eps, xn, p.d);
    return hipGetLastError();
}

hipError_t launch_combine_block(const Plan &p) {
    const size_t lds = (size_t)p.d * sizeof(float);
    const bool ybf16 = !p.use_stream;
#define FGS_CB2(XB, YB, KT) hipLaunchKernelGGL((combine_block_kernel<XB, YB, KT>), dim3(p.N), dim3(256), lds, \
                                               p.stream, p.Y, p.tw, p.rop, p.norm_post, p.eps, p.out, p.N, p.d, p.k)
#define FGS_CB(XB, YB)                                 \
    do {                                               \
        if (p.k == 6) FGS_CB2(XB, YB, 6);              \
        else if (p.k == 8) FGS_CB2(XB, YB, 8);         \
        else FGS_CB2(XB, YB, 0);                       \
    } while (0)
    if (p.xdt == MOE_DTYPE_BF16) {
        if (ybf16) FGS_CB(true, true); else FGS_CB(true, false);
    } else {
        if (ybf16) FGS_CB(false, true); else FGS_CB(false, false);
    }
#undef FGS_CB
#undef FGS_CB2
    return hipGetLastError();
}

}  // namespace fgs
