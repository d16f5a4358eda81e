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

// VEC consecutive values of Y as floats: 8 bf16 (16 bytes) or 4 FP32 (16
// bytes).  Y is read exactly once: non-temporal loads.
template <bool YBF16>
__device__ __forceinline__ void load_y(const void *Y, size_t elem, float (&v)[YBF16 ? 8 : 4]) {
    if constexpr (YBF16) {
        const uint4 q = ld_stream16((const uint16_t *)Y + elem);
        v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
        v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z); v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
    } else {
        const uint4 q = ld_stream16((const float *)Y + elem);
        v[0] = __uint_as_float(q.x); v[1] = __uint_as_float(q.y); v[2] = __uint_as_float(q.z); v[3] = __uint_as_float(q.w);
    }
}

// grid: (N, column blocks); each thread combines VEC consecutive columns per pass.
// KT: the top-k (6 or 8) as a constant, or 0 for any k <= 8 (slots past k then
// repeat slot k-1 and are not added)
template <bool BF16OUT, bool YBF16, int KT>
__global__ __launch_bounds__(1024) void combine_kernel(
    const void *__restrict__ Y, const float *__restrict__ tw, const int32_t *__restrict__ rop, void *out,
    int N, int d, int k_arg, bool accumulate) {
    constexpr int VEC = YBF16 ? 8 : 4;
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
    for (int c = (blockIdx.y * blockDim.x + threadIdx.x) * VEC; c < d; c += gridDim.y * blockDim.x * VEC) {
        // all rows are requested at once, then added in slot order
        float a[VEC], y[KS][VEC];
        load_y<YBF16>(Y, shared_row * d + c, a);
#pragma unroll
        for (int j = 0; j < KS; ++j) load_y<YBF16>(Y, (size_t)rs[j] * d + c, y[j]);
#pragma unroll
        for (int j = 0; j < KS; ++j) {   // per-value selects, not branches: the loads stay ahead of every use
            const bool on = j < k;
#pragma unroll
            for (int q = 0; q < VEC; ++q) a[q] = on ? fmaf(ws[j], y[j][q], a[q]) : a[q];
        }
        if (BF16OUT) {
            uint16_t *o = (uint16_t *)out + (size_t)t * d + c;
            uint32_t w[VEC / 2];
            if (accumulate) {
#pragma unroll
                for (int q = 0; q < VEC / 2; ++q) w[q] = reinterpret_cast<const uint32_t *>(o)[q];
#pragma unroll
                for (int q = 0; q < VEC / 2; ++q) { a[2 * q] += bf16_lo(w[q]); a[2 * q + 1] += bf16_hi(w[q]); }
            }
#pragma unroll
            for (int q = 0; q < VEC / 2; ++q) w[q] = pack_bf16x2(a[2 * q], a[2 * q + 1]);
            if constexpr (VEC == 8) *reinterpret_cast<uint4 *>(o) = make_uint4(w[0], w[1], w[2], w[3]);
            else *reinterpret_cast<uint2 *>(o) = make_uint2(w[0], w[1]);
        } else {
            float *o = (float *)out + (size_t)t * d + c;
#pragma unroll
            for (int q = 0; q < VEC; q += 4) {
                float4 v = make_float4(a[q], a[q + 1], a[q + 2], a[q + 3]);
                if (accumulate) {
                    const float4 old = *reinterpret_cast<const float4 *>(o + q);
                    v.x += old.x; v.y += old.y; v.z += old.z; v.w += old.w;
                }
                *reinterpret_cast<float4 *>(o + q) = v;
            }
        }
    }
}

hipError_t launch_combine(const Plan &p) {
    const bool acc = (p.flags & MOE_FLAG_ACCUMULATE) != 0;
    const bool ybf16 = !p.use_stream;  // the grouped GEMMs store Y in bfloat16
    // stream path (FP32 Y, small N): 256 threads x 4 columns per block, several
    // blocks per token; GEMM path (bf16 Y): one block per token covering the row
    // in 8-column pieces (d = 2560: 320 threads)
    const int vec = ybf16 ? 8 : 4;
    const int threads = ybf16 ? min(1024, ((p.d / vec + 63) / 64) * 64) : 256;
    dim3 grid(p.N, (p.d + threads * vec - 1) / (threads * vec)), block(threads);
#define FGS_COMBINE2(OB, YB, KT) hipLaunchKernelGGL((combine_kernel<OB, YB, KT>), grid, block, 0, p.stream, p.Y, p.tw, \
                                                  p.rop, p.out, p.N, p.d, p.k, acc)
#define FGS_COMBINE(OB, YB)                                       \
    do {                                                          \
        if (p.k == 6) FGS_COMBINE2(OB, YB, 6);                    \
        else if (p.k == 8) FGS_COMBINE2(OB, YB, 8);               \
        else FGS_COMBINE2(OB, YB, 0);                             \
    } while (0)
    if (p.xdt == MOE_DTYPE_BF16) {
        if (ybf16) FGS_COMBINE(true, true); else FGS_COMBINE(true, false);
    } else {
        if (ybf16) FGS_COMBINE(false, true); else FGS_COMBINE(false, false);
    }
#undef FGS_COMBINE
#undef FGS_COMBINE2
    return hipGetLastError();
}

}  // namespace fgs
