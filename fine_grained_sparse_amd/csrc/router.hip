// Router logits h = x W_r^T in FP32.
//
// "Inside Kolibri 1" (flozi.net), section "Routing: selection bias and
// mixture weights are separate": the router maps flattened tokens [N, 2560] to
// FP32 logits [N, 384]; section "The FP8 path is explicitly mixed precision":
// the router output logits stay FP32.
//
// bfloat16 x: matrix cores.  Every FP32 router weight is split exactly into
// three bfloat16 terms w = hi + mid + lo (hi and mid by truncation, so each
// remainder is exact; lo takes the last <= 8 significant bits).  A product of
// two bfloat16 values is exact in FP32, so three bf16 MFMAs with FP32
// accumulation give an FP32-accurate logit at matrix-core rate.
//
// FP32 x: a plain FP32 FMA loop (small problems only).
//
// Batches above 64 tokens use the router GEMM of the expert-GEMM file (same
// split, with the operands staged through LDS).
//
// The logits are written as partial sums over `ks` contiguous k-slices,
// partial[s][t][e]; the top-k kernel adds the slices in a fixed order.  Small
// token counts use several slices so that the 3.9 MB router matrix is read by
// enough waves to stream it at full bandwidth.
#include "moe_common.h"
#include "moe_plan.h"

namespace fgs {

// split 8 FP32 weights into three bfloat16 x 8 fragments (exact sum)
__device__ __forceinline__ void split3(const float4 &a, const float4 &b, uint4 &hi, uint4 &mid, uint4 &lo) {
    float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t h[8], m[8], l[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t u = __float_as_uint(v[i]);
        uint32_t uh = u & 0xFFFF0000u;
        float r1 = v[i] - __uint_as_float(uh);
        uint32_t um = __float_as_uint(r1) & 0xFFFF0000u;
        float r2 = r1 - __uint_as_float(um);
        h[i] = uh >> 16;
        m[i] = um >> 16;
        l[i] = f32_to_bf16_rne(r2);
    }
    hi = make_uint4(h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16);
    mid = make_uint4(m[0] | m[1] << 16, m[2] | m[3] << 16, m[4] | m[5] << 16, m[6] | m[7] << 16);
    lo = make_uint4(l[0] | l[1] << 16, l[2] | l[3] << 16, l[4] | l[5] << 16, l[6] | l[7] << 16);
}

__device__ __forceinline__ f32x4_t mfma16x16x32(const uint4 &a, const uint4 &b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// One wave computes a (16*MT tokens) x (16*NT experts) tile over one k-slice.
// MFMA 16x16x32 operand layout: lane l feeds row (l % 16) of A and column
// (l % 16) of B with the 8 consecutive k at 8*(l / 16); both operands use the
// same k mapping, so the k order inside the instruction does not matter.
// Result: lane l holds D[4*(l/16) + i][l % 16], i = 0..3.
// KW > 1: a workgroup of KW waves per job, wave w taking the w-th of KW equal
// parts of the k-slice; the parts' sums are added in wave order through LDS
// (fewer bytes per wave in flight without more slices for the top-k to add).
template <int MT, int NT, int KW = 1>
__global__ __launch_bounds__(256) void router_mfma_kernel(
    const uint16_t *__restrict__ x, const float *__restrict__ rw, float *__restrict__ partial,
    int N, int d, int E, int kslice, int n_tb, int n_eb, int n_jobs, int32_t *route_cnt) {
    if (blockIdx.x == 0 && threadIdx.x == 0) *route_cnt = 0;   // for the top-k's last-workgroup dispatch
    const int lane = threadIdx.x & 63;
    const int kw = KW > 1 ? (int)(threadIdx.x >> 6) : 0;
    const int job = KW > 1 ? (int)blockIdx.x : (int)(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6));
    if (job >= n_jobs) return;
    const int tb = job % n_tb;
    const int rest = job / n_tb;
    const int eb = rest % n_eb;
    const int s = rest / n_eb;
    const int kpart = kslice / KW;
    const int t0 = tb * 16 * MT, e0 = eb * 16 * NT, k0 = s * kslice + kw * kpart;
    const int r = lane & 15, kq = (lane >> 4) * 8;

    const uint16_t *xrow[MT];
    bool xok[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        int t = t0 + 16 * i + r;
        xok[i] = t < N;
        xrow[i] = x + (size_t)(xok[i] ? t : 0) * d + k0 + kq;
    }
    const float *wrow[NT];
    bool wok[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        int e = e0 + 16 * j + r;
        wok[j] = e < E;
        wrow[j] = rw + (size_t)(wok[j] ? e : 0) * d + k0 + kq;
    }

    f32x4_t acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll 8
    for (int kk = 0; kk < kpart; kk += 32) {
        uint4 a[MT];
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            a[i] = *reinterpret_cast<const uint4 *>(xrow[i] + kk);
            if (!xok[i]) a[i] = make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            float4 w0 = *reinterpret_cast<const float4 *>(wrow[j] + kk);
            float4 w1 = *reinterpret_cast<const float4 *>(wrow[j] + kk + 4);
            if (!wok[j]) { w0 = make_float4(0.f, 0.f, 0.f, 0.f); w1 = w0; }
            uint4 hi, mid, lo;
            split3(w0, w1, hi, mid, lo);
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                acc[i][j] = mfma16x16x32(a[i], lo, acc[i][j]);
                acc[i][j] = mfma16x16x32(a[i], mid, acc[i][j]);
                acc[i][j] = mfma16x16x32(a[i], hi, acc[i][j]);
            }
        }
    }

    if constexpr (KW > 1) {   // the whole workgroup has a job: n_jobs workgroups
        __shared__ f32x4_t red[KW - 1][MT][NT][64];
        if (kw > 0)
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j) red[kw - 1][i][j][lane] = acc[i][j];
        __syncthreads();
        if (kw > 0) return;
#pragma unroll
        for (int w = 0; w < KW - 1; ++w)
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const f32x4_t o = red[w][i][j][lane];
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[i][j][q] += o[q];
                }
    }
    float *dst = partial + (size_t)s * N * E;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            int e = e0 + 16 * j + r;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                int t = t0 + 16 * i + (lane >> 4) * 4 + q;
                if (t < N && e < E) dst[(size_t)t * E + e] = acc[i][j][q];
            }
        }
}

// Plain FP32 FMA router for FP32 activations: one thread per (token, expert).
__global__ __launch_bounds__(256) void router_f32_kernel(
    const float *__restrict__ x, const float *__restrict__ rw, float *__restrict__ partial,
    int N, int d, int E, int32_t *route_cnt) {
    if (blockIdx.x == 0 && threadIdx.x == 0) *route_cnt = 0;   // for the top-k's last-workgroup dispatch
    long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long)N * E) return;
    int t = (int)(idx / E), e = (int)(idx % E);
    const float4 *xr = reinterpret_cast<const float4 *>(x + (size_t)t * d);
    const float4 *wr = reinterpret_cast<const float4 *>(rw + (size_t)e * d);
    float acc = 0.f;
    for (int i = 0; i < d / 4; ++i) {
        float4 a = xr[i], b = wr[i];
        acc = fmaf(a.x, b.x, acc);
        acc = fmaf(a.y, b.y, acc);
        acc = fmaf(a.z, b.z, acc);
        acc = fmaf(a.w, b.w, acc);
    }
    partial[idx] = acc;
}

hipError_t launch_router(const Plan &p) {
    if (p.xdt == MOE_DTYPE_F32) {
        long total = (long)p.N * p.E;
        dim3 grid((unsigned)((total + 255) / 256));
        hipLaunchKernelGGL(router_f32_kernel, grid, dim3(256), 0, p.stream,
                           (const float *)p.x, p.rw, p.partial, p.N, p.d, p.E, p.route_cnt);
        return hipGetLastError();
    }
    if (router_gemm(p.N, p.xdt)) return launch_router_gemm(p, p.w3);
    const uint16_t *x = (const uint16_t *)p.x;
    RouterTiling rt = router_tiling(p.N, p.d, p.E);
    int n_tb = (p.N + 16 * rt.mt - 1) / (16 * rt.mt);
    int n_eb = (p.E + 16 * rt.nt - 1) / (16 * rt.nt);
    int n_jobs = n_tb * n_eb * p.ks;
    if (rt.mt == 2) {
        // one wave per workgroup: the few hundred jobs of a small batch spread
        // over as many CUs, each pulling its slice of W_r with its own loads
        // several waves per job, each a part of the k-slice of 32 or more k
        // (N = 32, d = 2560: router 6.3 us with one wave, 5.1 with two, 4.8 with four)
        if (p.kslice % 128 == 0)
            hipLaunchKernelGGL((router_mfma_kernel<2, 1, 4>), dim3(n_jobs), dim3(256), 0, p.stream,
                               x, p.rw, p.partial, p.N, p.d, p.E, p.kslice, n_tb, n_eb, n_jobs, p.route_cnt);
        else if (p.kslice % 64 == 0)
            hipLaunchKernelGGL((router_mfma_kernel<2, 1, 2>), dim3(n_jobs), dim3(128), 0, p.stream,
                               x, p.rw, p.partial, p.N, p.d, p.E, p.kslice, n_tb, n_eb, n_jobs, p.route_cnt);
        else
            hipLaunchKernelGGL((router_mfma_kernel<2, 1>), dim3(n_jobs), dim3(64), 0, p.stream,
                               x, p.rw, p.partial, p.N, p.d, p.E, p.kslice, n_tb, n_eb, n_jobs, p.route_cnt);
    } else {
        dim3 grid((n_jobs + 3) / 4);
        hipLaunchKernelGGL((router_mfma_kernel<4, 4>), grid, dim3(256), 0, p.stream,
                           x, p.rw, p.partial, p.N, p.d, p.E, p.kslice, n_tb, n_eb, n_jobs, p.route_cnt);
    }
    return hipGetLastError();
}

}  // namespace fgs
