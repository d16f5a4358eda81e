// Decode-shaped expert path: stream only the touched experts' weight rows.
//
// "Inside Kolibri 1" (flozi.net), section "Routing: selection bias and
// mixture weights are separate": each routed or shared expert is a SwiGLU MLP,
// two 2560 -> 512 projections forming SiLU(gate) x up, then 512 -> 2560; a
// token touches six routed experts plus the shared one, and sparse activation
// lowers the weight traffic per token.  "Kolibri 1 Deep Dive"
// (abrarakhunji.com), section 1: the unselected experts stay idle in memory.
//
// For small batches each touched expert holds only a few token rows, so the
// layer is bound by reading the touched experts' weights once from HBM.  The
// kernels here give every workgroup a slice of one expert's weight rows, keep
// those rows in registers (16-byte coalesced loads: consecutive lanes read
// consecutive 16-byte chunks of a row), and dot them against that expert's
// token rows staged in LDS.  Cross-lane sums use a butterfly reduce-scatter:
// at each halving step a lane keeps half of its partial sums and trades the
// other half with its partner, so V sums over 64 lanes cost about V shuffles.
//
// Work list: one tile per non-empty group (routed experts, and the shared
// expert as group E with all N tokens), written by the dispatch scan.
#include "moe_common.h"
#include "moe_plan.h"

namespace fgs {

// Reduce-scatter V partial sums (V a power of two <= 64) over the wave.
// On return v[0] of lane l holds the full sum of value index
// butterfly_index<V>(l).
template <int V>
__device__ __forceinline__ void butterfly_reduce(float (&v)[V]) {
    int n = V;
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
        if (n > 1) {
            const bool upper = (threadIdx.x & s) != 0;
            const int h = n / 2;
#pragma unroll
            for (int i = 0; i < V / 2; ++i) {
                if (i < h) {
                    float send = upper ? v[i] : v[i + h];
                    float keep = upper ? v[i + h] : v[i];
                    v[i] = keep + __shfl_xor(send, s, kWave);
                }
            }
            n = h;
        } else {
            v[0] += __shfl_xor(v[0], s, kWave);
        }
    }
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

template <bool FP8> struct WChunk;            // 8 weights of one row
template <> struct WChunk<false> { typedef uint4 T; };
template <> struct WChunk<true> { typedef uint2 T; };

template <bool FP8>
__device__ __forceinline__ typename WChunk<FP8>::T load_chunk(const void *base, size_t elem_off) {
    if constexpr (FP8) return *reinterpret_cast<const uint2 *>((const uint8_t *)base + elem_off);
    else return *reinterpret_cast<const uint4 *>((const uint16_t *)base + elem_off);
}
template <bool FP8>
__device__ __forceinline__ float dot8(const typename WChunk<FP8>::T &w, const uint4 &x, float c) {
    if constexpr (FP8) return dot8_e4m3_bf16(w, x, c);
    else return dot8_bf16(w, x, c);
}

// 8 activations -> bfloat16 x 8 (FP32 x is rounded to nearest even)
__device__ __forceinline__ uint4 load_x8(const void *x, int xdt, size_t elem_off) {
    if (xdt == MOE_DTYPE_BF16) return *reinterpret_cast<const uint4 *>((const uint16_t *)x + elem_off);
    const float4 *p = reinterpret_cast<const float4 *>((const float *)x + elem_off);
    float4 a = p[0], b = p[1];
    return make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y), pack_bf16x2(b.z, b.w));
}

constexpr int kGuTC = 8;   // token rows staged per pass (gate/up)
constexpr int kGuRB = 8;   // H columns per workgroup (2 per wave)

// grid: (tile list capacity, ceil(max(f, fs) / 8)); block 256; dynamic LDS kGuTC*d*2 bytes
template <int CPL, bool FP8>
__global__ __launch_bounds__(256) void gate_up_stream_kernel(
    const void *__restrict__ x, int xdt, const void *__restrict__ wg, const void *__restrict__ wu,
    const float *__restrict__ sg, const float *__restrict__ su, const void *__restrict__ wsg,
    const void *__restrict__ wsu, const float *__restrict__ ssg, const float *__restrict__ ssu,
    const int32_t *__restrict__ tiles, const int32_t *__restrict__ n_tiles, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ por, uint16_t *__restrict__ H, int ldh, int d, int E, int k, int f, int fs,
    int bm) {
    extern __shared__ uint4 xs[];  // [kGuTC][d/8]
    const int u = blockIdx.x;
    if (u >= *n_tiles) return;
    const int g = tiles[2 * u];
    const bool shared = g == E;
    const int fg = shared ? fs : f;
    if ((int)blockIdx.y * kGuRB >= fg) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c0 = blockIdx.y * kGuRB + wave * 2;
    const int gstart = offsets[g], m0 = tiles[2 * u + 1];
    const int row0 = gstart + m0, m = min(bm, offsets[g + 1] - row0);
    const int nch = d / 8;

    // this wave's 4 weight rows: gate c0, c0+1, up c0, c0+1
    const void *gbase = shared ? wsg : wg;
    const void *ubase = shared ? wsu : wu;
    const size_t rbase = shared ? 0 : (size_t)g * f;
    typename WChunk<FP8>::T w[4][CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int ch = lane + 64 * i;
        const bool ok = ch < nch;
        const int chc = ok ? ch : 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const void *b = r < 2 ? gbase : ubase;
            w[r][i] = load_chunk<FP8>(b, (rbase + c0 + (r & 1)) * (size_t)d + (size_t)chc * 8);
            if (!ok) w[r][i] = typename WChunk<FP8>::T{};
        }
    }
    float scl[4] = {1.f, 1.f, 1.f, 1.f};
    if (FP8) {
        const float *gs = shared ? ssg : sg + (size_t)g * f;
        const float *us = shared ? ssu : su + (size_t)g * f;
        scl[0] = gs[c0]; scl[1] = gs[c0 + 1]; scl[2] = us[c0]; scl[3] = us[c0 + 1];
    }

    for (int tc0 = 0; tc0 < m; tc0 += kGuTC) {
        const int mc = min(kGuTC, m - tc0);
        __syncthreads();
        for (int idx = threadIdx.x; idx < mc * nch; idx += blockDim.x) {
            const int tok = idx / nch, ch = idx - tok * nch;
            const int r = row0 + tc0 + tok;
            const int t = shared ? (r - gstart) : por[r] / k;
            xs[tok * nch + ch] = load_x8(x, xdt, (size_t)t * d + (size_t)ch * 8);
        }
        __syncthreads();
        float acc[4 * kGuTC];
#pragma unroll
        for (int i = 0; i < 4 * kGuTC; ++i) acc[i] = 0.f;
#pragma unroll
        for (int t = 0; t < kGuTC; ++t) {
            if (t < mc) {
#pragma unroll
                for (int i = 0; i < CPL; ++i) {
                    const int ch = lane + 64 * i;
                    if (ch < nch) {
                        const uint4 xv = xs[t * nch + ch];
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[r * kGuTC + t] = dot8<FP8>(w[r][i], xv, acc[r * kGuTC + t]);
                    }
                }
            }
        }
        butterfly_reduce<4 * kGuTC>(acc);
        // lane holds value (r, t) = idx / kGuTC, idx % kGuTC; gate r in {0,1}, up r + 2
        const int idx = butterfly_index<4 * kGuTC>(lane);
        const float upv = __shfl_xor(acc[0], 32, kWave);  // up partner differs in the top index bit
        const int r = idx / kGuTC, t = idx % kGuTC;
        if (r < 2 && (lane & 1) == 0 && t < mc) {
            const float gv = acc[0] * (r ? scl[1] : scl[0]);
            const float uv = upv * (r ? scl[3] : scl[2]);
            const float hv = silu(gv) * uv;
            H[(size_t)(row0 + tc0 + t) * ldh + c0 + r] = (uint16_t)f32_to_bf16_rne(hv);
        }
    }
}

constexpr int kDnTC = 16;  // H rows staged per pass (down)
constexpr int kDnRW = 16;  // output rows per wave

// grid: (tile list capacity, d / 64); block 256.  Needs f, fs <= 512.
template <bool FP8>
__global__ __launch_bounds__(256) void down_stream_kernel(
    const uint16_t *__restrict__ H, int ldh, const void *__restrict__ wd, const float *__restrict__ sd,
    const void *__restrict__ wsd, const float *__restrict__ ssd, const int32_t *__restrict__ tiles,
    const int32_t *__restrict__ n_tiles, const int32_t *__restrict__ offsets, float *__restrict__ Y, int d, int E,
    int f, int fs, int bm) {
    __shared__ uint4 hs[kDnTC * 64];  // [kDnTC][fg/8], fg <= 512
    const int u = blockIdx.x;
    if (u >= *n_tiles) return;
    const int g = tiles[2 * u];
    const bool shared = g == E;
    const int fg = shared ? fs : f;
    const int nch = fg / 8;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int o0 = blockIdx.y * 64 + wave * kDnRW;
    const int row0 = offsets[g] + tiles[2 * u + 1], m = min(bm, offsets[g + 1] - row0);

    const void *base = shared ? wsd : wd;
    const size_t obase = shared ? 0 : (size_t)g * d;
    const bool ok = lane < nch;
    typename WChunk<FP8>::T w[kDnRW];
#pragma unroll
    for (int r = 0; r < kDnRW; ++r) {
        w[r] = load_chunk<FP8>(base, (obase + o0 + r) * (size_t)fg + (size_t)(ok ? lane : 0) * 8);
        if (!ok) w[r] = typename WChunk<FP8>::T{};
    }
    const int myrow = butterfly_index<kDnRW>(lane);
    float scl = 1.f;
    if (FP8) scl = shared ? ssd[o0 + myrow] : sd[obase + o0 + myrow];

    for (int tc0 = 0; tc0 < m; tc0 += kDnTC) {
        const int mc = min(kDnTC, m - tc0);
        __syncthreads();
        for (int idx = threadIdx.x; idx < mc * nch; idx += blockDim.x) {
            const int tok = idx / nch, ch = idx - tok * nch;
            hs[tok * 64 + ch] = *reinterpret_cast<const uint4 *>(H + (size_t)(row0 + tc0 + tok) * ldh + ch * 8);
        }
        __syncthreads();
        for (int t = 0; t < mc; ++t) {
            const uint4 hv = ok ? hs[t * 64 + lane] : make_uint4(0, 0, 0, 0);
            float p[kDnRW];
#pragma unroll
            for (int r = 0; r < kDnRW; ++r) p[r] = dot8<FP8>(w[r], hv, 0.f);
            butterfly_reduce<kDnRW>(p);
            if ((lane & 3) == 0) Y[(size_t)(row0 + tc0 + t) * d + o0 + myrow] = p[0] * scl;
        }
    }
}

hipError_t launch_gate_up(const Plan &p) {
    const int fmax = p.f > p.fs ? p.f : p.fs;
    dim3 grid(p.max_tiles, (fmax + kGuRB - 1) / kGuRB), block(256);
    const size_t lds = (size_t)kGuTC * p.d * 2;
    const int cpl = (p.d / 8 + 63) / 64;
    const bool fp8 = p.wdt == MOE_DTYPE_FP8_E4M3;
#define FGS_GU(C, F8)                                                                                          \
    hipLaunchKernelGGL((gate_up_stream_kernel<C, F8>), grid, block, lds, p.stream, p.x, p.xdt, p.W.w_gate,    \
                       p.W.w_up, p.W.s_gate, p.W.s_up, p.W.ws_gate, p.W.ws_up, p.W.ss_gate, p.W.ss_up, p.tiles, \
                       p.n_tiles, p.offsets, p.por, p.H, p.ldh, p.d, p.E, p.k, p.f, p.fs, p.bm)
#define FGS_GU_C(C) do { if (fp8) FGS_GU(C, true); else FGS_GU(C, false); } while (0)
    switch (cpl) {
        case 1: FGS_GU_C(1); break;
        case 2: FGS_GU_C(2); break;
        case 3: FGS_GU_C(3); break;
        case 4: FGS_GU_C(4); break;
        case 5: FGS_GU_C(5); break;
        case 6: FGS_GU_C(6); break;
        case 7: FGS_GU_C(7); break;
        case 8: FGS_GU_C(8); break;
        default: return hipErrorInvalidValue;
    }
#undef FGS_GU_C
#undef FGS_GU
    return hipGetLastError();
}

hipError_t launch_down(const Plan &p) {
    dim3 grid(p.max_tiles, p.d / 64), block(256);
    if (p.wdt == MOE_DTYPE_FP8_E4M3)
        hipLaunchKernelGGL((down_stream_kernel<true>), grid, block, 0, p.stream, p.H, p.ldh, p.W.w_down, p.W.s_down,
                           p.W.ws_down, p.W.ss_down, p.tiles, p.n_tiles, p.offsets, p.Y, p.d, p.E, p.f, p.fs, p.bm);
    else
        hipLaunchKernelGGL((down_stream_kernel<false>), grid, block, 0, p.stream, p.H, p.ldh, p.W.w_down, p.W.s_down,
                           p.W.ws_down, p.W.ss_down, p.tiles, p.n_tiles, p.offsets, p.Y, p.d, p.E, p.f, p.fs, p.bm);
    return hipGetLastError();
}

}  // namespace fgs
