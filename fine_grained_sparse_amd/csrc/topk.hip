// Bias-corrected top-k selection and sigmoid mixture weights.
//
// "Inside Kolibri 1" (flozi.net), section "Routing: selection bias and
// mixture weights are separate": (1) add the learned expert-correction bias to
// the logits and select the top six ids; (2) gather the unbiased logits of
// those ids, apply a sigmoid and use the results as mixture weights without
// renormalising them.  With MOE_FLAG_RENORMALIZE the weights are instead the
// softmax of the selected unbiased logits ("Kolibri 1 Deep Dive",
// "Mathematical Routing & Load Balancing Formulation").
//
// One wave per token.  Lane l owns experts l, l+64, l+128, ...  Each of the
// k+1 rounds takes the wave-wide maximum of a 64-bit key built from the score
// (order-preserving bit map, -0 folded onto +0) and the complemented expert
// id, so equal scores go to the lower id and the result is independent of the
// reduction order.  A (k+1)-th round, run only when the gap is requested,
// yields the selection gap.
#include "dispatch_small.h"
#include "moe_common.h"
#include "moe_plan.h"

namespace fgs {

__device__ __forceinline__ uint32_t orderable(float s) {
    if (s == 0.0f) s = 0.0f;  // -0 and +0 compare equal
    uint32_t u = __float_as_uint(s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_orderable(uint32_t o) {
    uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
    return __uint_as_float(u);
}

// Selection and mixture weights of token t from its logits h[v] (lane l
// holds experts l + 64 v) and the biases bv[v]; writes ids, tw, gap and the
// optional logits of the token.
template <int VPL>
__device__ __forceinline__ void select_token(const float (&h)[VPL], const float (&bv)[VPL], int lane, int t, int E,
                                             int k, bool renorm, float *__restrict__ logits_out,
                                             int32_t *__restrict__ ids, float *__restrict__ tw,
                                             float *__restrict__ gap, int32_t *ids_lds = nullptr) {
    uint64_t key[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        const int e = lane + 64 * v;
        // the key is formed unconditionally (a select, no branch), so the bias
        // load cannot be sunk behind the partial sums
        const float sc = h[v] + bv[v];
        const uint64_t kv = ((uint64_t)orderable(sc) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
        key[v] = e < E ? kv : 0;  // 0 is below every real key
        if (e < E && logits_out) logits_out[(size_t)t * E + e] = h[v];
    }

    // k <= 8: fully unrolled rounds keep every array in registers
    int sel[8];
    float selh[8];
    float sk = 0.f, sk1 = 0.f;
    const int rounds = (gap && k < E) ? k + 1 : k;   // the extra round only measures the gap
#pragma unroll
    for (int r = 0; r < 9; ++r) {
        if (r < 8) { sel[r] = 0x7FFFFFFF; selh[r] = 0.f; }
        if (r >= rounds) continue;
        uint64_t best = 0;
#pragma unroll
        for (int v = 0; v < VPL; ++v) best = key[v] > best ? key[v] : best;
        best = wave_max_u64(best);
        const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
        const float sc = from_orderable((uint32_t)(best >> 32));
        if (r < k) {
            // the owner lane retires the winner; everybody learns its logit
            const int owner = e & 63, slot = e >> 6;
            float hv = 0.f;
#pragma unroll
            for (int v = 0; v < VPL; ++v) {
                if (v == slot) {
                    hv = h[v];
                    if (lane == owner) key[v] = 0;
                }
            }
            hv = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(hv), owner));
            if (r < 8) { sel[r] = e; selh[r] = hv; }
            sk = sc;
        } else {
            sk1 = sc;
        }
    }

    // ascending id order: compare-exchange network over the 8 slots (unused
    // slots hold INT_MAX and sink to the end)
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 7 - i; ++j) {
            if (sel[j] > sel[j + 1]) {
                int te = sel[j]; sel[j] = sel[j + 1]; sel[j + 1] = te;
                float th = selh[j]; selh[j] = selh[j + 1]; selh[j + 1] = th;
            }
        }
    // renormalised variant: exp(h_j - max) / sum over the selected ids, summed in slot order
    float hmax = -__builtin_inff(), zsum = 0.f;
    if (renorm) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < k) hmax = fmaxf(hmax, selh[j]);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < k) zsum += expf(selh[j] - hmax);
    }
    if (lane < k) {
        int e = 0;
        float hv = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j == lane) { e = sel[j]; hv = selh[j]; }
        ids[(size_t)t * k + lane] = e;
        if (ids_lds) ids_lds[t * k + lane] = e;
        tw[(size_t)t * k + lane] = renorm ? expf(hv - hmax) / zsum : sigmoidf_(hv);
    }
    if (gap && lane == 0) gap[t] = (k < E) ? sk - sk1 : __builtin_inff();
}

// Logits of one token from the router's k-slice partial sums (no split-term
// flags): slices added in order 0..ks-1 (ks <= 10).  Every load is issued up
// front from a valid address (experts past E read expert 0, slices past ks
// re-read slice ks-1) and masked afterwards, so the loads of all slices and
// experts are in flight together.
template <int VPL>
__device__ __forceinline__ void sum_slices(const float *row, size_t slice, int ks, int lane, int E, float (&h)[VPL]) {
    constexpr int kMaxSlices = 10;
    constexpr bool kAllAtOnce = VPL * kMaxSlices <= 60;
    float part[kAllAtOnce ? VPL : 1][kMaxSlices];
    if constexpr (kAllAtOnce) {
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            const int e = lane + 64 * v, ec = e < E ? e : 0;
#pragma unroll
            for (int s = 0; s < kMaxSlices; ++s) part[v][s] = row[(size_t)min(s, ks - 1) * slice + ec];
        }
    }
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        const int e = lane + 64 * v, ec = e < E ? e : 0;
        float p[kMaxSlices];
#pragma unroll
        for (int s = 0; s < kMaxSlices; ++s)
            p[s] = kAllAtOnce ? part[kAllAtOnce ? v : 0][s] : row[(size_t)min(s, ks - 1) * slice + ec];
        float acc = p[0];
#pragma unroll
        for (int s = 1; s < kMaxSlices; ++s) acc += s < ks ? p[s] : 0.0f;
        h[v] = acc;
    }
}

// FLAGS: partial sums from the router GEMM, whose mid/lo slices are skipped
// per rflags.  (Two or four tokens per wave, the next token's partial sums
// loaded while the current one is selected, measured slower: the selection
// rounds, not the loads, set the pace.)
template <int VPL, bool FLAGS>
__global__ __launch_bounds__(256) void topk_kernel(
    const float *__restrict__ partial, int ks, const int32_t *__restrict__ rflags, const float *__restrict__ bias,
    float *__restrict__ logits_out, int32_t *__restrict__ ids, float *__restrict__ tw,
    float *__restrict__ gap, int N, int E, int k, bool renorm) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (t >= N) return;
    const float *row = partial + (size_t)t * E;

    const size_t slice = (size_t)N * E;
    // the biases go out first, from clamped indices, so no load waits behind another
    // (with the router GEMM's split, rflags[e] == 0 says the slices of the mid
    // and lo terms, the last two thirds, are all zero for expert e: not added)
    float bv[VPL];
    int fl[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        const int e = lane + 64 * v;
        bv[v] = bias[e < E ? e : 0];
        fl[v] = FLAGS ? rflags[e < E ? e : 0] : 1;
    }

    if constexpr (!FLAGS) {
        float h[VPL];
        sum_slices<VPL>(row, slice, ks, lane, E, h);
        select_token<VPL>(h, bv, lane, t, E, k, renorm, logits_out, ids, tw, gap);
    } else {
        // hi-term slices (c = ks/3 <= 4) per token; the mid and lo slices (2c)
        // are fetched in a second round, and only when some expert of this
        // wave has nonzero terms there, so bf16-valued router weights cost
        // one pass over c slices.  Slices are added in order 0..ks-1.
        constexpr int kMaxHi = 4;
        const int hi = ks / 3;
        int need = 0;
#pragma unroll
        for (int v = 0; v < VPL; ++v) need |= (lane + 64 * v < E) && fl[v];
        float part[VPL][kMaxHi];
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            const int e = lane + 64 * v, ec = e < E ? e : 0;
#pragma unroll
            for (int s = 0; s < kMaxHi; ++s) part[v][s] = s < hi ? row[(size_t)s * slice + ec] : 0.0f;
        }
        float h[VPL];
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            float acc = part[v][0];
#pragma unroll
            for (int s = 1; s < kMaxHi; ++s) acc += s < hi ? part[v][s] : 0.0f;
            h[v] = acc;
        }
        if (__any(need)) {
#pragma unroll
            for (int v = 0; v < VPL; ++v) {
                const int e = lane + 64 * v, ec = e < E ? e : 0;
                float ml[2 * kMaxHi];
#pragma unroll
                for (int s = 0; s < 2 * kMaxHi; ++s)
                    ml[s] = (hi + s < ks && fl[v]) ? row[(size_t)(hi + s) * slice + ec] : 0.0f;
#pragma unroll
                for (int s = 0; s < 2 * kMaxHi; ++s) h[v] += ml[s];
            }
        }
        select_token<VPL>(h, bv, lane, t, E, k, renorm, logits_out, ids, tw, gap);
    }
}

// Top-k and dispatch in one launch for batches of at most kFusedRouteN tokens
// (router_mfma partial sums, no split-term flags): wave t selects token t's
// experts as topk_kernel does and keeps its ids in LDS; after a barrier the
// first wave lays out the dispatch (dispatch_small).  One launch less in the
// small-batch chain; the selections of a few tokens fit one CU.
template <int VPL>
__global__ __launch_bounds__(64 * kFusedRouteCap) void topk_dispatch_kernel(
    const float *__restrict__ partial, int ks, const float *__restrict__ bias, float *__restrict__ logits_out,
    int32_t *__restrict__ ids, float *__restrict__ tw, float *__restrict__ gap, int N, int E, int k, bool renorm,
    int32_t *g_offsets, int32_t *g_exp_off, int32_t *tiles, int32_t *n_tiles, int32_t *por, int32_t *rop) {
    __shared__ int32_t sids[kFusedRouteCap * 8];
    const int lane = threadIdx.x & 63, t = threadIdx.x >> 6;
    if (t < N) {
        float bv[VPL];
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            const int e = lane + 64 * v;
            bv[v] = bias[e < E ? e : 0];
        }
        float h[VPL];
        sum_slices<VPL>(partial + (size_t)t * E, (size_t)N * E, ks, lane, E, h);
        select_token<VPL>(h, bv, lane, t, E, k, renorm, logits_out, ids, tw, gap, sids);
    }
    __syncthreads();
    dispatch_small(sids, N, k, E, g_offsets, g_exp_off, tiles, n_tiles, por, rop);
}

// Top-k of one token per workgroup (one wave, router_mfma partial sums, no
// split-term flags) with the dispatch laid out by the workgroup that finishes
// last: each workgroup publishes its ids (release fence), counts itself on
// route_cnt (zeroed by this call's router kernel), and the one that brings
// the count to N reads every token's ids after an acquire fence and runs
// dispatch_small.  No workgroup waits for another.
template <int VPL>
__global__ __launch_bounds__(64) void topk_tail_kernel(
    const float *__restrict__ partial, int ks, const float *__restrict__ bias, float *__restrict__ logits_out,
    int32_t *ids, float *__restrict__ tw, float *__restrict__ gap, int N, int E, int k, bool renorm,
    int32_t *route_cnt, int32_t *g_offsets, int32_t *g_exp_off, int32_t *tiles, int32_t *n_tiles, int32_t *por,
    int32_t *rop) {
    const int lane = threadIdx.x, t = blockIdx.x;
    float bv[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        const int e = lane + 64 * v;
        bv[v] = bias[e < E ? e : 0];
    }
    float h[VPL];
    sum_slices<VPL>(partial + (size_t)t * E, (size_t)N * E, ks, lane, E, h);
    select_token<VPL>(h, bv, lane, t, E, k, renorm, logits_out, ids, tw, gap);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    int done = 0;
    if (lane == 0) done = __hip_atomic_fetch_add(route_cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    done = __shfl(done, 0, kWave);
    if (done != N - 1) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    dispatch_small(ids, N, k, E, g_offsets, g_exp_off, tiles, n_tiles, por, rop);
}

hipError_t launch_topk(const Plan &p) {
    // one token per wave; small batches put each wave in a workgroup of its own,
    // so the selections spread over as many CUs (N = 32: 6.0 against 7.1 us
    // with four waves per workgroup)
    const int wpb = p.N <= 64 ? 1 : 4;
    dim3 grid((p.N + wpb - 1) / wpb), block(64 * wpb);
    int vpl = (p.E + 63) / 64;
    if (p.fused_route) {   // top-k and dispatch in one workgroup of N waves
#define FGS_TOPKD(V)                                                                                          \
    hipLaunchKernelGGL((topk_dispatch_kernel<V>), dim3(1), dim3(64 * p.N), 0, p.stream, p.partial, p.ks, p.rb,   \
                       p.logits, p.ids, p.tw, p.gap, p.N, p.E, p.k, (p.flags & MOE_FLAG_RENORMALIZE) != 0,        \
                       p.offsets, p.exp_off_out, p.tiles, p.n_tiles, p.por, p.rop)
        if (vpl <= 1) FGS_TOPKD(1);
        else if (vpl <= 2) FGS_TOPKD(2);
        else if (vpl <= 4) FGS_TOPKD(4);
        else if (vpl <= 6) FGS_TOPKD(6);
        else if (vpl <= 8) FGS_TOPKD(8);
        else FGS_TOPKD(16);
#undef FGS_TOPKD
        return hipGetLastError();
    }
    if (p.tail_dispatch) {   // one wave per token, the last one lays out the dispatch
#define FGS_TOPKT(V)                                                                                        \
    hipLaunchKernelGGL((topk_tail_kernel<V>), dim3(p.N), dim3(64), 0, p.stream, p.partial, p.ks, p.rb, p.logits, \
                       p.ids, p.tw, p.gap, p.N, p.E, p.k, (p.flags & MOE_FLAG_RENORMALIZE) != 0, p.route_cnt,     \
                       p.offsets, p.exp_off_out, p.tiles, p.n_tiles, p.por, p.rop)
        if (vpl <= 1) FGS_TOPKT(1);
        else if (vpl <= 2) FGS_TOPKT(2);
        else if (vpl <= 4) FGS_TOPKT(4);
        else if (vpl <= 6) FGS_TOPKT(6);
        else if (vpl <= 8) FGS_TOPKT(8);
        else FGS_TOPKT(16);
#undef FGS_TOPKT
        return hipGetLastError();
    }
#define FGS_TOPK2(V, F)                                                                             \
    hipLaunchKernelGGL((topk_kernel<V, F>), grid, block, 0, p.stream, p.partial, p.ks, p.rflags, p.rb, \
                       p.logits, p.ids, p.tw, p.gap, p.N, p.E, p.k, (p.flags & MOE_FLAG_RENORMALIZE) != 0)
#define FGS_TOPK(V) do { if (p.rflags) FGS_TOPK2(V, true); else FGS_TOPK2(V, false); } while (0)
    if (vpl <= 1) FGS_TOPK(1);
    else if (vpl <= 2) FGS_TOPK(2);
    else if (vpl <= 4) FGS_TOPK(4);
    else if (vpl <= 6) FGS_TOPK(6);
    else if (vpl <= 8) FGS_TOPK(8);
    else FGS_TOPK(16);
#undef FGS_TOPK
#undef FGS_TOPK2
    return hipGetLastError();
}

}  // namespace fgs
