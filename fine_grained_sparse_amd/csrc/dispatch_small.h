// Dispatch of a batch of at most 64 tokens by one wave (every group within one
// tile), shared by the dispatch kernels and the fused top-k + dispatch kernel.
//
// "Inside Kolibri 1" (flozi.net), section "Routing: selection bias and
// mixture weights are separate": token-choice routing with no per-expert
// capacity, so the per-expert row counts are whatever the selection produced.
// Layout as in dispatch.hip: a stable counting sort of pairs t*k + j by
// expert id, the shared expert as group E (rows N*k .. N*k + N), and the tile
// list (shared group first, then the non-empty experts in id order).
#pragma once

#include "moe_common.h"

namespace fgs {

// The k <= 8 expert ids of token t in registers: all loads issued at once
// (slots past k repeat slot k-1; a thread without a token reads token 0).
__device__ __forceinline__ void load_token_ids(const int32_t *ids, int t, int k, bool live, int (&e)[8]) {
    const int32_t *p = ids + (size_t)(live ? t : 0) * k;
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = p[j < k ? j : k - 1];
}

// inclusive prefix sum over the 64 lanes
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
        const int o = __shfl_up(v, s, kWave);
        if (lane >= s) v += o;
    }
    return v;
}

// The first wave of the workgroup does the work, lane t holding token t; the
// other waves (if any) only take part in the workgroup barriers.  Per-expert
// counts and 64-bit token masks come from LDS atomics; the offsets and the
// tile list are wave-wide prefix sums over 16 experts per lane; a token's rank
// in its expert is the popcount of the mask below it.  `ids` may be global
// memory or LDS.
__device__ __forceinline__ void dispatch_small(const int32_t *ids, int N, int k, int E, int32_t *g_offsets,
                                               int32_t *g_exp_off, int32_t *tiles, int32_t *n_tiles, int32_t *por,
                                               int32_t *rop) {
    __shared__ int cnt[1024];
    __shared__ unsigned long long mask[1024];
    __shared__ int off[1024];
    const bool w0 = threadIdx.x < 64;
    const int lane = threadIdx.x & 63;
    const bool live = w0 && lane < N;
    int my[8];
    load_token_ids(ids, lane, k, live, my);
    if (w0)
        for (int e = lane; e < E; e += 64) { cnt[e] = 0; mask[e] = 0ull; }
    __syncthreads();
    if (live) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < k) {
                atomicAdd(&cnt[my[j]], 1);
                atomicOr(&mask[my[j]], 1ull << lane);
            }
    }
    __syncthreads();
    if (w0) {
        // lane l owns experts [C l, C l + C): exclusive offsets and tile slots
        const int C = (E + 63) / 64;   // <= 16
        int c[16], sum = 0, nonempty = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int e = C * lane + i;
            c[i] = (i < C && e < E) ? cnt[e] : 0;
            sum += c[i];
            nonempty += c[i] > 0;
        }
        const int base = wave_inclusive_scan(sum) - sum;
        const int tbase = wave_inclusive_scan(nonempty) - nonempty;   // routed tiles before this lane's experts
        const int total = N * k;
        int run = base, trun = 1 + tbase;   // tile 0 is the shared group
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int e = C * lane + i;
            if (i < C && e < E) {
                off[e] = run;
                g_offsets[e] = run;
                if (g_exp_off) g_exp_off[e] = run;
                if (c[i] > 0) {
                    tiles[2 * trun] = e;
                    tiles[2 * trun + 1] = 0;
                    ++trun;
                }
                run += c[i];
            }
        }
        if (lane == 63) *n_tiles = trun;   // the last lane's running count is the total
        if (lane == 0) {
            g_offsets[E] = total;
            g_offsets[E + 1] = total + N;
            if (g_exp_off) g_exp_off[E] = total;
            tiles[0] = E;
            tiles[1] = 0;
        }
    }
    __syncthreads();
    // rank of token t among expert e's tokens: the tokens below t in e's mask
    if (live) {
        const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j >= k) break;
            const int e = my[j];
            const int pos = off[e] + __popcll(mask[e] & below);
            por[pos] = lane * k + j;
            rop[(size_t)lane * k + j] = pos;
        }
    }
}

}  // namespace fgs
