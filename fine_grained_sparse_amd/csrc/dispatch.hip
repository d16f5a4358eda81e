// Token-choice dispatch without capacity: histogram -> scan -> stable scatter.
//
// "Inside Kolibri 1" (flozi.net), section "Routing: selection bias and
// mixture weights are separate": routing is token-choice top-k with no exact
// per-batch capacity per expert, so every (token, slot) pair is kept and the
// per-expert row counts are whatever the selection produced (zero included).
//
// Layout (a stable counting sort of pairs p = t*k + j by expert id):
//   offsets[e]      first row of expert e; offsets[E] = N*k
//   offsets[E+1]    = N*k + N: rows [N*k, N*k + N) belong to the shared
//                   expert, token t at row N*k + t (the "group" E)
//   pair_of_row[r]  pair stored at row r;  row_of_pair[p] its inverse
// Within an expert, rows follow increasing token index.  The rank of a pair
// inside its 256-token block comes from a per-expert token bitmap (popcount of
// the lower tokens), so no atomic order ever reaches the output.
//
// The scan also writes the tile list of the expert kernels: one entry
// (group, first row within the group) per `bm` rows of every non-empty group,
// shared group first, then routed experts in id order.
#include "dispatch_small.h"
#include "moe_common.h"
#include "moe_plan.h"

namespace fgs {

constexpr int kBT = 256;     // tokens per dispatch block
constexpr int kBTW = kBT / 32;

// Exclusive scan of v[0..L) in LDS, L <= 2 * blockDim.x, blockDim.x == 1024.
// Returns the total.  `wsum` needs 16 ints.
__device__ int block_exclusive_scan_1024(int *v, int L, int *wsum) {
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int i0 = 2 * tid;
    int a = i0 < L ? v[i0] : 0;
    int b = i0 + 1 < L ? v[i0 + 1] : 0;
    int local = a + b;
    int inc = local;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
        int o = __shfl_up(inc, s, kWave);
        if (lane >= s) inc += o;
    }
    if (lane == 63) wsum[wid] = inc;
    __syncthreads();
    if (wid == 0) {
        int w = lane < 16 ? wsum[lane] : 0;
        int winc = w;
#pragma unroll
        for (int s = 1; s < 16; s <<= 1) {
            int o = __shfl_up(winc, s, kWave);
            if (lane >= s) winc += o;
        }
        if (lane < 16) wsum[lane] = winc - w;  // exclusive wave bases
        if (lane == 15) wsum[16] = winc;       // total
    }
    __syncthreads();
    int base = wsum[wid] + inc - local;
    if (i0 < L) v[i0] = base;
    if (i0 + 1 < L) v[i0 + 1] = base + a;
    int total = wsum[16];
    __syncthreads();
    return total;
}

// After `cnt[0..E)` holds per-expert counts (LDS): offsets, tile list.
// Leaves offsets in off[0..E+2).  PER_TILE: the tile list is written one
// thread per tile (large batches), else one thread per group.
template <bool PER_TILE>
__device__ void tile_list(const int *off, int *ntile, int *wsum, int E, int bm, int32_t *tiles, int32_t *n_tiles);

template <bool PER_TILE>
__device__ void offsets_and_tiles(const int *cnt, int *off, int *ntile, int *wsum, int N, int k, int E,
                                  int bm, int32_t *g_offsets, int32_t *g_exp_off, int32_t *tiles,
                                  int32_t *n_tiles, int32_t *tiles2 = nullptr, int32_t *n_tiles2 = nullptr) {
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += blockDim.x) off[e] = cnt[e];
    __syncthreads();
    int total = block_exclusive_scan_1024(off, E, wsum);
    if (tid == 0) {
        off[E] = total;          // == N*k
        off[E + 1] = total + N;  // shared expert rows
    }
    __syncthreads();
    for (int e = tid; e < E + 2; e += blockDim.x) {
        g_offsets[e] = off[e];
        if (g_exp_off && e <= E) g_exp_off[e] = off[e];
    }
    tile_list<PER_TILE>(off, ntile, wsum, E, bm, tiles, n_tiles);
    // with 256-row gate/up tiles: the down product's 128-row list as well
    if (tiles2) {
        __syncthreads();
        tile_list<PER_TILE>(off, ntile, wsum, E, bm / 2, tiles2, n_tiles2);
    }
}

// The tile list of `bm` rows per tile: tiles per group; the shared group (E, N
// rows, the most rows per expert at small N) is listed first so its
// workgroups start first.  Slot 0 of ntile[] is the shared group, slot 1 + e
// the routed expert e.
template <bool PER_TILE>
__device__ void tile_list(const int *off, int *ntile, int *wsum, int E, int bm, int32_t *tiles, int32_t *n_tiles) {
    const int tid = threadIdx.x;
    for (int q = tid; q <= E; q += blockDim.x) {
        const int g = q == 0 ? E : q - 1;
        const int m = off[g + 1] - off[g];
        ntile[q] = (m + bm - 1) / bm;
    }
    __syncthreads();
    int nt = block_exclusive_scan_1024(ntile, E + 1, wsum);
    if constexpr (PER_TILE) {
        // one thread per tile: its slot q is the last one whose first tile is
        // at or before it (an empty slot shares its successor's start and
        // loses the tie); no thread walks a long group alone
        for (int s = tid; s < nt; s += blockDim.x) {
            int lo = 0, hi = E;   // ntile[lo] <= s; find the largest such q
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (ntile[mid] <= s) lo = mid; else hi = mid - 1;
            }
            tiles[2 * s] = lo == 0 ? E : lo - 1;
            tiles[2 * s + 1] = (s - ntile[lo]) * bm;
        }
    } else {
        // one thread per group (small batches: one tile per group, no search)
        for (int q = tid; q <= E; q += blockDim.x) {
            const int g = q == 0 ? E : q - 1;
            const int m = off[g + 1] - off[g];
            const int start = ntile[q];
            for (int i = 0; i * bm < m; ++i) {
                tiles[2 * (start + i)] = g;
                tiles[2 * (start + i) + 1] = i * bm;
            }
        }
    }
    if (tid == 0) *n_tiles = nt;
    __syncthreads();   // ntile[] is reused by a second list
}

// Rank of every pair of one block inside its expert, then the scatter.
// `e` holds the ids of this thread's token (block b, token b*kBT + tid).
__device__ void block_scatter(const int (&e)[8], uint32_t *bits, const int *base, int b, int N, int k, int E,
                              int32_t *por, int32_t *rop) {
    const int tid = threadIdx.x;
    for (int i = tid; i < E * kBTW; i += blockDim.x) bits[i] = 0;
    __syncthreads();
    const int t = b * kBT + tid;
    const bool live = tid < kBT && t < N;
    if (live) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < k) atomicOr(&bits[e[j] * kBTW + (tid >> 5)], 1u << (tid & 31));
    }
    __syncthreads();
    if (live)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j >= k) break;
            const uint32_t *row = bits + e[j] * kBTW;
            int rank = __popc(row[tid >> 5] & ((1u << (tid & 31)) - 1u));
            for (int w = 0; w < (tid >> 5); ++w) rank += __popc(row[w]);
            int pos = base[e[j]] + rank;
            por[pos] = t * k + j;
            rop[(size_t)t * k + j] = pos;
        }
}

// ---- one-wave path (N <= 64, every group within one tile): dispatch_small.h

__global__ __launch_bounds__(64) void dispatch_wave_kernel(
    const int32_t *__restrict__ ids, int N, int k, int E, int32_t *g_offsets, int32_t *g_exp_off,
    int32_t *tiles, int32_t *n_tiles, int32_t *por, int32_t *rop) {
    dispatch_small(ids, N, k, E, g_offsets, g_exp_off, tiles, n_tiles, por, rop);
}

// ---- one-block path (N <= 256): everything in one workgroup of 1024 threads

__global__ __launch_bounds__(1024) void dispatch_fused_kernel(
    const int32_t *__restrict__ ids, int N, int k, int E, int bm, int32_t *g_offsets, int32_t *g_exp_off,
    int32_t *tiles, int32_t *n_tiles, int32_t *por, int32_t *rop) {
    __shared__ int cnt[1024];
    __shared__ int off[1026];
    __shared__ int ntile[1025];
    __shared__ int wsum[17];
    __shared__ uint32_t bits[1024 * kBTW];
    const int tid = threadIdx.x;
    const bool live = tid < N;   // N <= kBT
    int my[8];
    load_token_ids(ids, tid, k, live, my);
    for (int e = tid; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    if (live) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < k) atomicAdd(&cnt[my[j]], 1);
    }
    __syncthreads();
    offsets_and_tiles<false>(cnt, off, ntile, wsum, N, k, E, bm, g_offsets, g_exp_off, tiles, n_tiles);
    __syncthreads();
    block_scatter(my, bits, off, 0, N, k, E, por, rop);
}

// ---- multi-block path

__global__ __launch_bounds__(256) void dispatch_hist_kernel(const int32_t *__restrict__ ids, int N, int k, int E,
                                                            int32_t *__restrict__ blk) {
    __shared__ int cnt[1024];
    const int tid = threadIdx.x, b = blockIdx.x;
    const int t = b * kBT + tid;
    int my[8];
    load_token_ids(ids, t, k, t < N, my);
    for (int e = tid; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    if (t < N) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < k) atomicAdd(&cnt[my[j]], 1);
    }
    __syncthreads();
    for (int e = tid; e < E; e += blockDim.x) blk[(size_t)b * E + e] = cnt[e];
}

__global__ __launch_bounds__(1024) void dispatch_scan_kernel(int32_t *blk, int nblk, int N, int k, int E, int bm,
                                                             int32_t *g_offsets, int32_t *g_exp_off,
                                                             int32_t *tiles, int32_t *n_tiles, int32_t *tiles2,
                                                             int32_t *n_tiles2) {
    __shared__ int cnt[1024];
    __shared__ int off[1026];
    __shared__ int ntile[1025];
    __shared__ int wsum[17];
    constexpr int kChunk = 32768;   // block counts staged in LDS per pass (128 KB)
    __shared__ int stage[kChunk];
    const int tid = threadIdx.x;
    // per expert: exclusive prefix over blocks (in place), total count.  The
    // counts of cb blocks at a time are loaded by the whole workgroup at once
    // (coalesced, all loads in flight), scanned per expert in LDS and stored back.
    for (int e = tid; e < E; e += blockDim.x) cnt[e] = 0;
    const int cb = kChunk / E;   // E <= 1024: at least 32 blocks per pass
    for (int b0 = 0; b0 < nblk; b0 += cb) {
        const int nb = min(cb, nblk - b0), n = nb * E;
        const int32_t *src = blk + (size_t)b0 * E;
        for (int i = tid; i < n; i += blockDim.x) stage[i] = src[i];
        __syncthreads();
        for (int e = tid; e < E; e += blockDim.x) {
            // 16 blocks per step: all reads issued before the first write
            int run = cnt[e];
            for (int b = 0; b < nb; b += 16) {
                int c[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) c[i] = b + i < nb ? stage[(b + i) * E + e] : 0;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    if (b + i < nb) stage[(b + i) * E + e] = run;
                    run += c[i];
                }
            }
            cnt[e] = run;
        }
        __syncthreads();
        for (int i = tid; i < n; i += blockDim.x) blk[(size_t)b0 * E + i] = stage[i];
        __syncthreads();
    }
    offsets_and_tiles<true>(cnt, off, ntile, wsum, N, k, E, bm, g_offsets, g_exp_off, tiles, n_tiles, tiles2,
                            n_tiles2);
}

// blk[b][e]: rows of expert e in the blocks before b (from the scan)
__global__ __launch_bounds__(256) void dispatch_scatter_kernel(const int32_t *__restrict__ ids, const int32_t *blk,
                                                               const int32_t *__restrict__ offsets, int N, int k,
                                                               int E, int32_t *por, int32_t *rop) {
    __shared__ uint32_t bits[1024 * kBTW];
    __shared__ int base[1024];
    const int t = blockIdx.x * kBT + threadIdx.x;
    for (int e = threadIdx.x; e < E; e += blockDim.x) base[e] = offsets[e] + blk[(size_t)blockIdx.x * E + e];
    int my[8];
    load_token_ids(ids, t, k, t < N, my);
    block_scatter(my, bits, base, blockIdx.x, N, k, E, por, rop);   // its first barrier publishes base
}

// ---- scan and scatter in one launch (after dispatch_hist_kernel).  Every
// block reads all blocks' counts (nblk x E values, coalesced over the
// experts), forms the expert totals and its own per-expert prefix, scans the
// totals into the group offsets and scatters its tokens; block 0 also writes
// the offsets and the tile lists.  This trades the single-workgroup scan
// kernel and one launch for nblk x E reads per block, which is cheap up to
// kFusedScanMaxBlk blocks (one MI355X, d = 2560, E = 384, top-6, per layer
// step: N = 1024 / 4096 / 8192 / 16384 (Zipf) 4-7 us faster, E4M3 weights at
// N = 4096 10 us).
#ifndef FGS_DISPATCH_FUSED_SCAN
#define FGS_DISPATCH_FUSED_SCAN 1
#endif
constexpr int kFusedScanMaxBlk = 64;   // N <= 16384 tokens
__global__ __launch_bounds__(1024) void dispatch_scan_scatter_kernel(
    const int32_t *__restrict__ ids, const int32_t *__restrict__ blk, int nblk, int N, int k, int E, int bm,
    int32_t *g_offsets, int32_t *g_exp_off, int32_t *tiles, int32_t *n_tiles, int32_t *tiles2, int32_t *n_tiles2,
    int32_t *por, int32_t *rop) {
    __shared__ int cnt[1024];
    __shared__ int pre[1024];
    __shared__ int off[1026];
    __shared__ int ntile[1025];
    __shared__ int wsum[17];
    __shared__ uint32_t bits[1024 * kBTW];
    const int tid = threadIdx.x, b = blockIdx.x;
    const int t = b * kBT + tid;
    int my[8];
    load_token_ids(ids, t, k, tid < kBT && t < N, my);
    // expert e: total over all blocks and the rows in blocks before b, 16 loads in flight
    for (int e = tid; e < E; e += blockDim.x) {
        int tot = 0, before = 0;
        for (int b0 = 0; b0 < nblk; b0 += 16) {
            int c[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) c[i] = b0 + i < nblk ? blk[(size_t)(b0 + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                tot += c[i];
                before += b0 + i < b ? c[i] : 0;
            }
        }
        cnt[e] = tot;
        pre[e] = before;
    }
    __syncthreads();
    if (b == 0) {
        offsets_and_tiles<true>(cnt, off, ntile, wsum, N, k, E, bm, g_offsets, g_exp_off, tiles, n_tiles, tiles2,
                                n_tiles2);
    } else {
        for (int e = tid; e < E; e += blockDim.x) off[e] = cnt[e];
        __syncthreads();
        block_exclusive_scan_1024(off, E, wsum);
    }
    __syncthreads();
    for (int e = tid; e < E; e += blockDim.x) pre[e] += off[e];
    block_scatter(my, bits, pre, b, N, k, E, por, rop);   // its first barrier publishes pre
}

hipError_t launch_dispatch(const Plan &p) {
    if (p.fused_route || p.tail_dispatch) return hipSuccess;   // done by the top-k kernel
    if (p.N <= 64 && p.bm >= p.N) {   // one wave; every group fits one tile
        hipLaunchKernelGGL(dispatch_wave_kernel, dim3(1), dim3(64), 0, p.stream, p.ids, p.N, p.k, p.E, p.offsets,
                           p.exp_off_out, p.tiles, p.n_tiles, p.por, p.rop);
        return hipGetLastError();
    }
    if (p.nblk == 1) {
        hipLaunchKernelGGL(dispatch_fused_kernel, dim3(1), dim3(1024), 0, p.stream, p.ids, p.N, p.k, p.E, p.bm,
                           p.offsets, p.exp_off_out, p.tiles, p.n_tiles, p.por, p.rop);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(dispatch_hist_kernel, dim3(p.nblk), dim3(256), 0, p.stream, p.ids, p.N, p.k, p.E, p.blk);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
#if FGS_DISPATCH_FUSED_SCAN
    if (p.nblk <= kFusedScanMaxBlk) {
        hipLaunchKernelGGL(dispatch_scan_scatter_kernel, dim3(p.nblk), dim3(1024), 0, p.stream, p.ids, p.blk, p.nblk,
                           p.N, p.k, p.E, p.bm, p.offsets, p.exp_off_out, p.tiles, p.n_tiles, p.tiles2, p.n_tiles2,
                           p.por, p.rop);
        return hipGetLastError();
    }
#endif
    hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(1024), 0, p.stream, p.blk, p.nblk, p.N, p.k, p.E, p.bm,
                       p.offsets, p.exp_off_out, p.tiles, p.n_tiles, p.tiles2, p.n_tiles2);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(dispatch_scatter_kernel, dim3(p.nblk), dim3(256), 0, p.stream, p.ids, p.blk, p.offsets, p.N,
                       p.k, p.E, p.por, p.rop);
    return hipGetLastError();
}

}  // namespace fgs
