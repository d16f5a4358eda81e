// Host-side description of one moe_forward call, shared by the launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fgs_moe.h"

namespace fgs {

struct Plan {
    // problem
    int N, d, E, k, f, fs;
    int xdt, wdt;
    uint32_t flags;
    // caller buffers
    const void *x;
    const float *rw, *rb;
    moe_weights W;
    void *out;
    // routing buffers (caller's aux buffers when given, else workspace)
    float *partial;      // [ks][N][E] router partial sums over k-slices
    int ks;              // number of k-slices of the router
    int kslice;          // k-slice length (d / ks)
    float *logits;       // [N][E] or nullptr
    int32_t *ids;        // [N][k]
    float *tw;           // [N][k]
    float *gap;          // [N] or nullptr
    int32_t *blk;        // [nblk][E] per-block counts, then rows of each expert in earlier blocks
    int nblk;
    int32_t *offsets;    // [E+2]: routed groups, then the shared group's rows
    int32_t *exp_off_out;// caller's [E+1] copy, or nullptr
    int32_t *tiles;      // [max_tiles] packed (group << 16... see dispatch) entries
    int32_t *n_tiles;    // [1]
    int max_tiles;
    int32_t *tiles2;     // with wide gate/up tiles (bm 256): the down product's 128-row list, else nullptr
    int32_t *n_tiles2;
    int max_tiles2;
    int bm;              // rows per tile of the expert kernels
    int32_t *por, *rop;  // [N*k]
    uint16_t *H;         // [N*k + N][ldh] bfloat16 SwiGLU activations
    int ldh;
    float *Y;            // [N*k + N][d] expert outputs: float32 (stream path) or bfloat16 (GEMM path)
    uint16_t *w3;        // [E][3d] bf16 split of the router weights (router GEMM only)
    int32_t *rflags;     // [E] router GEMM only: nonzero if expert e's mid or lo split term is nonzero
    const float *norm_post;  // block variant: post-norm weights [d] (out = the residual row)
    float eps;
    // 1 x 128 activation quantisation (FP8 x FP8 expert matmuls)
    bool aq;
    uint8_t *xq;         // [N][d] E4M3 codes of the experts' input
    float *xs;           // [N][d/128] its group scales
    uint8_t *hq;         // [N*k + N][ldh] E4M3 codes of the hidden activations
    float *hs;           // [N*k + N][ldh/128] their group scales
    float *hf;           // [N*k + N][ldh] FP32 hidden activations (stream path, before quantisation)
    bool use_stream;     // decode-shaped expert path; otherwise the grouped GEMMs
    bool fused_route;    // top-k and dispatch in one kernel (fused_route_ok)
    bool tail_dispatch;  // the last top-k workgroup lays out the dispatch (tail_dispatch_ok)
    int32_t *route_cnt;  // [1] top-k workgroups done; zeroed by the router kernel of each call
    hipStream_t stream;
};

// launchers (each returns the hipError_t of its launch)
hipError_t launch_router(const Plan &p);
hipError_t launch_topk(const Plan &p);
hipError_t launch_dispatch(const Plan &p);
hipError_t launch_gate_up(const Plan &p);
hipError_t launch_down(const Plan &p);
hipError_t launch_combine(const Plan &p);
hipError_t launch_gate_up_gemm(const Plan &p);
hipError_t launch_down_gemm(const Plan &p);
hipError_t launch_router_gemm(const Plan &p, uint16_t *w3);
hipError_t launch_prenorm(const Plan &p, const void *resid, const float *g, float eps, void *xn);
hipError_t launch_combine_block(const Plan &p);
hipError_t gemm_kernels_init();  // once per process: raise the kernels' LDS limit
hipError_t launch_quant_groups(const void *v, int v_bf16, int ldv, long rows, int cols, uint8_t *q, int ldq,
                               float *s, int lds, hipStream_t stream);

// Decode-shaped expert kernels keep whole weight rows in registers and take
// tiles of at most 64 rows (one token per lane).  Against the grouped GEMMs
// (one MI355X, d = 2560, E = 384, top-6) they are faster up to about 192
// tokens: bf16 weights at N = 65 / 128 / 192: 0.322 / 0.438 / 0.516 ms
// against 0.387 / 0.503 / 0.534; at 224 both take 0.55; E4M3 weights at
// N = 128: 0.293 against 0.359, at 192 both 0.373.
constexpr int kStreamMaxN = 192;
constexpr int kStreamBM = 64;
inline bool stream_path(int N, int d, int f, int fs) {
    return N <= kStreamMaxN && d <= 4096 && f <= 512 && fs <= 512;
}
constexpr int kGemmBM = 128;  // rows per tile of the grouped GEMMs
// bf16 activations with bf16 or per-channel E4M3 weights at large batches take
// 256-row tiles for gate/up (the wide tile: more flops per operand byte a CU
// takes in); the down product takes each such entry as two 128-row items.  Their DMAs use
// 32-bit byte offsets, so x and H must stay below 4 GB.
constexpr int kGemmBMWide = 256;
#ifndef FGS_WIDE_MIN_N
#define FGS_WIDE_MIN_N 8192
#endif
constexpr int kWideMinN = FGS_WIDE_MIN_N;
// only the multi-block dispatch (more than 256 tokens) writes the down product's own list
static_assert(kWideMinN > 256, "wide tiles need the multi-block dispatch");
inline int gemm_bm(int N, int d, int k, int f, int fs, int xdt, int wdt, uint32_t flags) {
    const long ldh = f > fs ? f : fs;
    const bool fits32 = (long)N * d * 2 < (1L << 32) && ((long)N * k + N) * ldh * 2 < (1L << 32);
    // bf16 or per-channel E4M3 weights with bf16 activations; or, with 1 x 128 activation
    // quantisation, E4M3 weights of either scale layout and K up to 24 blocks of 128
    const bool aq = (flags & MOE_FLAG_FP8_ACT_QUANT) != 0;
#ifndef FGS_WIDE_F8
#define FGS_WIDE_F8 1
#endif
    const bool wide_w = aq ? FGS_WIDE_F8 && wdt == MOE_DTYPE_FP8_E4M3 && d / 128 <= 24
                           : wdt == MOE_DTYPE_BF16 || (wdt == MOE_DTYPE_FP8_E4M3 && !(flags & MOE_FLAG_FP8_BLOCK128));
    if (xdt == MOE_DTYPE_BF16 && wide_w && N >= kWideMinN && fits32) return kGemmBMWide;
    return kGemmBM;
}

// Router tiling: wave tile of (16*MT tokens) x (16*NT experts); the k range is
// cut into ks slices so that small batches still spread over many waves.
struct RouterTiling { int mt, nt, ks; };
// Batches above kRouterGemmN (bf16 activations) use the router GEMM instead
// (one k-slice, W_r split into three bf16 terms along K).
constexpr int kRouterGemmN = 64;
inline bool router_gemm(int N, int xdt) { return xdt == MOE_DTYPE_BF16 && N > kRouterGemmN; }

// Batches of at most kFusedRouteN tokens run top-k and dispatch as one kernel
// (router_mfma partial sums; on the stream path every group is one tile).
// One MI355X, d = 2560, E = 384, top-6: 29.8 against 32.1 us per layer step at
// N = 1, 37.7 against 39.4 at N = 2, equal at N = 4 (the selections of more
// tokens on one CU then cost what the launch saves).
#ifndef FGS_FUSED_ROUTE_N
#define FGS_FUSED_ROUTE_N 4
#endif
constexpr int kFusedRouteN = FGS_FUSED_ROUTE_N;   // 0 switches the fusion off
static_assert(kFusedRouteN >= 0 && kFusedRouteN <= 7, "one workgroup of at most 7 waves");
constexpr int kFusedRouteCap = kFusedRouteN > 0 ? kFusedRouteN : 1;   // array and workgroup bounds
inline bool fused_route_ok(int N, int xdt) { return N >= 1 && N <= kFusedRouteN && !router_gemm(N, xdt); }
// Past kFusedRouteN and up to 64 tokens (one wave of dispatch, every group in
// one tile of the stream path) the top-k runs one workgroup per token as
// usual, and the workgroup that finishes last (a counter the router kernel of
// the same call zeroes) lays out the dispatch: one launch less per step.
#ifndef FGS_TAIL_DISPATCH
#define FGS_TAIL_DISPATCH 1
#endif
inline bool tail_dispatch_ok(int N, int bm) { return FGS_TAIL_DISPATCH && N >= 1 && N <= 64 && bm >= N; }
// k-slices of the router GEMM: 3 c slices, c per split term (hi, mid, lo),
// so that a slice never straddles two terms and the slices of all-zero terms
// can be skipped; c <= 4 divides the d/64 K stages of a term and is raised
// while the hi term alone fills at most one 128 x 256 tile per CU (256).
inline int router_gemm_ks(int N, int d, int E) {
    const long wgs = (long)((N + 127) / 128) * ((E + 255) / 256);
    const int stages = d / 64;
    int c = 1;
    for (int cand : {2, 3, 4})
        if (stages % cand == 0 && wgs * cand <= 256) c = cand;
    return 3 * c;
}
inline RouterTiling router_tiling(int N, int d, int E) {
    RouterTiling r;
    if (N <= kRouterGemmN) { r.mt = 2; r.nt = 1; } else { r.mt = 4; r.nt = 4; }
    long n_tb = (N + 16 * r.mt - 1) / (16 * r.mt);
    long n_eb = (E + 16 * r.nt - 1) / (16 * r.nt);
    long tiles = n_tb * n_eb;
    r.ks = 1;
    const int cands[] = {10, 8, 5, 4, 2};
    if (tiles < 512) {
        for (int c : cands) {
            if ((d / 32) % c == 0 && tiles * c <= 2048) { r.ks = c; break; }
        }
    }
    return r;
}

// largest tile-list length for a given row tile
inline int max_tiles_for(int N, int k, int E, int bm) {
    long nk = (long)N * k;
    long routed = (nk + bm - 1) / bm + (nk < E ? nk : E);
    long shared = (N + bm - 1) / bm;
    return (int)(routed + shared);
}

}  // namespace fgs
