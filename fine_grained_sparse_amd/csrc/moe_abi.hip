// C ABI of the MoE layer: argument checks, workspace carving, launch order.
// The declarations and their documentation are in include/fgs_moe.h.
#include <atomic>
#include <cstring>
#include <mutex>

#include "moe_plan.h"

// Intermediates of moe_forward_noalloc: one copy of this array per GPU, in
// the code object's static storage, held until the process ends.  On the
// host the name is a stand-in object, not a device address: host code takes
// the address from hipGetSymbolAddress, once per device (scratch_ptr below),
// and passes that pointer on.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace fgs {
namespace {

thread_local int g_last_hip_error = 0;
std::atomic<int> g_arch_state[64];  // 0 unknown, 1 gfx950, 2 other

std::atomic<int> g_gemm_init[64];   // per device: 0 not yet, 1 the GEMM kernels' LDS limits are raised

std::atomic<void *> g_scratch_ptr[64];   // per device: the address of `scratch`, resolved on first use
std::mutex g_scratch_mu;

// Device address of this device's copy of `scratch` (dev must be current).
int scratch_ptr(int dev, void **out) {
    void *q = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!q) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        q = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!q) {
            hipError_t e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !q) {
                g_last_hip_error = (int)(e != hipSuccess ? e : hipErrorInvalidSymbol);
                return MOE_ERR_HIP;
            }
            g_scratch_ptr[dev].store(q, std::memory_order_release);
        }
    }
    *out = q;
    return MOE_OK;
}

int check_device(int *dev_out = nullptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) { g_last_hip_error = (int)e; return MOE_ERR_HIP; }
    if (dev < 0 || dev >= 64) return MOE_ERR_UNSUPPORTED;
    int st = g_arch_state[dev].load(std::memory_order_acquire);
    if (st == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) { g_last_hip_error = (int)e; return MOE_ERR_HIP; }
        st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_arch_state[dev].store(st, std::memory_order_release);
    }
    if (dev_out) *dev_out = dev;
    return st == 1 ? MOE_OK : MOE_ERR_UNSUPPORTED;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_desc(const moe_desc *d) {
    if (!d) return MOE_ERR_ARG;
    if (d->n_tokens < 0 || d->n_experts < 1 || d->n_experts > 1024) return MOE_ERR_ARG;
    if (d->top_k < 1 || d->top_k > 8 || d->top_k > d->n_experts) return MOE_ERR_ARG;
    if (d->d_model <= 0 || d->d_model % 64 || d->d_ff <= 0 || d->d_ff % 64 || d->d_ff_shared <= 0 ||
        d->d_ff_shared % 64)
        return MOE_ERR_ARG;
    if ((long)d->n_tokens * d->top_k + d->n_tokens >= (1L << 31)) return MOE_ERR_ARG;
    if (d->flags & ~(MOE_FLAG_ACCUMULATE | MOE_FLAG_RENORMALIZE | MOE_FLAG_FP8_BLOCK128 | MOE_FLAG_FP8_ACT_QUANT))
        return MOE_ERR_ARG;
    if (d->x_dtype != MOE_DTYPE_F32 && d->x_dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;
    if (d->w_dtype != MOE_DTYPE_BF16 && d->w_dtype != MOE_DTYPE_FP8_E4M3) return MOE_ERR_UNSUPPORTED;
    if ((d->flags & MOE_FLAG_FP8_BLOCK128) &&
        (d->w_dtype != MOE_DTYPE_FP8_E4M3 || d->d_model % 128 || d->d_ff % 128 || d->d_ff_shared % 128))
        return MOE_ERR_ARG;
    if ((d->flags & MOE_FLAG_FP8_ACT_QUANT) &&
        (d->w_dtype != MOE_DTYPE_FP8_E4M3 || d->x_dtype != MOE_DTYPE_BF16 || d->d_model % 128 || d->d_ff % 128 ||
         d->d_ff_shared % 128))
        return MOE_ERR_ARG;
    return MOE_OK;
}

struct Layout {
    size_t partial, ids, tw, blk, offsets, tiles, n_tiles, tiles2, n_tiles2, por, rop, H, Y, w3, rflags, xq, xs, hq,
        hs, hf, route_cnt, total;
    int ks, kslice, nblk, max_tiles, max_tiles2, bm, ldh;
    bool stream, rgemm, aq;
};

size_t take(size_t &cur, size_t bytes) {
    size_t at = cur;
    cur += (bytes + 255) & ~size_t(255);
    return at;
}

Layout layout_for(const moe_desc *d) {
    Layout L{};
    const size_t N = d->n_tokens, E = d->n_experts, k = d->top_k;
    L.rgemm = router_gemm(d->n_tokens, d->x_dtype);
    if (d->x_dtype == MOE_DTYPE_F32) {
        L.ks = 1;
    } else if (L.rgemm) {
        L.ks = router_gemm_ks(d->n_tokens, d->d_model, d->n_experts);
    } else {
        L.ks = router_tiling(d->n_tokens, d->d_model, d->n_experts).ks;
    }
    L.kslice = d->d_model / L.ks;
    L.nblk = (int)((N + 255) / 256);
    if (L.nblk < 1) L.nblk = 1;
    L.stream = stream_path(d->n_tokens, d->d_model, d->d_ff, d->d_ff_shared);
    L.bm = L.stream ? (d->n_tokens < 1 ? 1 : d->n_tokens < kStreamBM ? d->n_tokens : kStreamBM)
                    : gemm_bm(d->n_tokens, d->d_model, d->top_k, d->d_ff, d->d_ff_shared, d->x_dtype, d->w_dtype,
                              d->flags);
    L.max_tiles = max_tiles_for(d->n_tokens, d->top_k, d->n_experts, L.bm);
    L.max_tiles2 = L.bm == kGemmBMWide ? max_tiles_for(d->n_tokens, d->top_k, d->n_experts, kGemmBM) : 0;
    L.ldh = d->d_ff > d->d_ff_shared ? d->d_ff : d->d_ff_shared;
    const size_t rows = N * k + N;
    size_t cur = 0;
    L.partial = take(cur, (size_t)L.ks * N * E * 4);
    L.ids = take(cur, N * k * 4);
    L.tw = take(cur, N * k * 4);
    L.blk = take(cur, (size_t)L.nblk * E * 4);
    L.offsets = take(cur, (E + 2) * 4);
    L.tiles = take(cur, (size_t)L.max_tiles * 2 * 4);
    L.n_tiles = take(cur, 4);
    L.tiles2 = take(cur, (size_t)L.max_tiles2 * 2 * 4);
    L.n_tiles2 = take(cur, L.max_tiles2 ? 4 : 0);
    L.por = take(cur, N * k * 4);
    L.rop = take(cur, N * k * 4);
    L.H = take(cur, rows * L.ldh * 2);
    L.Y = take(cur, rows * (size_t)d->d_model * 4);
    L.w3 = take(cur, L.rgemm ? E * 3 * (size_t)d->d_model * 2 : 0);
    L.rflags = take(cur, L.rgemm ? E * 4 : 0);
    L.aq = (d->flags & MOE_FLAG_FP8_ACT_QUANT) != 0;
    const size_t dm = d->d_model;
    L.xq = take(cur, L.aq ? N * dm : 0);
    L.xs = take(cur, L.aq ? N * (dm / 128) * 4 : 0);
    L.hq = take(cur, L.aq ? rows * L.ldh : 0);
    L.hs = take(cur, L.aq ? rows * (L.ldh / 128) * 4 : 0);
    L.hf = take(cur, L.aq && L.stream ? rows * L.ldh * 4 : 0);
    L.route_cnt = take(cur, 4);
    L.total = cur;
    return L;
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    uintptr_t x0 = (uintptr_t)a, x1 = x0 + na, y0 = (uintptr_t)b, y1 = y0 + nb;
    return x0 < y1 && y0 < x1;
}

}  // namespace
}  // namespace fgs

using namespace fgs;

extern "C" {

size_t moe_workspace_size(const moe_desc *desc) {
    if (check_desc(desc) != MOE_OK) return 0;
    return layout_for(desc).total;
}

const char *moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported configuration or device";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

int moe_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"

namespace fgs {
namespace {

// Sandwich-norm arguments of the block entry point (null for moe_forward).
struct BlockArgs {
    void *resid;
    const float *norm_pre, *norm_post;
    float eps;
};

// static_scratch: the workspace is this device's `scratch` array (moe_forward_noalloc);
// `workspace` is then ignored and workspace_bytes is the array's size
int run_layer(const moe_desc *desc, const void *x, const float *router_w, const float *router_bias,
              const moe_weights *weights, void *out, void *workspace, size_t workspace_bytes, const moe_aux *aux,
              void *stream, const BlockArgs *blk, bool static_scratch = false) {
    int st = check_desc(desc);
    if (st != MOE_OK) return st;
    if (blk && (desc->flags & MOE_FLAG_ACCUMULATE)) return MOE_ERR_ARG;
    if (desc->n_tokens == 0) return MOE_OK;
    if (!x || !router_w || !router_bias || !weights || !out || (!workspace && !static_scratch)) return MOE_ERR_ARG;
    if (blk && (!blk->norm_pre || !blk->norm_post || !(blk->eps >= 0.0f))) return MOE_ERR_ARG;
    if (blk && desc->d_model > 16384) return MOE_ERR_UNSUPPORTED;  // the fused combine keeps a row in LDS
    const moe_weights &W = *weights;
    if (!W.w_gate || !W.w_up || !W.w_down || !W.ws_gate || !W.ws_up || !W.ws_down) return MOE_ERR_ARG;
    const bool fp8 = desc->w_dtype == MOE_DTYPE_FP8_E4M3;
    const bool have_scales[6] = {W.s_gate != nullptr, W.s_up != nullptr, W.s_down != nullptr,
                                 W.ss_gate != nullptr, W.ss_up != nullptr, W.ss_down != nullptr};
    for (bool h : have_scales)
        if (h != fp8) return MOE_ERR_ARG;
    const void *ptrs16[] = {x, out, W.w_gate, W.w_up, W.w_down, W.ws_gate, W.ws_up, W.ws_down, router_w};
    for (const void *q : ptrs16)
        if (!aligned(q, 16)) return MOE_ERR_ARG;
    if (blk && (!aligned(blk->norm_pre, 16) || !aligned(blk->norm_post, 16))) return MOE_ERR_ARG;
    if (!static_scratch && !aligned(workspace, 256)) return MOE_ERR_ARG;

    const size_t xbytes = (size_t)desc->n_tokens * desc->d_model * (desc->x_dtype == MOE_DTYPE_F32 ? 4 : 2);
    if (!blk && overlaps(x, xbytes, out, xbytes)) {
        if (!(desc->flags & MOE_FLAG_ACCUMULATE) || x != out) return MOE_ERR_ARG;
    }
    const Layout L = layout_for(desc);
    const size_t need = L.total + (blk ? ((xbytes + 255) & ~size_t(255)) : 0);
    if (workspace_bytes < need) return MOE_ERR_WORKSPACE;
    int dev = 0;
    st = check_device(&dev);
    if (st != MOE_OK) return st;
    if (static_scratch) {
        st = scratch_ptr(dev, &workspace);
        if (st != MOE_OK) return st;
    }
    if (!L.stream && g_gemm_init[dev].load(std::memory_order_acquire) != 1) {   // the expert GEMMs' LDS limits
        // idempotent: concurrent first calls may both set the same attributes
        hipError_t e = gemm_kernels_init();
        if (e != hipSuccess) { g_last_hip_error = (int)e; return MOE_ERR_HIP; }
        g_gemm_init[dev].store(1, std::memory_order_release);
    }

    char *ws = (char *)workspace;
    Plan p{};
    p.N = desc->n_tokens; p.d = desc->d_model; p.E = desc->n_experts; p.k = desc->top_k;
    p.f = desc->d_ff; p.fs = desc->d_ff_shared; p.xdt = desc->x_dtype; p.wdt = desc->w_dtype;
    p.flags = desc->flags;
    p.x = x; p.rw = router_w; p.rb = router_bias; p.W = W; p.out = out;
    p.partial = (float *)(ws + L.partial);
    p.ks = L.ks; p.kslice = L.kslice;
    p.logits = aux ? aux->logits : nullptr;
    p.ids = (aux && aux->topk_ids) ? aux->topk_ids : (int32_t *)(ws + L.ids);
    p.tw = (aux && aux->topk_w) ? aux->topk_w : (float *)(ws + L.tw);
    p.gap = aux ? aux->gap : nullptr;
    p.blk = (int32_t *)(ws + L.blk); p.nblk = L.nblk;
    p.offsets = (int32_t *)(ws + L.offsets);
    p.exp_off_out = aux ? aux->expert_offsets : nullptr;
    p.tiles = (int32_t *)(ws + L.tiles); p.n_tiles = (int32_t *)(ws + L.n_tiles);
    p.max_tiles = L.max_tiles; p.bm = L.bm;
    p.tiles2 = L.max_tiles2 ? (int32_t *)(ws + L.tiles2) : nullptr;
    p.n_tiles2 = L.max_tiles2 ? (int32_t *)(ws + L.n_tiles2) : nullptr;
    p.max_tiles2 = L.max_tiles2;
    p.por = (aux && aux->pair_of_row) ? aux->pair_of_row : (int32_t *)(ws + L.por);
    p.rop = (aux && aux->row_of_pair) ? aux->row_of_pair : (int32_t *)(ws + L.rop);
    p.H = (uint16_t *)(ws + L.H); p.ldh = L.ldh;
    p.Y = (float *)(ws + L.Y);
    p.w3 = (uint16_t *)(ws + L.w3);
    p.rflags = L.rgemm ? (int32_t *)(ws + L.rflags) : nullptr;
    p.use_stream = L.stream;
    p.fused_route = L.stream && fused_route_ok(p.N, p.xdt);
    p.tail_dispatch = L.stream && !p.fused_route && tail_dispatch_ok(p.N, p.bm);
    p.route_cnt = (int32_t *)(ws + L.route_cnt);
    p.stream = (hipStream_t)stream;
    p.aq = L.aq;
    if (L.aq) {
        p.xq = (uint8_t *)(ws + L.xq);
        p.xs = (float *)(ws + L.xs);
        p.hq = (uint8_t *)(ws + L.hq);
        p.hs = (float *)(ws + L.hs);
        p.hf = L.stream ? (float *)(ws + L.hf) : nullptr;
    }
    if (blk) {
        // the normalised input lives after the layer's own workspace; the
        // layer reads it as x and the fused combine updates the residual
        p.x = ws + L.total;
        p.out = blk->resid;
        p.norm_post = blk->norm_post;
        p.eps = blk->eps;
        hipError_t e = launch_prenorm(p, blk->resid, blk->norm_pre, blk->eps, ws + L.total);
        if (e != hipSuccess) { g_last_hip_error = (int)e; return MOE_ERR_HIP; }
    }

    void **ev = (aux && aux->stage_events) ? aux->stage_events : nullptr;
    typedef hipError_t (*Stage)(const Plan &);
    const Stage stages[MOE_NUM_STAGES] = {launch_router, launch_topk, launch_dispatch,
                                          p.use_stream ? launch_gate_up : launch_gate_up_gemm,
                                          p.use_stream ? launch_down : launch_down_gemm,
                                          blk ? launch_combine_block : launch_combine};
    for (int s = 0; s < MOE_NUM_STAGES; ++s) {
        hipError_t e;
        if (ev && ev[2 * s]) {
            e = hipEventRecord((hipEvent_t)ev[2 * s], p.stream);
            if (e != hipSuccess) { g_last_hip_error = (int)e; return MOE_ERR_HIP; }
        }
        e = stages[s](p);
        if (e != hipSuccess) { g_last_hip_error = (int)e; return MOE_ERR_HIP; }
        if (ev && ev[2 * s + 1]) {
            e = hipEventRecord((hipEvent_t)ev[2 * s + 1], p.stream);
            if (e != hipSuccess) { g_last_hip_error = (int)e; return MOE_ERR_HIP; }
        }
    }
    return MOE_OK;
}

}  // namespace
}  // namespace fgs

extern "C" {

int moe_forward(const moe_desc *desc, const void *x, const float *router_w, const float *router_bias,
                const moe_weights *weights, void *out, void *workspace, size_t workspace_bytes,
                const moe_aux *aux, void *stream) {
    return run_layer(desc, x, router_w, router_bias, weights, out, workspace, workspace_bytes, aux, stream, nullptr);
}

int moe_forward_noalloc(const moe_desc *desc, const void *x, const float *router_w, const float *router_bias,
                        const moe_weights *weights, void *out, const moe_aux *aux, void *stream) {
    return run_layer(desc, x, router_w, router_bias, weights, out, nullptr, MOE_NOALLOC_SCRATCH_BYTES, aux, stream,
                     nullptr, true);
}

size_t moe_block_workspace_size(const moe_desc *desc) {
    if (check_desc(desc) != MOE_OK) return 0;
    const size_t xbytes = (size_t)desc->n_tokens * desc->d_model * (desc->x_dtype == MOE_DTYPE_F32 ? 4 : 2);
    return layout_for(desc).total + ((xbytes + 255) & ~size_t(255));
}

int moe_quantize_groups(const void *v, int v_dtype, int64_t rows, int32_t cols, uint8_t *q, float *scales,
                        void *stream) {
    if (rows < 0 || cols <= 0 || cols % 128 || rows * (int64_t)cols >= (int64_t(1) << 40)) return MOE_ERR_ARG;
    if (v_dtype != MOE_DTYPE_F32 && v_dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;
    if (rows == 0) return MOE_OK;
    if (!v || !q || !scales || !aligned(v, 16) || !aligned(q, 8) || !aligned(scales, 4)) return MOE_ERR_ARG;
    int st = check_device();
    if (st != MOE_OK) return st;
    hipError_t e = launch_quant_groups(v, v_dtype == MOE_DTYPE_BF16, cols, rows, cols, q, cols, scales, cols / 128,
                                       (hipStream_t)stream);
    if (e != hipSuccess) { g_last_hip_error = (int)e; return MOE_ERR_HIP; }
    return MOE_OK;
}

int moe_block_forward(const moe_desc *desc, void *resid, const float *norm_pre, const float *norm_post, float eps,
                      const float *router_w, const float *router_bias, const moe_weights *weights, void *workspace,
                      size_t workspace_bytes, const moe_aux *aux, void *stream) {
    const BlockArgs blk{resid, norm_pre, norm_post, eps};
    // x is only checked for presence and alignment; the layer reads the normalised copy
    return run_layer(desc, resid, router_w, router_bias, weights, resid, workspace, workspace_bytes, aux, stream,
                     &blk);
}

}  // extern "C"
