// Grouped expert GEMMs on the matrix cores (batches larger than the decode path).
//
// "Inside Kolibri 1" (flozi.net), section "Routing: selection bias and
// mixture weights are separate": every routed or shared expert is a SwiGLU
// MLP (two 2560 -> 512 projections forming SiLU(gate) x up, then 512 -> 2560)
// and there is no per-expert capacity, so the rows per expert vary from zero
// to most of the batch.  Section "The FP8 path is explicitly mixed precision":
// FP8 E4M3 weights with FP32 scales.  A per-output-channel scale factors out
// of the dot product and is applied exactly in the epilogue.  With one scale
// per 128 x 128 block the scale changes along K: every 128-wide K block (two
// 64-wide stages) is accumulated on its own and added into the running sum
// times its block's scale, one FP32 multiply-add per accumulator per block.
//
// Work list: the dispatch scan writes one tile per 128 rows of every
// non-empty group (shared expert first).  Work items are handed out
// XCD-aware (xcd_item below), so the workgroups that share an expert's weight
// slices and token rows run on one XCD and hit in its L2.  Skewed routing
// just yields more row tiles for the popular experts.
//
// Workgroup tile: 128 rows x 256 GEMM columns, 512 threads = 8 waves in a 2
// (rows) x 4 (columns) layout, each wave 64 x 64; a wave skips the 16-row
// MFMA sub-tiles that lie entirely past the group's last row.
//   gate/up: A = x rows gathered through pair_of_row; B rows 0..127 are gate
//            rows c0..c0+127 and B rows 128..255 the matching up rows, so
//            every lane holds a gate and an up result of the same (row,
//            column) and the SwiGLU epilogue is lane-local.  Writes H (bf16).
//   down:    A = H rows of the group (contiguous), B = down rows; writes Y
//            (bf16) for the combine kernel.
// The tile routines share this layout:
//   tile_mma_dma  bf16 activations and weights: operand tiles fetched straight
//                 into three LDS stages (64-wide K stages, unpadded rows with
//                 an XOR chunk swizzle), MFMA 16x16x32 bf16;
//   tile_mma_dma_w8  bf16 activations, FP8 weights with per-channel scales:
//                 the same with E4M3 weight rows (64 bytes per stage), four
//                 stages, codes widened to bf16 (exact) as fragments are read;
//                 tile_mma_dma_w8b the same for 128 x 128 block scales (each
//                 stage's products folded in with its block's scale);
//   tile_mma      every other combination: operands through registers into
//                 two padded LDS stages (rows of 80 elements, measured free of
//                 bank conflicts); FP8 weights are decoded to bf16 (exact) and
//                 FP32 activations rounded to bf16 on the way into LDS;
//   tile_mma_f8   1 x 128 quantised activations: E4M3 operands, 128-wide K
//                 stages of the same byte layout, MFMA 16x16x128 f8f6f4, each
//                 stage folded in with its activation and weight scales;
//                 tile_mma_dma_f8 is the same product with both operand tiles
//                 fetched straight into LDS (K up to 24 blocks of 128).
// A 128 x 256 stage of 128 bytes per row moves 48 KB for 4.2 MFLOP (bf16) or
// 8.4 MFLOP (FP8).
//
// From 8192 tokens the gate/up product takes 256 x 256 tiles: 16 waves with
// bf16 activations (gate_up_gemm_wide_kernel), 8 waves with 1 x 128 quantised
// ones (gate_up_gemm_f8_wide_kernel).  The down product (K = f, only eight
// 64-wide or four 128-wide stages per item) runs persistent kernels whose DMA
// rings cross item boundaries: down_gemm_persist_kernel on 128 x 256 items
// (bf16 weights, E4M3 with per-channel or block scales), with the wide gate/up
// tiles down_gemm_wide_persist_kernel on 256 x 256 items, and for quantised
// activations down_gemm_f8_persist_kernel (FP8 x FP8, 128 x 256 items).
#include <atomic>

#include "moe_common.h"
#include "moe_plan.h"

namespace fgs {

constexpr int kBM = 128;        // rows per tile (the dispatch row tile)
constexpr int kBK = 64;         // K per stage
constexpr int kLdsStride = 80;  // padded row length in LDS (elements): conflict-free 16-byte fragment reads

// Tile geometry for WN column waves: 2 x WN waves (128 * WN threads), tile
// 128 rows x 64*WN columns (the GEMMs use WN = 4).
template <int WN>
struct Geo {
    static constexpr int kThreads = 128 * WN;
    static constexpr int kBN = 64 * WN;
    static constexpr int kAElems = kBM * kLdsStride;
    static constexpr int kBElems = kBN * kLdsStride;
    static constexpr int kStageElems = kAElems + kBElems;
    static constexpr int kAPer = kBM * 8 / kThreads;  // 16-byte A chunks per thread per stage
    static constexpr int kBPer = kBN * 8 / kThreads;  // 16-byte B chunks per thread per stage (4)
    static constexpr size_t kLds = 2 * kStageElems * sizeof(uint16_t);
};
constexpr int kWN = 4;
constexpr int kThreads = Geo<kWN>::kThreads;  // 512
constexpr int kBN = Geo<kWN>::kBN;            // 256
constexpr int kAPer = Geo<kWN>::kAPer;
constexpr int kBPer = Geo<kWN>::kBPer;
constexpr size_t kGemmLds = Geo<kWN>::kLds;   // 120 KiB
// direct-to-LDS variant: three stages of unpadded 128-byte rows
constexpr int kDmaStages = 3;
constexpr int kDmaRowB = 128;
constexpr int kDmaStageB = (kBM + kBN) * kDmaRowB;                 // 48 KiB
constexpr size_t kGemmLdsDma = (size_t)kDmaStages * kDmaStageB;    // 144 KiB, static
static_assert(kGemmLdsDma <= 160 * 1024, "the direct-to-LDS stages must fit one CU's LDS");

// XCD-aware work order.  Workgroups are handed to the 8 XCDs round-robin by
// launch index, and each XCD has its own L2.  Work items (column block
// fastest, then the tile list, whose tiles of one expert are adjacent) are
// grouped in blocks of kXcdTiles tile rows; XCD c takes blocks c, c+8, c+16,
// ... in order.  The workgroups that share an expert's weight slices and
// token rows thus run on one XCD and hit in its L2, while heavy stretches of
// the list (the shared expert's tiles come first) spread over all XCDs.
// Launch slot L = 8 s + c runs item ((s / B) * 8 + c) * B + s % B, with
// B = kXcdTiles * gridDim.x; every item below n has a slot below n + 8 B, so
// the grid must hold that many workgroups.  Returns false for a workgroup
// without an item.
constexpr int kXcds = 8;
constexpr int kXcdTiles = 2;   // blocks of 1, 4, 8 tile rows measured slower (Zipf 1.347 / 1.358 / 1.347 ms against 1.341)
__device__ __forceinline__ bool xcd_item(int n_items, int &item) {
    const int L = blockIdx.y * gridDim.x + blockIdx.x;
    const int B = kXcdTiles * gridDim.x;
    const int c = L % kXcds, slot = L / kXcds;
    item = ((slot / B) * kXcds + c) * B + slot % B;
    return item < n_items;
}

__device__ __forceinline__ f32x4_t mfma_bf16(const uint4 &a, const uint4 &b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// 8 E4M3 codes -> 8 bf16, exact (v_cvt_scalef32_pk_bf16_fp8 with scale 1; this
// conversion was checked against the format definition for all 256 codes)
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
__device__ __forceinline__ uint4 e4m3x8_to_bf16x8(const uint2 &q) {
    return make_uint4(e4m3x2_to_bf16x2<false>(q.x), e4m3x2_to_bf16x2<true>(q.x), e4m3x2_to_bf16x2<false>(q.y),
                      e4m3x2_to_bf16x2<true>(q.y));
}

template <bool FP8> struct WRaw;
template <> struct WRaw<false> { typedef uint4 T; };   // 8 bf16
template <> struct WRaw<true> { typedef uint2 T; };    // 8 e4m3

template <bool FP8>
__device__ __forceinline__ typename WRaw<FP8>::T load_w8(const void *base, size_t elem) {
    if constexpr (FP8) return *reinterpret_cast<const uint2 *>((const uint8_t *)base + elem);
    else return *reinterpret_cast<const uint4 *>((const uint16_t *)base + elem);
}
template <bool FP8>
__device__ __forceinline__ uint4 w8_to_bf16(const typename WRaw<FP8>::T &v) {
    if constexpr (FP8) return e4m3x8_to_bf16x8(v);
    else return v;
}

// Raw activation chunk of 8 elements: bf16 (one uint4) or FP32 (two float4,
// rounded to bf16 when written to LDS)
template <bool XF32> struct ARaw;
template <> struct ARaw<false> { uint4 v; };
template <> struct ARaw<true> { float4 lo, hi; };

template <bool XF32>
__device__ __forceinline__ ARaw<XF32> load_a8(const void *base, size_t elem) {
    ARaw<XF32> r;
    if constexpr (XF32) {
        const float4 *p = reinterpret_cast<const float4 *>((const float *)base + elem);
        r.lo = p[0];
        r.hi = p[1];
    } else {
        r.v = *reinterpret_cast<const uint4 *>((const uint16_t *)base + elem);
    }
    return r;
}
template <bool XF32>
__device__ __forceinline__ uint4 a8_to_bf16(const ARaw<XF32> &r, bool ok) {
    uint4 v;
    if constexpr (XF32)
        v = make_uint4(pack_bf16x2(r.lo.x, r.lo.y), pack_bf16x2(r.lo.z, r.lo.w), pack_bf16x2(r.hi.x, r.hi.y),
                       pack_bf16x2(r.hi.z, r.hi.w));
    else
        v = r.v;
    return ok ? v : make_uint4(0, 0, 0, 0);
}

// Barrier for LDS hand-off only: waits for this wave's LDS operations, not
// for its global loads, so prefetches stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// B tile row of a wave's column fragment ni: the wave in column wn owns B rows
// [wn*32, wn*32+32) (first half: gate rows for gate/up) and the rows
// kBN/2 + [wn*32, wn*32+32) (second half: the matching up rows).
template <int WN = kWN>
__device__ __forceinline__ int b_row_of(int wn, int ni) {
    return ni < 2 ? wn * 32 + ni * 16 : Geo<WN>::kBN / 2 + wn * 32 + (ni - 2) * 16;
}

// One 128 x 256 x K tile product.  Per K stage each thread fetches kAPer A
// chunks and kBPer B chunks of 16 bytes (tile row r = tid/8 + 64*j, chunk
// tid%8) into one of two register slots, two stages ahead of their use; LDS
// holds two stages.  Stage kt: issue the loads of stage kt+2, multiply stage
// kt from LDS, write stage kt+1 (loaded one stage earlier) to the other LDS
// buffer, barrier.  Fetches are plain loads from valid addresses (rows past
// the tile end read a valid row); masking and format conversion happen when a
// stage is written to LDS, so no instruction waits on a load early.
template <bool FP8, bool XF32, int WN>
struct Stage {
    ARaw<XF32> a[Geo<WN>::kAPer];
    typename WRaw<FP8>::T b[Geo<WN>::kBPer];
};

// The product covers GEMM columns [k_base, k_base + K).  `a_kmod`: the A
// column read for GEMM column k is k mod a_kmod (the router repeats x three
// times along K); pass a value above every k for a plain product.
// BLK: block-scaled weights (k_base = 0, K a multiple of 128); K block kb of
// column fragments ni < 2 is scaled by sc_lo[kb], of ni >= 2 by sc_hi[kb].
template <bool FP8, bool XF32, int WN = kWN, bool BLK = false>
__device__ __forceinline__ void tile_mma(const void *a_base, const size_t (&a_off)[Geo<WN>::kAPer],
                                         const bool (&a_ok)[Geo<WN>::kAPer], const void *const (&b_base)[Geo<WN>::kBPer],
                                         const size_t (&b_off)[Geo<WN>::kBPer], int k_base, int K, int a_kmod,
                                         int m, uint16_t *lds, f32x4_t (&acc)[4][4],
                                         const float *sc_lo = nullptr, const float *sc_hi = nullptr) {
    using G = Geo<WN>;
    constexpr int kRowStep = G::kThreads / 8;  // tile rows covered by one pass of the loader
    // the wave index is uniform: in a scalar register, the live-row tests are scalar branches
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int chunk = (tid & 7) * 8;
    const int r0 = tid >> 3;
    uint16_t *const As[2] = {lds, lds + G::kStageElems};
    uint16_t *const Bs[2] = {lds + G::kAElems, lds + G::kStageElems + G::kAElems};
    const int fr = lane & 15, fk = (lane >> 4) * 8;
    // 16-row sub-tiles of this wave that hold at least one row of the group
    const int live = min(4, max(0, (m - wm * 64 + 15) / 16));

    auto fetch = [&](Stage<FP8, XF32, WN> &st, int kl) {
        const int k0 = k_base + kl;
        const int ka = k0 % a_kmod;
#pragma unroll
        for (int j = 0; j < G::kAPer; ++j) st.a[j] = load_a8<XF32>(a_base, a_off[j] + ka + chunk);
#pragma unroll
        for (int j = 0; j < G::kBPer; ++j) st.b[j] = load_w8<FP8>(b_base[j], b_off[j] + k0 + chunk);
    };
    auto stash = [&](const Stage<FP8, XF32, WN> &st, int buf) {
#pragma unroll
        for (int j = 0; j < G::kAPer; ++j)
            *reinterpret_cast<uint4 *>(As[buf] + (r0 + kRowStep * j) * kLdsStride + chunk) =
                a8_to_bf16<XF32>(st.a[j], a_ok[j]);
#pragma unroll
        for (int j = 0; j < G::kBPer; ++j)
            *reinterpret_cast<uint4 *>(Bs[buf] + (r0 + kRowStep * j) * kLdsStride + chunk) = w8_to_bf16<FP8>(st.b[j]);
    };
    // BLK: the current K block's products, folded into acc after its second stage
    f32x4_t accb[4][4];
    if (BLK) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) accb[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    f32x4_t (&dst)[4][4] = BLK ? accb : acc;
    auto fold = [&](float slo, float shi) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[mi][ni][q] = fmaf(accb[mi][ni][q], ni < 2 ? slo : shi, acc[mi][ni][q]);
                    accb[mi][ni][q] = 0.f;
                }
    };
    // All 16 fragment reads of a stage (both 32-wide K halves) are issued
    // before the first MFMA, so the second half's reads land while the first
    // half multiplies.  Rows past the group end are zero in LDS; their reads
    // are harmless and their MFMAs are skipped.  With block scales the second
    // accumulator set leaves no room for both halves' fragments, so each half
    // is read just before it is used.
    auto compute = [&](int buf) {
        constexpr int kHalves = BLK ? 1 : 2;   // halves whose fragments are in registers at once
#pragma unroll
        for (int h0 = 0; h0 < 2; h0 += kHalves) {
            uint4 af[kHalves][4], bf[kHalves][4];
#pragma unroll
            for (int h = 0; h < kHalves; ++h) {
                const int kk = 32 * (h0 + h);
#pragma unroll
                for (int ni = 0; ni < 4; ++ni)
                    bf[h][ni] =
                        *reinterpret_cast<const uint4 *>(Bs[buf] + (b_row_of<WN>(wn, ni) + fr) * kLdsStride + kk + fk);
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
                    af[h][mi] =
                        *reinterpret_cast<const uint4 *>(As[buf] + (wm * 64 + mi * 16 + fr) * kLdsStride + kk + fk);
                __builtin_amdgcn_sched_barrier(0);   // keep the first half's reads ahead of the second's
            }
#pragma unroll
            for (int h = 0; h < kHalves; ++h)
#pragma unroll
                for (int mi = 0; mi < 4; ++mi) {
                    if (mi < live) {  // wave-uniform
                        // B fragment as the MFMA's first operand: the result is
                        // transposed, so a lane holds 4 consecutive output columns
                        // of one row (lane % 16 = row, 4 * (lane / 16) + q = column)
#pragma unroll
                        for (int ni = 0; ni < 4; ++ni) dst[mi][ni] = mfma_bf16(bf[h][ni], af[h][mi], dst[mi][ni]);
                    }
                }
        }
    };

    const int nk = K / kBK;
    Stage<FP8, XF32, WN> s0, s1;
    fetch(s0, 0);
    if (nk > 1) fetch(s1, kBK);
    stash(s0, 0);
    lds_barrier();
    // Steady state, two stages per trip with no conditional loads or stores
    // (slot s1 holds stage kt+1, issued one trip half earlier).  A branch-free
    // body lets the compiler's load counters see that only the other slot's
    // loads are outstanding; sched_barrier(0) pins the phase order so the
    // loads are issued first and stay in flight through two multiply phases.
    // With BLK each trip is exactly one 128-wide K block (kt is even).
    int kt = 0;
    for (; kt + 3 < nk; kt += 2) {
        float slo = 0.f, shi = 0.f;
        if (BLK) { slo = sc_lo[kt >> 1]; shi = sc_hi[kt >> 1]; }
        fetch(s0, (kt + 2) * kBK);
        __builtin_amdgcn_sched_barrier(0);
        compute(0);
        __builtin_amdgcn_sched_barrier(0);
        stash(s1, 1);
        lds_barrier();
        fetch(s1, (kt + 3) * kBK);
        __builtin_amdgcn_sched_barrier(0);
        compute(1);
        if (BLK) fold(slo, shi);
        __builtin_amdgcn_sched_barrier(0);
        stash(s0, 0);
        lds_barrier();
    }
    // tail: 1, 2 or 3 stages left (stage kt in LDS buffer 0, stage kt+1 in s1);
    // with BLK always 2 (K is a multiple of 128)
    const int left = nk - kt;
    if (left == 3) fetch(s0, (kt + 2) * kBK);
    compute(0);
    if (left >= 2) {
        stash(s1, 1);
        lds_barrier();
        compute(1);
        if (left == 3) {
            stash(s0, 0);
            lds_barrier();
            compute(0);
        }
    }
    if (BLK) fold(sc_lo[kt >> 1], sc_hi[kt >> 1]);
}

// weight modes: bfloat16, FP8 with per-channel scales, FP8 with 128x128 block scales
// (kWFp8BlkDma: block scales on the direct-to-LDS tile, chosen by the launcher)
enum { kWBf16 = 0, kWFp8Row = 1, kWFp8Blk = 2, kWFp8BlkDma = 3 };

// ---------------------------------------------------------------- direct-to-LDS tile
// bf16 x bf16 tile product with the operand tiles fetched straight into LDS
// (global_load_lds_dwordx4: each lane's 16 bytes land at the wave's LDS
// destination + 16 * lane), three stages deep, one barrier per stage, no
// register staging.  LDS rows are 128 bytes, unpadded; 16-byte chunk c of
// tile row r sits at chunk position c ^ (r & 7), which keeps the fragment
// reads free of bank conflicts.  Each lane therefore fetches, for its LDS
// slot, the chunk that the swizzle puts there: the callers pass per-lane
// source pointers for K = 0 that already include it.
//
// DMA j of wave w covers tile rows 8 * (w * n + j) .. + 7 (n = 2 for A, 4 for
// B): lane i fills row 8 * (w * n + j) + i / 8, position i % 8.
//
// Synchronisation and software pipeline.  Each 64-wide stage is consumed in
// two 32-wide K halves, and a wave holds two fragment sets: while the MFMAs
// of one half run from registers, the fragment reads of the next half are
// issued between them (sched_group_barrier interleaves the two streams), so
// LDS reads and matrix-core work overlap instead of alternating.  Before the
// reads of stage kt+1 (after the first half of stage kt has been
// multiplied) a wave waits until its own DMAs of stage kt+1 have landed
// (vmcnt counts only these loads: stage kt+2's may stay in flight), and the
// LDS barrier, whose release fence also completes the wave's own fragment
// reads, makes every wave's stage kt+1 data visible.  Right after it stage
// kt+3 is fetched into the buffer of stage kt: every wave has passed the
// barrier, so every wave's reads of that buffer are complete.  Rows past the
// group end hold some valid row's data; a wave's 16-row sub-tiles that lie
// wholly past it are neither read nor multiplied (the count of live sub-tiles
// is fixed per wave for the whole product, so each count has its own
// straight-line loop), and the remaining junk rows are never stored.
//
// The DMA is issued from inline assembly: the compiler's wait insertion
// cannot tell the three buffers apart across the loop and would wait for
// every DMA in flight before each stage's reads, which removes the prefetch.
// The instruction has no register result (its data goes to LDS), its address
// registers are read at issue, it saves and restores M0, and the explicit
// vmcnt waits above order it; the compiler's own waits only count its own
// loads, which vmcnt completes in order, so they can only wait longer.

// s_waitcnt vmcnt(N) with expcnt and lgkmcnt left at their no-wait maxima
#define FGS_VMCNT(N) (((N) & 0xF) | (((N) >> 4) << 14) | (0x7 << 4) | (0xF << 8))

typedef __attribute__((address_space(3))) void lds_void_t;

// 16 bytes per lane from `src` into LDS at `lds_addr` (wave-uniform) + 16 * lane
__device__ __forceinline__ void dma16(const void *src, const void *lds_dst) {
    const uint32_t dst = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t *)lds_dst);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(dst)
        : "memory");
}

// MFMA / fragment-read interleave for the scheduler: R reads spread over M
// MFMAs, the MFMAs first (their operands are already in registers)
template <int R, int M>
__device__ __forceinline__ void interleave_mfma_reads() {
    if constexpr (R > 0) {
        constexpr int mm = M / R;
        if constexpr (mm > 0) __builtin_amdgcn_sched_group_barrier(0x008, mm, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        interleave_mfma_reads<R - 1, M - mm>();
    } else if constexpr (M > 0) {
        __builtin_amdgcn_sched_group_barrier(0x008, M, 0);
    }
}

template <int N> struct Live { static constexpr int value = N; };

// The three stage buffers are distinct LDS objects and the stage loop is
// unrolled by three, so every buffer reference is static: the compiler then
// knows that a stage's fragment reads never alias the DMAs just issued into
// another buffer and does not wait for them.
__device__ __forceinline__ void tile_mma_dma(const uint16_t *const (&a_src)[kAPer],
                                             const uint16_t *const (&b_src)[kBPer], int K, int m,
                                             f32x4_t (&acc)[4][4]) {
    static_assert(kAPer == 2 && kBPer == 4, "six DMAs per wave and stage");
    __shared__ __attribute__((aligned(16))) uint8_t L0[kDmaStageB];
    __shared__ __attribute__((aligned(16))) uint8_t L1[kDmaStageB];
    __shared__ __attribute__((aligned(16))) uint8_t L2[kDmaStageB];
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / kWN, wn = wave % kWN;
    const int fr = lane & 15, fg = lane >> 4;
    const int nk = K / kBK;
    auto fetch = [&](int kt, uint8_t *buf) {
        const int k0 = kt * kBK;
#pragma unroll
        for (int j = 0; j < kAPer; ++j) dma16(a_src[j] + k0, buf + (wave * kAPer + j) * 1024);
#pragma unroll
        for (int j = 0; j < kBPer; ++j) dma16(b_src[j] + k0, buf + kBM * kDmaRowB + (wave * kBPer + j) * 1024);
    };
    // 16-byte fragment of tile row r, logical chunk c (8 bf16 along K)
    auto frag = [&](const uint8_t *base, int r, int c) {
        return *reinterpret_cast<const uint4 *>(base + r * kDmaRowB + ((c ^ (r & 7)) << 4));
    };
    auto wait_own = [&](int kt) {   // this wave's DMAs of stage kt landed (stage kt+1's may be in flight)
        if (kt + 1 < nk) __builtin_amdgcn_s_waitcnt(FGS_VMCNT(kAPer + kBPer));
        else __builtin_amdgcn_s_waitcnt(FGS_VMCNT(0));
    };

    fetch(0, L0);
    if (nk > 1) fetch(1, L1);
    wait_own(0);
    lds_barrier();
    if (nk > 2) fetch(2, L2);
    __builtin_amdgcn_sched_barrier(0);

    auto run = [&](auto live_c) {
        constexpr int LV = decltype(live_c)::value;   // live 16-row sub-tiles of this wave
        constexpr int R = LV > 0 ? 4 + LV : 0;         // fragment reads per half
        auto read_half = [&](const uint8_t *cur, int h, uint4 (&af)[4], uint4 (&bf)[4]) {
            if constexpr (LV > 0) {
                const int c = 4 * h + fg;   // K elements 32 h + 8 (lane / 16) ..
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) bf[ni] = frag(cur + kBM * kDmaRowB, b_row_of(wn, ni) + fr, c);
#pragma unroll
                for (int mi = 0; mi < LV; ++mi) af[mi] = frag(cur, wm * 64 + mi * 16 + fr, c);
            }
        };
        auto mma_half = [&](const uint4 (&af)[4], const uint4 (&bf)[4]) {
#pragma unroll
            for (int mi = 0; mi < LV; ++mi)
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = mfma_bf16(bf[ni], af[mi], acc[mi][ni]);
        };
        uint4 fa0[4], fb0[4], fa1[4], fb1[4];
        read_half(L0, 0, fa0, fb0);
        // stage kt from buffer `cur`; stage kt+1 is in `nxt`; stage kt+3 goes into `cur`
        auto stage = [&](int kt, uint8_t *cur, const uint8_t *nxt) {
            __builtin_amdgcn_sched_barrier(0);
            read_half(cur, 1, fa1, fb1);
            mma_half(fa0, fb0);
            interleave_mfma_reads<R, 4 * LV>();
            __builtin_amdgcn_sched_barrier(0);
            if (kt + 1 < nk) {
                wait_own(kt + 1);
                lds_barrier();
                if (kt + 3 < nk) fetch(kt + 3, cur);
                __builtin_amdgcn_sched_barrier(0);
                read_half(nxt, 0, fa0, fb0);
                mma_half(fa1, fb1);
                interleave_mfma_reads<R, 4 * LV>();
            } else {
                mma_half(fa1, fb1);
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        int kt = 0;
        for (; kt + 3 <= nk; kt += 3) {   // stage s uses buffer s % 3
            stage(kt, L0, L1);
            stage(kt + 1, L1, L2);
            stage(kt + 2, L2, L0);
        }
        if (kt < nk) stage(kt, L0, L1);
        if (kt + 1 < nk) stage(kt + 1, L1, L2);
    };
    // wave-uniform: the scalar branch picks the straight-line loop for this wave
    const int live = min(4, max(0, (m - wm * 64 + 15) / 16));
    switch (live) {
        case 4: run(Live<4>{}); break;
        case 3: run(Live<3>{}); break;
        case 2: run(Live<2>{}); break;
        case 1: run(Live<1>{}); break;
        default: run(Live<0>{}); break;
    }
}

// ---------------------------------------------------------------- FP8 weights, direct to LDS
// bf16 activations x E4M3 weights (one scale per output channel, applied in
// the epilogue) with both operand tiles fetched straight into LDS.  A 64-wide
// K stage holds 128 activation rows of 128 bytes and 256 weight rows of 64
// bytes, 32 KB, so four stages fit and the prefetch runs one stage deeper
// than the bf16 tile.  Weight rows: 16-byte chunk c of row r sits at
// position c ^ ((r >> 2) & 3), which spreads the 8-byte fragment reads of
// 16 consecutive rows over all banks.  A fragment read takes the 8 code bytes
// of its K range and widens them to bf16 exactly.  Synchronisation as in
// tile_mma_dma, with stage kt+4 fetched into the buffer of stage kt.
// K blocks of 128 whose scales a direct-to-LDS tile keeps in LDS for the whole
// product (K <= 3072); larger K takes the register-staged tiles
constexpr int kF8DmaMaxKb = 24;
constexpr int kW8RowB = 64;                                  // weight-row bytes per stage
constexpr int kW8StageB = kBM * kDmaRowB + kBN * kW8RowB;    // 32 KiB
static_assert(4 * kW8StageB <= 160 * 1024, "four FP8-weight stages must fit one CU's LDS");

__device__ __forceinline__ void tile_mma_dma_w8(const uint16_t *const (&a_src)[kAPer],
                                                const uint8_t *const (&b_src)[2], int K, int m,
                                                f32x4_t (&acc)[4][4]) {
    constexpr int G = kAPer + 2;   // DMAs per wave and stage
    __shared__ __attribute__((aligned(16))) uint8_t L0[kW8StageB];
    __shared__ __attribute__((aligned(16))) uint8_t L1[kW8StageB];
    __shared__ __attribute__((aligned(16))) uint8_t L2[kW8StageB];
    __shared__ __attribute__((aligned(16))) uint8_t L3[kW8StageB];
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / kWN, wn = wave % kWN;
    const int fr = lane & 15, fg = lane >> 4;
    const int nk = K / kBK;
    auto fetch = [&](int kt, uint8_t *buf) {
        const int k0 = kt * kBK;
#pragma unroll
        for (int j = 0; j < kAPer; ++j) dma16(a_src[j] + k0, buf + (wave * kAPer + j) * 1024);
#pragma unroll
        for (int j = 0; j < 2; ++j) dma16(b_src[j] + k0, buf + kBM * kDmaRowB + (wave * 2 + j) * 1024);
    };
    auto frag_a = [&](const uint8_t *base, int r, int c) {
        return *reinterpret_cast<const uint4 *>(base + r * kDmaRowB + ((c ^ (r & 7)) << 4));
    };
    // 8 weights of row r, K elements 8 u .. 8 u + 7 of the stage, as bf16
    auto frag_b = [&](const uint8_t *base, int r, int u) {
        const uint2 q = *reinterpret_cast<const uint2 *>(base + kBM * kDmaRowB + r * kW8RowB +
                                                         ((((u >> 1) ^ (r >> 2)) & 3) << 4) + ((u & 1) << 3));
        return e4m3x8_to_bf16x8(q);
    };
    // this wave's DMAs of stage kt+1 landed; later stages' may stay in flight
    auto wait_next = [&](int kt) {
        const int later = min(2, nk - 2 - kt);   // stages kt+2, kt+3 already issued
        if (later >= 2) __builtin_amdgcn_s_waitcnt(FGS_VMCNT(2 * G));
        else if (later == 1) __builtin_amdgcn_s_waitcnt(FGS_VMCNT(G));
        else __builtin_amdgcn_s_waitcnt(FGS_VMCNT(0));
    };

    fetch(0, L0);
    if (nk > 1) fetch(1, L1);
    if (nk > 2) fetch(2, L2);
    wait_next(-1);
    lds_barrier();
    if (nk > 3) fetch(3, L3);
    __builtin_amdgcn_sched_barrier(0);

    auto run = [&](auto live_c) {
        constexpr int LV = decltype(live_c)::value;
        constexpr int R = LV > 0 ? 4 + LV : 0;
        auto read_half = [&](const uint8_t *cur, int h, uint4 (&af)[4], uint4 (&bf)[4]) {
            if constexpr (LV > 0) {
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) bf[ni] = frag_b(cur, b_row_of(wn, ni) + fr, 4 * h + fg);
#pragma unroll
                for (int mi = 0; mi < LV; ++mi) af[mi] = frag_a(cur, wm * 64 + mi * 16 + fr, 4 * h + fg);
            }
        };
        auto mma_half = [&](const uint4 (&af)[4], const uint4 (&bf)[4]) {
#pragma unroll
            for (int mi = 0; mi < LV; ++mi)
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = mfma_bf16(bf[ni], af[mi], acc[mi][ni]);
        };
        uint4 fa0[4], fb0[4], fa1[4], fb1[4];
        read_half(L0, 0, fa0, fb0);
        auto stage = [&](int kt, uint8_t *cur, const uint8_t *nxt) {
            __builtin_amdgcn_sched_barrier(0);
            read_half(cur, 1, fa1, fb1);
            mma_half(fa0, fb0);
            interleave_mfma_reads<R, 4 * LV>();
            __builtin_amdgcn_sched_barrier(0);
            if (kt + 1 < nk) {
                wait_next(kt);
                lds_barrier();
                if (kt + 4 < nk) fetch(kt + 4, cur);
                __builtin_amdgcn_sched_barrier(0);
                read_half(nxt, 0, fa0, fb0);
                mma_half(fa1, fb1);
                interleave_mfma_reads<R, 4 * LV>();
            } else {
                mma_half(fa1, fb1);
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        int kt = 0;
        for (; kt + 4 <= nk; kt += 4) {   // stage s uses buffer s % 4
            stage(kt, L0, L1);
            stage(kt + 1, L1, L2);
            stage(kt + 2, L2, L3);
            stage(kt + 3, L3, L0);
        }
        if (kt < nk) stage(kt, L0, L1);
        if (kt + 1 < nk) stage(kt + 1, L1, L2);
        if (kt + 2 < nk) stage(kt + 2, L2, L3);
    };
    const int live = min(4, max(0, (m - wm * 64 + 15) / 16));
    switch (live) {
        case 4: run(Live<4>{}); break;
        case 3: run(Live<3>{}); break;
        case 2: run(Live<2>{}); break;
        case 1: run(Live<1>{}); break;
        default: run(Live<0>{}); break;
    }
}

// ---- FP8 weights with 128 x 128 block scales, bf16 activations, direct to
// LDS: the stages and swizzles of tile_mma_dma_w8 without its fragment
// pipeline.  The scale changes every other 64-wide stage, so each stage's
// products of a 16-row sub-tile are formed in fresh accumulators and folded
// into the running sum times the block's scale (the two stages of a block
// fold with the same scale), one sub-tile row behind the MFMAs as in
// tile_mma_f8.  The weight block scales of the whole K range are staged in
// LDS before the loop (K up to kF8DmaMaxKb blocks).
__device__ __forceinline__ void tile_mma_dma_w8b(const uint16_t *const (&a_src)[kAPer],
                                                 const uint8_t *const (&b_src)[2], const float *sw_lo,
                                                 const float *sw_hi, int K, int m, f32x4_t (&acc)[4][4]) {
    constexpr int G = kAPer + 2;   // DMAs per wave and stage
    __shared__ __attribute__((aligned(16))) uint8_t L0[kW8StageB];
    __shared__ __attribute__((aligned(16))) uint8_t L1[kW8StageB];
    __shared__ __attribute__((aligned(16))) uint8_t L2[kW8StageB];
    __shared__ __attribute__((aligned(16))) uint8_t L3[kW8StageB];
    __shared__ float sw_l[2][kF8DmaMaxKb];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / kWN, wn = wave % kWN;
    const int fr = lane & 15, fg = lane >> 4;
    const int nk = K / kBK, nkb = K / 128;
    auto fetch = [&](int kt, uint8_t *buf) {
        const int k0 = kt * kBK;
#pragma unroll
        for (int j = 0; j < kAPer; ++j) dma16(a_src[j] + k0, buf + (wave * kAPer + j) * 1024);
#pragma unroll
        for (int j = 0; j < 2; ++j) dma16(b_src[j] + k0, buf + kBM * kDmaRowB + (wave * 2 + j) * 1024);
    };
    auto frag_a = [&](const uint8_t *base, int r, int c) {
        return *reinterpret_cast<const uint4 *>(base + r * kDmaRowB + ((c ^ (r & 7)) << 4));
    };
    auto frag_b = [&](const uint8_t *base, int r, int u) {
        const uint2 q = *reinterpret_cast<const uint2 *>(base + kBM * kDmaRowB + r * kW8RowB +
                                                         ((((u >> 1) ^ (r >> 2)) & 3) << 4) + ((u & 1) << 3));
        return e4m3x8_to_bf16x8(q);
    };
    // this wave's DMAs of stage kt landed; stages kt+1, kt+2 (issued) may stay in flight
    auto wait_own = [&](int kt) {
        const int later = min(2, nk - 1 - kt);
        if (later >= 2) __builtin_amdgcn_s_waitcnt(FGS_VMCNT(2 * G));
        else if (later == 1) __builtin_amdgcn_s_waitcnt(FGS_VMCNT(G));
        else __builtin_amdgcn_s_waitcnt(FGS_VMCNT(0));
    };

    fetch(0, L0);
    if (nk > 1) fetch(1, L1);
    if (nk > 2) fetch(2, L2);
    const float wv = tid < 2 * nkb ? (tid < nkb ? sw_lo[tid] : sw_hi[tid - nkb]) : 0.f;
    if (tid < 2 * nkb) sw_l[tid / nkb][tid % nkb] = wv;   // waits for the loads above: prologue only

    const int live = min(4, max(0, (m - wm * 64 + 15) / 16));
    auto compute = [&](int kt, const uint8_t *cur) {
        uint4 bf[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) bf[h][ni] = frag_b(cur, b_row_of(wn, ni) + fr, 4 * h + fg);
        const float slo = sw_l[0][kt >> 1], shi = sw_l[1][kt >> 1];
        auto products = [&](int mi, f32x4_t (&pr)[4]) {
            const int r = wm * 64 + mi * 16 + fr;
            const uint4 a0 = frag_a(cur, r, fg), a1 = frag_a(cur, r, 4 + fg);
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
                pr[ni] = mfma_bf16(bf[1][ni], a1, mfma_bf16(bf[0][ni], a0, f32x4_t{0.f, 0.f, 0.f, 0.f}));
        };
        auto fold = [&](int mi, const f32x4_t (&pr)[4]) {
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) {
                const float c = ni < 2 ? slo : shi;
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[mi][ni][q] = fmaf(pr[ni][q], c, acc[mi][ni][q]);
            }
        };
        f32x4_t p0[4], p1[4];
        if (live > 0) products(0, p0);
        if (live > 1) products(1, p1);
        if (live > 0) fold(0, p0);
        if (live > 2) products(2, p0);
        if (live > 1) fold(1, p1);
        if (live > 3) products(3, p1);
        if (live > 2) fold(2, p0);
        if (live > 3) fold(3, p1);
    };
    // stage kt: own DMAs landed, barrier (every wave's stage kt visible, every
    // wave done with stage kt - 1), fetch stage kt + 3 into the buffer of
    // stage kt - 1, multiply
    auto step = [&](int kt, const uint8_t *cur, uint8_t *refill) {
        wait_own(kt);
        lds_barrier();
        if (kt + 3 < nk) fetch(kt + 3, refill);
        __builtin_amdgcn_sched_barrier(0);
        compute(kt, cur);
        __builtin_amdgcn_sched_barrier(0);
    };
    int kt = 0;
    for (; kt + 4 <= nk; kt += 4) {   // stage s uses buffer s % 4
        step(kt, L0, L3);
        step(kt + 1, L1, L0);
        step(kt + 2, L2, L1);
        step(kt + 3, L3, L2);
    }
    if (kt < nk) step(kt, L0, L3);
    if (kt + 1 < nk) step(kt + 1, L1, L0);
    if (kt + 2 < nk) step(kt + 2, L2, L1);
}

// ---------------------------------------------------------------- wide bf16 tile
// 256 rows x 256 GEMM columns per workgroup for bf16 activations and weights
// at large batches.  Per K stage the tile moves 64 KB of operands for 8.4
// MFLOP, 1.5 times the flops per byte of the 128-row tile; the rate at which
// one CU takes in operand bytes (a few tens of bytes per clock, whether they
// come from HBM or from L2) is what bounds both tiles, so the wider tile does
// more work per byte it takes in.  At prefill size (about 128-170 rows per
// expert) a 256-row tile also covers an expert's rows in one tile, so each
// weight slice is streamed once instead of once per 128 rows.
//
// 8 waves in 2 (rows) x 4 (columns), each wave 128 x 64 (8 x 4 sub-tiles of
// MFMA 16x16x32 bf16).  LDS (160 KB, all of it): activation tiles in two
// 32 KB buffers, weight tiles in three: the weights, read from HBM, are
// fetched two stages ahead, the activations (mostly L2 hits) one stage
// ahead.  Row layout and swizzle as in tile_mma_dma (128-byte rows, 16-byte
// chunk c of row r at position c ^ (r & 7)).  DMAs take a wave-uniform base
// in scalar registers (advanced by 128 bytes per stage) and a 32-bit
// per-lane byte offset, so the eight DMA sources of a wave cost eight VGPRs.
//
// Stage kt reads activation buffer kt % 2 and weight buffer kt % 3, its
// fragments read just before the MFMAs that use them (holding a whole half
// stage of fragments on top of 128 accumulator registers does not fit a
// wave's 256).  At the barrier that ends stage kt (every wave is done with
// stage kt's buffers, and its own DMAs of stage kt+1 have landed) the
// activations of stage kt+2 are fetched into buffer kt % 2 and the weights of
// stage kt+3 into buffer kt % 3.  DMAs are issued in the order A(kt+1),
// B(kt+2), A(kt+2), B(kt+3), ..., so "stage kt+1 landed" is vmcnt(4) (only
// the weight DMAs of stage kt+2 remain, which keeps the memory pipe busy
// across the barrier), or vmcnt(0) near the end.
#ifndef FGS_WIDE_WMW
#define FGS_WIDE_WMW 4
#endif
constexpr int kBMW = 256;                        // rows per wide tile
constexpr int kWideBufB = kBMW * kDmaRowB;       // 32 KB: one operand tile of one stage
// WMW waves along the rows (4 along the columns): 4 * WMW waves, each (256 / WMW) x 64
template <int WMW> struct Wide {
    static constexpr int kWaves = 4 * WMW;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kRowsPerWave = kBMW / WMW;
    static constexpr int kSub = kRowsPerWave / 16;        // 16-row sub-tiles per wave
    static constexpr int kDma = 32 / kWaves;              // DMAs per wave per operand and stage (1 KB each)
};
constexpr int kWideWMW = FGS_WIDE_WMW;
static_assert(2 * kWideBufB + 3 * kWideBufB <= 160 * 1024, "the wide tile's buffers must fit one CU's LDS");

// 16 bytes per lane from sbase + voff into LDS at `lds_dst` (wave-uniform) + 16 * lane
__device__ __forceinline__ const uint8_t *uniform_ptr(const void *p);
__device__ __forceinline__ void dma16s(const void *sbase_any, uint32_t voff, const void *lds_dst) {
    const uint32_t dst = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t *)lds_dst);
    const uint8_t *sbase = uniform_ptr(sbase_any);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(sbase), "s"(dst)
        : "memory");
}

// 4 bytes per lane from sbase + voff into LDS at `lds_dst` (wave-uniform) + 4 * lane
__device__ __forceinline__ void dma4s(const void *sbase_any, uint32_t voff, const void *lds_dst) {
    const uint32_t dst = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t *)lds_dst);
    const uint8_t *sbase = uniform_ptr(sbase_any);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "global_load_lds_dword %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(sbase), "s"(dst)
        : "memory");
}

// a pointer known to be the same in every lane, kept in scalar registers
__device__ __forceinline__ const uint8_t *uniform_ptr(const void *p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const uint8_t *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// a_base/b_base[j]: wave-uniform bases of DMA j; a_off/b_off[j]: this lane's
// byte offset (row and swizzled chunk of its LDS slot) at K = 0.
typedef __attribute__((address_space(3))) const u32x4_t lds_u32x4_t;
// 4-byte LDS read at a 32-bit LDS byte address
__device__ __forceinline__ float lds_read_f32(uint32_t addr) {
    return *reinterpret_cast<__attribute__((address_space(3))) const float *>((size_t)addr);
}
// 16-byte LDS read at a 32-bit LDS byte address
__device__ __forceinline__ uint4 lds_read16(uint32_t addr) {
    const u32x4_t v = *reinterpret_cast<lds_u32x4_t *>((size_t)addr);
    return make_uint4(v.x, v.y, v.z, v.w);
}

template <int WMW>
__device__ __forceinline__ void tile_mma_wide(const uint8_t *a_base, const uint32_t (&a_off)[Wide<WMW>::kDma],
                                              const uint8_t *const (&b_base)[Wide<WMW>::kDma],
                                              const uint32_t (&b_off)[Wide<WMW>::kDma], int K, int m,
                                              f32x4_t (&acc)[Wide<WMW>::kSub][4]) {
    using WG = Wide<WMW>;
    constexpr int kAPerW = WG::kDma, kBPerW = WG::kDma, kSub = WG::kSub, kRW = WG::kRowsPerWave;
    // one LDS array: activation buffers at 0 and 32 KB, weight buffers at 64, 96 and 128 KB
    __shared__ __attribute__((aligned(1024))) uint8_t smem[5 * kWideBufB];
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / kWN, wn = wave % kWN;
    const int fr = lane & 15, fg = lane >> 4;
    const int nk = K / kBK;
    const uint32_t s0 = (uint32_t)(uintptr_t)(lds_void_t *)smem;
    auto fetch_a = [&](int kt, int buf) {
        const uint8_t *sb = a_base + kt * (kBK * 2);
#pragma unroll
        for (int j = 0; j < kAPerW; ++j)
            dma16s(sb, a_off[j], smem + buf * kWideBufB + (wave * kAPerW + j) * 1024);
    };
    auto fetch_b = [&](int kt, int buf) {
#pragma unroll
        for (int j = 0; j < kBPerW; ++j)
            dma16s(b_base[j] + kt * (kBK * 2), b_off[j], smem + (2 + buf) * kWideBufB + (wave * kBPerW + j) * 1024);
    };
    // this lane's fragment byte offsets within a buffer, per 32-wide K half h: row
    // (wave row base + lane % 16) or B row (wave column base + lane % 16) and the
    // swizzled chunk 4 h + lane / 16 (the row's low three bits are those of lane % 16)
    const int r_a = wm * kRW + fr, r_b = wn * 32 + fr;
    const uint32_t la0 = s0 + r_a * kDmaRowB + (((0 + fg) ^ (fr & 7)) << 4);
    const uint32_t la1 = s0 + r_a * kDmaRowB + (((4 + fg) ^ (fr & 7)) << 4);
    const uint32_t lb0 = s0 + 2 * kWideBufB + r_b * kDmaRowB + (((0 + fg) ^ (fr & 7)) << 4);
    const uint32_t lb1 = s0 + 2 * kWideBufB + r_b * kDmaRowB + (((4 + fg) ^ (fr & 7)) << 4);
    // weight buffers lie past 64 KB, beyond the LDS read's 16-bit offset: one base
    // register per buffer and half, the rest in the offset
    const uint32_t lbb[3][2] = {{lb0, lb1}, {lb0 + kWideBufB, lb1 + kWideBufB},
                                {lb0 + 2 * kWideBufB, lb1 + 2 * kWideBufB}};

    // prologue: A(0) B(0) A(1) B(1) B(2); stage 0 landed once only A(1) B(1) B(2) may remain
    fetch_a(0, 0);
    fetch_b(0, 0);
    if (nk > 1) { fetch_a(1, 1); fetch_b(1, 1); }
    if (nk > 2) fetch_b(2, 2);
    if (nk > 2) __builtin_amdgcn_s_waitcnt(FGS_VMCNT(kAPerW + 2 * kBPerW));
    else if (nk > 1) __builtin_amdgcn_s_waitcnt(FGS_VMCNT(kAPerW + kBPerW));
    else __builtin_amdgcn_s_waitcnt(FGS_VMCNT(0));
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);

    auto run = [&](auto live_c) {
        constexpr int LV = decltype(live_c)::value;   // live 16-row sub-tiles of this wave
        // stage kt: activation buffer AB (kt % 2), weight buffer BB (kt % 3).
        // Fragments are read as the MFMAs need them: the four weight fragments
        // of a 32-wide K half, then one activation fragment per 16-row sub-tile
        // (the next one requested before the current one's MFMAs)
        auto stage = [&](int kt, auto ab_c, auto bb_c) {
            constexpr int AB = decltype(ab_c)::value, BB = decltype(bb_c)::value;
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (LV > 0) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t la = (h ? la1 : la0) + AB * kWideBufB;
                    const uint32_t lb = lbb[BB][h];
                    uint4 bf[4];
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni)   // B rows wn*32 + 16 ni (ni < 2), 128 + wn*32 + 16 (ni - 2)
                        bf[ni] = lds_read16(lb + (ni < 2 ? ni * 16 : 128 + (ni - 2) * 16) * kDmaRowB);
                    uint4 a = lds_read16(la);
#pragma unroll
                    for (int mi = 0; mi < LV; ++mi) {
                        const uint4 an = mi + 1 < LV ? lds_read16(la + (mi + 1) * 16 * kDmaRowB) : a;
#pragma unroll
                        for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = mfma_bf16(bf[ni], a, acc[mi][ni]);
                        a = an;
                    }
                    // the next half's reads stay behind this half's MFMAs (registers: four
                    // waves per SIMD leave 128 a wave; the other waves hide the read latency)
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            if (kt + 1 < nk) {
                // own DMAs of stage kt+1 landed (the weights of stage kt+2 may remain), and
                // every wave is done with buffers kt % 2 and kt % 3: refill them
                if (kt + 2 < nk) __builtin_amdgcn_s_waitcnt(FGS_VMCNT(kBPerW));
                else __builtin_amdgcn_s_waitcnt(FGS_VMCNT(0));
                lds_barrier();
                if (kt + 2 < nk) fetch_a(kt + 2, AB);
                if (kt + 3 < nk) fetch_b(kt + 3, BB);
            }
        };
        int kt = 0;
        for (; kt + 6 <= nk; kt += 6) {   // stage s: activations s % 2, weights s % 3
            stage(kt, Live<0>{}, Live<0>{});
            stage(kt + 1, Live<1>{}, Live<1>{});
            stage(kt + 2, Live<0>{}, Live<2>{});
            stage(kt + 3, Live<1>{}, Live<0>{});
            stage(kt + 4, Live<0>{}, Live<1>{});
            stage(kt + 5, Live<1>{}, Live<2>{});
        }
        if (kt < nk) stage(kt, Live<0>{}, Live<0>{});
        if (kt + 1 < nk) stage(kt + 1, Live<1>{}, Live<1>{});
        if (kt + 2 < nk) stage(kt + 2, Live<0>{}, Live<2>{});
        if (kt + 3 < nk) stage(kt + 3, Live<1>{}, Live<0>{});
        if (kt + 4 < nk) stage(kt + 4, Live<0>{}, Live<1>{});
    };
    // wave-uniform live count (8 sub-tiles per wave: rounded up to even; the extra
    // sub-tile's rows are never stored)
    const int live = min(kSub, max(0, (m - wm * kRW + 15) / 16));
    if constexpr (kSub == 8) {
        switch ((live + 1) & ~1) {
            case 8: run(Live<8>{}); break;
            case 6: run(Live<6>{}); break;
            case 4: run(Live<4>{}); break;
            case 2: run(Live<2>{}); break;
            default: run(Live<0>{}); break;
        }
    } else {
        switch (live) {
            case 4: run(Live<4>{}); break;
            case 3: run(Live<3>{}); break;
            case 2: run(Live<2>{}); break;
            case 1: run(Live<1>{}); break;
            default: run(Live<0>{}); break;
        }
    }
}

// ---- the wide tile with E4M3 weights (one FP32 scale per output channel,
// applied in the epilogue) and bf16 activations: 16 waves of 64 x 64.  A
// stage holds 256 activation rows of 128 bytes (32 KB) and 256 weight rows of
// 64 bytes (16 KB; chunk c of row r at position c ^ ((r >> 2) & 3), as in
// tile_mma_dma_w8), three buffers of each (144 KB), both operands fetched two
// stages ahead: at the barrier that ends stage kt (own DMAs of stage kt+1
// landed; stage kt+2's may remain) stage kt+3 is fetched into buffers kt % 3.
// A fragment read takes the 8 code bytes of its K range and widens them to
// bf16 exactly.
constexpr int kWideW8BufB = kBMW * kW8RowB;   // 16 KB
typedef uint32_t u32x2v_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) const u32x2v_t lds_u32x2_t;
__device__ __forceinline__ uint2 lds_read8(uint32_t addr) {
    const u32x2v_t v = *reinterpret_cast<lds_u32x2_t *>((size_t)addr);
    return make_uint2(v.x, v.y);
}

template <int WMW>
__device__ __forceinline__ void tile_mma_wide_w8(const uint8_t *a_base, const uint32_t (&a_off)[Wide<WMW>::kDma],
                                                 const uint8_t *b_base, uint32_t b_off, int K, int m,
                                                 f32x4_t (&acc)[Wide<WMW>::kSub][4]) {
    using WG = Wide<WMW>;
    constexpr int kAPerW = WG::kDma, kSub = WG::kSub, kRW = WG::kRowsPerWave;
    static_assert(WG::kWaves == 16, "one weight DMA per wave and stage");
    constexpr int G = kAPerW + 1;   // DMAs per wave and stage
    // weight buffers at 0, 16 and 32 KB (their reads fit the 16-bit offset), activations at 48, 80, 112 KB
    constexpr int kAOff = 3 * kWideW8BufB;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[3 * kWideW8BufB + 3 * kWideBufB];
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / kWN, wn = wave % kWN;
    const int fr = lane & 15, fg = lane >> 4;
    const int nk = K / kBK;
    const uint32_t s0 = (uint32_t)(uintptr_t)(lds_void_t *)smem;
    auto fetch = [&](int kt, int buf) {
        const uint8_t *sa = a_base + kt * (kBK * 2);
#pragma unroll
        for (int j = 0; j < kAPerW; ++j)
            dma16s(sa, a_off[j], smem + kAOff + buf * kWideBufB + (wave * kAPerW + j) * 1024);
        dma16s(b_base + kt * kBK, b_off, smem + buf * kWideW8BufB + wave * 1024);
    };
    // this lane's fragment addresses per 32-wide K half h: activation row
    // (wave row base + lane % 16), chunk 4 h + lane / 16; weight row (wave
    // column base + lane % 16), code bytes 8 (4 h + lane / 16) .. + 7
    const int r_a = wm * kRW + fr, r_b = wn * 32 + fr;
    uint32_t la[3][2], lb[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int c = 4 * h + fg;
#pragma unroll
        for (int q = 0; q < 3; ++q) la[q][h] = s0 + kAOff + q * kWideBufB + r_a * kDmaRowB + ((c ^ (fr & 7)) << 4);
        lb[h] = s0 + r_b * kW8RowB + ((((c >> 1) ^ (fr >> 2)) & 3) << 4) + ((c & 1) << 3);
    }

    fetch(0, 0);
    if (nk > 1) fetch(1, 1);
    if (nk > 2) fetch(2, 2);
    if (nk > 2) __builtin_amdgcn_s_waitcnt(FGS_VMCNT(2 * G));
    else if (nk > 1) __builtin_amdgcn_s_waitcnt(FGS_VMCNT(G));
    else __builtin_amdgcn_s_waitcnt(FGS_VMCNT(0));
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);

    auto run = [&](auto live_c) {
        constexpr int LV = decltype(live_c)::value;
        auto stage = [&](int kt, auto s_c) {
            constexpr int S = decltype(s_c)::value;   // buffer kt % 3
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (LV > 0) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    uint4 bf[4];
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni)   // B rows wn*32 + 16 ni (ni < 2), 128 + wn*32 + 16 (ni - 2)
                        bf[ni] = e4m3x8_to_bf16x8(
                            lds_read8(lb[h] + S * kWideW8BufB + (ni < 2 ? ni * 16 : 128 + (ni - 2) * 16) * kW8RowB));
                    uint4 a = lds_read16(la[S][h]);
#pragma unroll
                    for (int mi = 0; mi < LV; ++mi) {
                        const uint4 an = mi + 1 < LV ? lds_read16(la[S][h] + (mi + 1) * 16 * kDmaRowB) : a;
#pragma unroll
                        for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = mfma_bf16(bf[ni], a, acc[mi][ni]);
                        a = an;
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            if (kt + 1 < nk) {
                if (kt + 2 < nk) __builtin_amdgcn_s_waitcnt(FGS_VMCNT(G));
                else __builtin_amdgcn_s_waitcnt(FGS_VMCNT(0));
                lds_barrier();
                if (kt + 3 < nk) fetch(kt + 3, S);
            }
        };
        int kt = 0;
        for (; kt + 3 <= nk; kt += 3) {   // stage s uses buffers s % 3
            stage(kt, Live<0>{});
            stage(kt + 1, Live<1>{});
            stage(kt + 2, Live<2>{});
        }
        if (kt < nk) stage(kt, Live<0>{});
        if (kt + 1 < nk) stage(kt + 1, Live<1>{});
    };
    const int live = min(kSub, max(0, (m - wm * kRW + 15) / 16));
    switch (live) {
        case 4: run(Live<4>{}); break;
        case 3: run(Live<3>{}); break;
        case 2: run(Live<2>{}); break;
        case 1: run(Live<1>{}); break;
        default: run(Live<0>{}); break;
    }
}

// bf16 x with bf16 weights (W8 false) or E4M3 weights with per-channel scales (W8 true),
// 256-row tiles.  grid: (ceil(max(f, fs) / 128), tile capacity); block 256 * WMW
template <int WMW, bool W8>
__global__ __launch_bounds__(Wide<WMW>::kThreads) void gate_up_gemm_wide_kernel(
    const uint16_t *__restrict__ x, const void *__restrict__ wg, const void *__restrict__ wu,
    const float *__restrict__ sg, const float *__restrict__ su, const void *__restrict__ wsg,
    const void *__restrict__ wsu, const float *__restrict__ ssg, const float *__restrict__ ssu,
    const int32_t *__restrict__ tiles, const int32_t *__restrict__ n_tiles, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ por, uint16_t *__restrict__ H, int ldh, int d, int E, int k, int f, int fs) {
    int item;
    if (!xcd_item(*n_tiles * (int)gridDim.x, item)) return;
    const int u = item / gridDim.x;
    const int g = tiles[2 * u], m0 = tiles[2 * u + 1];
    const bool shared = g == E;
    const int fg = shared ? fs : f;
    constexpr int kHalf = kBN / 2;  // H columns per tile
    const int c0 = (item % gridDim.x) * kHalf;
    if (c0 >= fg) return;
    const int gstart = offsets[g];
    const int row0 = gstart + m0, m = min(kBMW, offsets[g + 1] - row0);
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), pos = lane & 7;
    auto token_row = [&](int r) { return shared ? (row0 + r - gstart) : por[row0 + r] / k; };
    using WG = Wide<WMW>;
    constexpr int kAPerW = WG::kDma, kSub = WG::kSub, kRW = WG::kRowsPerWave;
    constexpr int kBPerW = W8 ? 1 : WG::kDma;
    constexpr int sw = W8 ? 1 : 2;   // bytes per weight
    // lane i of activation DMA j of wave w fills tile row 8 (n w + j) + i / 8 at swizzled chunk position i % 8
    uint32_t a_off[kAPerW], b_off[kBPerW];
    const uint8_t *b_base[kBPerW];
#pragma unroll
    for (int j = 0; j < kAPerW; ++j) {
        const int r = 8 * (w * kAPerW + j) + (lane >> 3);
        const int t = token_row(r < m ? r : 0);   // rows past the group end read row 0 (never stored)
        a_off[j] = (uint32_t)t * (uint32_t)(2 * d) + (uint32_t)((pos ^ (r & 7)) << 4);
    }
    // weight rows: tile rows [0, 128) are gate rows c0.., [128, 256) the matching up rows;
    // the first half of the waves fetch gate rows, the rest up rows
    const size_t wrow0 = shared ? 0 : (size_t)g * f;
    const uint8_t *gate_m = uniform_ptr((const uint8_t *)(shared ? wsg : wg) + wrow0 * d * sw);
    const uint8_t *up_m = uniform_ptr((const uint8_t *)(shared ? wsu : wu) + wrow0 * d * sw);
#pragma unroll
    for (int j = 0; j < kBPerW; ++j) {
        // bf16: lane i of DMA j fills row 8 (n w + j) + i / 8, position i % 8 (chunk (i % 8) ^ (row & 7));
        // E4M3: lane i of the wave's DMA fills row 16 w + i / 4, position i % 4 (chunk (i % 4) ^ ((row >> 2) & 3))
        const int r = W8 ? 16 * w + (lane >> 2) : 8 * (w * kBPerW + j) + (lane >> 3);
        const int c = c0 + (r & (kHalf - 1));
        const int chunk = W8 ? (((lane & 3) ^ (r >> 2)) & 3) : (pos ^ (r & 7));
        b_base[j] = w < WG::kWaves / 2 ? gate_m : up_m;
        // columns past f_g (only when f_g is not a multiple of 128) re-read column c0; never stored
        b_off[j] = (uint32_t)(c < fg ? c : c0) * (uint32_t)(sw * d) + (uint32_t)(chunk << 4);
    }
    f32x4_t acc[kSub][4];
#pragma unroll
    for (int i = 0; i < kSub; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if constexpr (W8) tile_mma_wide_w8<WMW>(uniform_ptr(x), a_off, b_base[0], b_off[0], d, m, acc);
    else tile_mma_wide<WMW>(uniform_ptr(x), a_off, b_base, b_off, d, m, acc);

    // epilogue: acc[mi][ni][q] is row wm*kRW + mi*16 + lane%16, GEMM column
    // b_row_of(wn, ni) + 4*(lane/16) + q; gate tile ni and up tile ni+2 share
    // (row, H column), so each lane writes 4 consecutive H values
    const int wm = w >> 2, wn = w & 3;
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
        const int col = c0 + wn * 32 + ni * 16 + (lane >> 4) * 4;
        if (col >= fg) continue;  // f_g is a multiple of 64: all four in range or all out
        float gs[4] = {1.f, 1.f, 1.f, 1.f}, us[4] = {1.f, 1.f, 1.f, 1.f};
        if (W8) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                gs[q] = shared ? ssg[col + q] : sg[wrow0 + col + q];
                us[q] = shared ? ssu[col + q] : su[wrow0 + col + q];
            }
        }
#pragma unroll
        for (int mi = 0; mi < kSub; ++mi) {
            const int r = wm * kRW + mi * 16 + (lane & 15);
            if (r < m) {
                float hv[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) hv[q] = silu(acc[mi][ni][q] * gs[q]) * (acc[mi][ni + 2][q] * us[q]);
                *reinterpret_cast<uint2 *>(H + (size_t)(row0 + r) * ldh + col) =
                    make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
            }
        }
    }
}

// grid: (ceil(max(f, fs) / 128), tile capacity); block 512; LDS kGemmLds
// (bf16 x and weights: none; the direct-to-LDS tile uses kGemmLdsDma of static LDS)
template <int WM, bool XF32>
__global__ __launch_bounds__(kThreads) void gate_up_gemm_kernel(
    const void *__restrict__ x, const void *__restrict__ wg, const void *__restrict__ wu,
    const float *__restrict__ sg, const float *__restrict__ su, const void *__restrict__ wsg,
    const void *__restrict__ wsu, const float *__restrict__ ssg, const float *__restrict__ ssu,
    const int32_t *__restrict__ tiles, const int32_t *__restrict__ n_tiles, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ por, uint16_t *__restrict__ H, int ldh, int d, int E, int k, int f, int fs) {
    constexpr bool FP8 = WM != kWBf16, BLK = WM == kWFp8Blk || WM == kWFp8BlkDma;
    extern __shared__ uint16_t lds[];
    int item;
    if (!xcd_item(*n_tiles * (int)gridDim.x, item)) return;
    const int u = item / gridDim.x;
    const int g = tiles[2 * u], m0 = tiles[2 * u + 1];
    const bool shared = g == E;
    const int fg = shared ? fs : f;
    constexpr int kHalf = kBN / 2;  // H columns per tile
    const int c0 = (item % gridDim.x) * kHalf;
    if (c0 >= fg) return;
    const int gstart = offsets[g];
    const int row0 = gstart + m0, m = min(kBM, offsets[g + 1] - row0);
    const int tid = threadIdx.x;

    size_t a_off[kAPer], b_off[kBPer];
    bool a_ok[kAPer];
    const void *b_base[kBPer];
    const size_t wrow0 = shared ? 0 : (size_t)g * f;
    auto token_row = [&](int r) { return shared ? (row0 + r - gstart) : por[row0 + r] / k; };
#pragma unroll
    for (int j = 0; j < kAPer; ++j) {
        const int r = (tid >> 3) + 64 * j;
        a_ok[j] = r < m;
        const int rr = a_ok[j] ? r : 0;  // rows past the group end read row 0 (masked when stored)
        a_off[j] = (size_t)token_row(rr) * d;
    }
#pragma unroll
    for (int j = 0; j < kBPer; ++j) {
        const int r = (tid >> 3) + 64 * j;
        const bool up = r >= kHalf;
        // columns past f_g (only when f_g is not a multiple of 128) re-read column c0; never stored
        const int c = c0 + (r & (kHalf - 1));
        b_base[j] = up ? (shared ? wsu : wu) : (shared ? wsg : wg);
        b_off[j] = (wrow0 + (c < fg ? c : c0)) * (size_t)d;
    }
    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if constexpr (WM == kWBf16 && !XF32) {
        // direct-to-LDS tile: lane i of DMA j of wave w fills tile row
        // 8 (w n + j) + i / 8 at swizzled chunk position i % 8
        const int lane = tid & 63, w = tid >> 6, pos = lane & 7;
        const uint16_t *a_src[kAPer], *b_src[kBPer];
#pragma unroll
        for (int j = 0; j < kAPer; ++j) {
            const int r = 8 * (w * kAPer + j) + (lane >> 3);
            const int t = token_row(r < m ? r : 0);
            a_src[j] = (const uint16_t *)x + (size_t)t * d + ((pos ^ (r & 7)) << 3);
        }
#pragma unroll
        for (int j = 0; j < kBPer; ++j) {
            const int r = 8 * (w * kBPer + j) + (lane >> 3);
            const bool up = r >= kHalf;
            const int c = c0 + (r & (kHalf - 1));
            const uint16_t *wb = (const uint16_t *)(up ? (shared ? wsu : wu) : (shared ? wsg : wg));
            b_src[j] = wb + (wrow0 + (c < fg ? c : c0)) * (size_t)d + ((pos ^ (r & 7)) << 3);
        }
        tile_mma_dma(a_src, b_src, d, m, acc);
    } else if constexpr ((WM == kWFp8Row || WM == kWFp8BlkDma) && !XF32) {
        // FP8 weights direct to LDS: activations as in the bf16 tile; lane i
        // of weight DMA j of wave w fills weight row 16 (2 w + j) + i / 4 at
        // chunk position i % 4 (source chunk (i % 4) ^ ((row >> 2) & 3))
        const int lane = tid & 63, w = tid >> 6, pos = lane & 7;
        const uint16_t *a_src[kAPer];
        const uint8_t *b_src[2];
#pragma unroll
        for (int j = 0; j < kAPer; ++j) {
            const int r = 8 * (w * kAPer + j) + (lane >> 3);
            const int t = token_row(r < m ? r : 0);
            a_src[j] = (const uint16_t *)x + (size_t)t * d + ((pos ^ (r & 7)) << 3);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int r = 16 * (w * 2 + j) + (lane >> 2);
            const bool up = r >= kHalf;
            const int c = c0 + (r & (kHalf - 1));
            const uint8_t *wb = (const uint8_t *)(up ? (shared ? wsu : wu) : (shared ? wsg : wg));
            b_src[j] = wb + (wrow0 + (c < fg ? c : c0)) * (size_t)d + ((((lane & 3) ^ (r >> 2)) & 3) << 4);
        }
        if constexpr (WM == kWFp8BlkDma) {
            // the tile's 128 gate (and up) rows are output block c0/128
            const size_t sb = ((shared ? 0 : (size_t)g * (f / 128)) + c0 / 128) * (size_t)(d / 128);
            tile_mma_dma_w8b(a_src, b_src, (shared ? ssg : sg) + sb, (shared ? ssu : su) + sb, d, m, acc);
        } else {
            tile_mma_dma_w8(a_src, b_src, d, m, acc);
        }
    } else {
        // block scales: the tile's 128 gate (and up) rows are output block c0/128
        const float *sc_lo = nullptr, *sc_hi = nullptr;
        if (BLK) {
            const size_t sb = ((shared ? 0 : (size_t)g * (f / 128)) + c0 / 128) * (size_t)(d / 128);
            sc_lo = (shared ? ssg : sg) + sb;
            sc_hi = (shared ? ssu : su) + sb;
        }
        tile_mma<FP8, XF32, kWN, BLK>(x, a_off, a_ok, b_base, b_off, 0, d, d, m, lds, acc, sc_lo, sc_hi);
    }

    // epilogue: acc[mi][ni][q] is row wm*64 + mi*16 + lane%16, GEMM column
    // (B row) b_row_of(wn, ni) + 4*(lane/16) + q; gate tile ni and up tile
    // ni+2 share (row, H column), so each lane writes 4 consecutive H values
    const int lane = tid & 63, wave = tid >> 6, wm = wave >> 2, wn = wave & 3;
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
        const int col = c0 + wn * 32 + ni * 16 + (lane >> 4) * 4;
        if (col >= fg) continue;  // f_g is a multiple of 64: all four in range or all out
        float gs[4] = {1.f, 1.f, 1.f, 1.f}, us[4] = {1.f, 1.f, 1.f, 1.f};
        if (WM == kWFp8Row) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                gs[q] = shared ? ssg[col + q] : sg[wrow0 + col + q];
                us[q] = shared ? ssu[col + q] : su[wrow0 + col + q];
            }
        }
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const int r = wm * 64 + mi * 16 + (lane & 15);
            if (r < m) {
                float hv[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) hv[q] = silu(acc[mi][ni][q] * gs[q]) * (acc[mi][ni + 2][q] * us[q]);
                *reinterpret_cast<uint2 *>(H + (size_t)(row0 + r) * ldh + col) =
                    make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
            }
        }
    }
}

// grid: (ceil(d / 256), tile capacity); block 512; LDS kGemmLds
template <int WM>
__global__ __launch_bounds__(kThreads) void down_gemm_kernel(
    const uint16_t *__restrict__ H, int ldh, const void *__restrict__ wd, const float *__restrict__ sd,
    const void *__restrict__ wsd, const float *__restrict__ ssd, const int32_t *__restrict__ tiles,
    const int32_t *__restrict__ n_tiles, const int32_t *__restrict__ offsets, uint16_t *__restrict__ Y, int d, int E,
    int f, int fs) {
    constexpr bool FP8 = WM != kWBf16, BLK = WM == kWFp8Blk || WM == kWFp8BlkDma;
    extern __shared__ uint16_t lds[];
    int item;
    if (!xcd_item(*n_tiles * (int)gridDim.x, item)) return;
    const int u = item / gridDim.x;
    const int g = tiles[2 * u], m0 = tiles[2 * u + 1];
    const bool shared = g == E;
    const int fg = shared ? fs : f;
    const int o0 = (item % gridDim.x) * kBN;
    const int row0 = offsets[g] + m0, m = min(kBM, offsets[g + 1] - row0);
    const int tid = threadIdx.x;
    const void *base = shared ? wsd : wd;
    const size_t obase = shared ? 0 : (size_t)g * d;

    size_t a_off[kAPer], b_off[kBPer];
    bool a_ok[kAPer];
    const void *b_base[kBPer];
#pragma unroll
    for (int j = 0; j < kAPer; ++j) {
        const int r = (tid >> 3) + 64 * j;
        a_ok[j] = r < m;
        a_off[j] = (size_t)(row0 + (a_ok[j] ? r : 0)) * ldh;
    }
#pragma unroll
    for (int j = 0; j < kBPer; ++j) {
        const int r = (tid >> 3) + 64 * j;
        b_base[j] = base;
        // B row r is output row o0 + r (rows past d re-read row 0; never stored)
        b_off[j] = (obase + (o0 + r < d ? o0 + r : 0)) * (size_t)fg;
    }
    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if constexpr (WM == kWBf16) {
        // direct-to-LDS tile (see the gate/up kernel for the lane -> row map)
        const int lane = tid & 63, w = tid >> 6, pos = lane & 7;
        const uint16_t *a_src[kAPer], *b_src[kBPer];
#pragma unroll
        for (int j = 0; j < kAPer; ++j) {
            const int r = 8 * (w * kAPer + j) + (lane >> 3);
            a_src[j] = H + (size_t)(row0 + (r < m ? r : 0)) * ldh + ((pos ^ (r & 7)) << 3);
        }
#pragma unroll
        for (int j = 0; j < kBPer; ++j) {
            const int r = 8 * (w * kBPer + j) + (lane >> 3);
            b_src[j] = (const uint16_t *)base + (obase + (o0 + r < d ? o0 + r : 0)) * (size_t)fg + ((pos ^ (r & 7)) << 3);
        }
        tile_mma_dma(a_src, b_src, fg, m, acc);
    } else if constexpr (WM == kWFp8Row || WM == kWFp8BlkDma) {
        // FP8 weights direct to LDS (see the gate/up kernel for the lane -> row map)
        const int lane = tid & 63, w = tid >> 6, pos = lane & 7;
        const uint16_t *a_src[kAPer];
        const uint8_t *b_src[2];
#pragma unroll
        for (int j = 0; j < kAPer; ++j) {
            const int r = 8 * (w * kAPer + j) + (lane >> 3);
            a_src[j] = H + (size_t)(row0 + (r < m ? r : 0)) * ldh + ((pos ^ (r & 7)) << 3);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int r = 16 * (w * 2 + j) + (lane >> 2);
            b_src[j] = (const uint8_t *)base + (obase + (o0 + r < d ? o0 + r : 0)) * (size_t)fg +
                       ((((lane & 3) ^ (r >> 2)) & 3) << 4);
        }
        if constexpr (WM == kWFp8BlkDma) {
            // B rows [0, 128) are output block o0/128, rows [128, 256) the next
            // one (clamped at the end of d: those rows are never stored)
            const int nkb = fg / 128, nob = d / 128, ob = o0 / 128;
            const float *sp = shared ? ssd : sd + (size_t)g * nob * nkb;
            tile_mma_dma_w8b(a_src, b_src, sp + (size_t)ob * nkb, sp + (size_t)(ob + 1 < nob ? ob + 1 : ob) * nkb,
                             fg, m, acc);
        } else {
            tile_mma_dma_w8(a_src, b_src, fg, m, acc);
        }
    } else {
        // block scales: B rows [0, 128) are output block o0/128, rows [128, 256)
        // the next one (clamped at the end of d: those rows are never stored)
        const float *sc_lo = nullptr, *sc_hi = nullptr;
        if (BLK) {
            const int nkb = fg / 128, nob = d / 128, ob = o0 / 128;
            const float *sp = shared ? ssd : sd + (size_t)g * nob * nkb;
            sc_lo = sp + (size_t)ob * nkb;
            sc_hi = sp + (size_t)(ob + 1 < nob ? ob + 1 : ob) * nkb;
        }
        tile_mma<FP8, false, kWN, BLK>(H, a_off, a_ok, b_base, b_off, 0, fg, fg, m, lds, acc, sc_lo, sc_hi);
    }

    const int lane = tid & 63, wave = tid >> 6, wm = wave >> 2, wn = wave & 3;
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
        // B tile row (= output column) of this lane's 4 values
        const int o = o0 + b_row_of(wn, ni) + (lane >> 4) * 4;
        if (o >= d) continue;  // d is a multiple of 64: o..o+3 all in range or all out
        float sc[4] = {1.f, 1.f, 1.f, 1.f};
        if (WM == kWFp8Row) {
#pragma unroll
            for (int q = 0; q < 4; ++q) sc[q] = shared ? ssd[o + q] : sd[obase + o + q];
        }
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const int r = wm * 64 + mi * 16 + (lane & 15);
            if (r < m)
                *reinterpret_cast<uint2 *>(Y + (size_t)(row0 + r) * d + o) =
                    make_uint2(pack_bf16x2(acc[mi][ni][0] * sc[0], acc[mi][ni][1] * sc[1]),
                               pack_bf16x2(acc[mi][ni][2] * sc[2], acc[mi][ni][3] * sc[3]));
        }
    }
}

// ---- persistent down product: bf16 H with bf16 weights (W8 false) or E4M3
// weights with per-channel scales (W8 true), d a multiple of 256 (whole
// column blocks).  The grid is one workgroup per CU; a workgroup
// walks the work items of its launch index in the XCD-aware order (its index
// modulo 8 fixes its XCD), and the DMA ring of tile_mma_dma (NB = 3 buffers
// of 48 KB) or tile_mma_dma_w8 (NB = 4 of 32 KB) runs on across item
// boundaries: the last NB stages of an item fetch the first NB of the next,
// so an item never waits for a workgroup launch or for its first operands.
// Stage s of the workgroup's sequence uses buffer s % NB, and at its barrier
// stage s + NB is fetched into that buffer.  An item's last stage waits for
// the next item's first stage, passes the barrier, finishes its MFMAs and
// stores its outputs before it fetches stage s + NB; the stores are then
// older than that fetch, and every later wait, which leaves only fetched
// stages in flight, also covers them (with NB = 4 the first wait of the next
// item also completes the stage fetched just before the stores).  Items
// shorter than NB stages are fine: the fetch cursor then runs more than one
// item ahead, and every wait counts only stages actually fetched.
#ifndef FGS_DOWN_PERSIST
#define FGS_DOWN_PERSIST 1
#endif
#ifndef FGS_DOWN_WIDE
#define FGS_DOWN_WIDE 1
#endif
#ifndef FGS_DOWN_F8P
#define FGS_DOWN_F8P 1
#endif
// Epilogue helpers of the persistent down kernels.  Inside their item loop a
// vector, flat or spilled memory access would make the compiler wait for
// every direct-to-LDS fetch in flight (its wait counts cannot see the
// fetches).  So the per-channel scales of an item are fetched into LDS with
// its first weight stage (one more DMA of wave 0, ahead of the stage's own)
// and read from there, and the output goes through a global (not flat)
// store whose address is a scalar base plus one lane offset.
typedef __attribute__((address_space(1))) uint8_t gbyte_t;
// four values of a lane, scaled and rounded to bf16, to blk (wave-uniform) + lane_off bytes
__device__ __forceinline__ void store_bf16x4(const uint16_t *blk, uint32_t lane_off, const f32x4_t &v,
                                             const float (&sc)[4]) {
    gbyte_t *b = (gbyte_t *)uniform_ptr(blk);
    *reinterpret_cast<__attribute__((address_space(1))) u32x2v_t *>(b + lane_off) =
        u32x2v_t{pack_bf16x2(v[0] * sc[0], v[1] * sc[1]), pack_bf16x2(v[2] * sc[2], v[3] * sc[3])};
}
// the 4 scales of a lane's columns 4 (lane/16) .. +3 of the 16-wide column fragment at
// column c of the item, from the item's scale slot in LDS (256 floats)
__device__ __forceinline__ void slot_scales(uint32_t slot, int c, int lane, float (&sc)[4]) {
    const uint4 v = lds_read16(slot + (uint32_t)(c + (lane >> 4) * 4) * 4u);
    sc[0] = __uint_as_float(v.x); sc[1] = __uint_as_float(v.y);
    sc[2] = __uint_as_float(v.z); sc[3] = __uint_as_float(v.w);
}

// Output staging of the 128 x 256 persistent down kernels: each wave owns 64
// contiguous columns of the item, and a 16 x 64 sub-tile of its results goes
// through a private 2 KB LDS region (16 rows of 128 bytes, 16-byte chunks
// XOR-swizzled by row) so that the global stores cover whole 128-byte row
// segments, 16 bytes per lane, instead of 32-byte pieces of 8 bytes per lane
// (prefill down 316 -> 283 us in a timing build with this store pattern).
constexpr int kOutStageB = 8 * 2048;
// a lane's four rounded values of column fragment ni (row lane % 16, columns
// 16 ni + 4 (lane / 16) .. +3) into the wave's region `ob`
__device__ __forceinline__ void stage_bf16x4(uint32_t ob, int ni, int lane, const f32x4_t &v, const float (&sc)[4]) {
    const int fr = lane & 15, fg = lane >> 4;
    const uint32_t a = ob + fr * 128 + ((((2 * ni + (fg >> 1)) ^ (fr & 7))) << 4) + ((fg & 1) << 3);
    *reinterpret_cast<__attribute__((address_space(3))) u32x2v_t *>((size_t)a) =
        u32x2v_t{pack_bf16x2(v[0] * sc[0], v[1] * sc[1]), pack_bf16x2(v[2] * sc[2], v[3] * sc[3])};
}
// rows 8 h + lane / 8 of the staged sub-tile, 16 bytes (chunk lane % 8) per lane, to
// blk (the sub-tile's first row and the wave's first column; wave-uniform) + lane_off.
// Non-temporal: Y is read once, by the combine (prefill down 283 -> 277 us).
__device__ __forceinline__ void store_staged(uint32_t ob, int h, int lane, const uint16_t *blk, uint32_t lane_off) {
    const int r = 8 * h + (lane >> 3), c = lane & 7;
    const uint4 v = lds_read16(ob + r * 128 + ((c ^ (r & 7)) << 4));
    gbyte_t *b = (gbyte_t *)uniform_ptr(blk);
    __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w},
                                reinterpret_cast<__attribute__((address_space(1))) u32x4_t *>(b + lane_off));
}

__device__ __forceinline__ int xcd_map(int slot, int B) {   // launch slot -> work item, as xcd_item
    const int c = slot % kXcds, s = slot / kXcds;
    return ((s / B) * kXcds + c) * B + s % B;
}

template <bool W8, bool BLK>
__global__ __launch_bounds__(kThreads) void down_gemm_persist_kernel(
    const uint16_t *__restrict__ H, int ldh, const uint8_t *__restrict__ wd, const float *__restrict__ sd,
    const uint8_t *__restrict__ wsd, const float *__restrict__ ssd, const int32_t *__restrict__ tiles,
    const int32_t *__restrict__ n_tiles, const int32_t *__restrict__ offsets, uint16_t *__restrict__ Y, int d, int E,
    int f, int fs) {
    static_assert(kAPer == 2 && kBPer == 4, "two activation DMAs per wave and stage");
    static_assert(W8 || !BLK, "block scales come with E4M3 weights");
    constexpr int NB = W8 ? 4 : 3;                          // ring buffers = fetch distance in stages
    constexpr int kStage = W8 ? kW8StageB : kDmaStageB;     // bytes per stage
    constexpr int kBDma = W8 ? 2 : kBPer;                   // weight DMAs per wave and stage
    constexpr int G = kAPer + kBDma;                        // DMAs per wave and stage
    constexpr int kWs = W8 ? 1 : 2;                         // bytes per weight
    // E4M3: 8 slots after the ring (the cursor runs at most NB items ahead) for an item's 256
    // column scales, or with block scales its two output blocks' K-block scales (2 f/128 values)
    constexpr int kSlots = W8 ? 8 : 0;
    constexpr int kOut = NB * kStage + kSlots * 1024;   // output staging, 2 KB per wave
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kOut + kOutStageB];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / kWN, wn = wave % kWN, fr = lane & 15, fg = lane >> 4;
    const int gx = d / kBN, B = kXcdTiles * gx;
    const int n_items = *n_tiles * gx;
    const int G_wg = gridDim.x;

    // fetch cursor: the item whose stages are fetched next, its next stage and buffer
    int fq = 0, fkt = 0, fnk = 0, fbuf = 0;
    bool fvalid = false;
    // DMA sources: a wave-uniform base (H, the item's weight matrix) and this
    // lane's 32-bit byte offset at K = 0 (H below 4 GiB: checked by the launcher)
    uint32_t a_off[kAPer], b_off[kBDma];
    const uint8_t *b_base = wd;
    const float *s_base = sd;   // the fetch item's scales (E4M3)
    int s_cnt = 0;              // block scales: values in the slot
    auto load_fetch_item = [&]() {
        const int item = xcd_map(blockIdx.x + fq * G_wg, B);
        fvalid = item < n_items;
        if (!fvalid) return;
        const int u = item / gx;
        const int g = tiles[2 * u], m0 = tiles[2 * u + 1];
        const bool shared = g == E;
        const int K = shared ? fs : f;
        const int o0 = (item % gx) * kBN;
        const int row0 = offsets[g] + m0, m = min(kBM, offsets[g + 1] - row0);
        b_base = shared ? wsd : wd + (size_t)g * d * K * kWs;
        if constexpr (BLK) {   // [E][d/128][K/128]: output blocks o0/128 and o0/128 + 1 are adjacent
            const int nob = d / 128, nkbk = K / 128;
            s_base = (shared ? ssd : sd + (size_t)g * nob * nkbk) + (size_t)(o0 / 128) * nkbk;
            s_cnt = 2 * nkbk;
        } else if constexpr (W8) {
            s_base = shared ? ssd + o0 : sd + (size_t)g * d + o0;
        }
        fnk = K / kBK;
#pragma unroll
        for (int j = 0; j < kAPer; ++j) {
            const int r = 8 * (wave * kAPer + j) + (lane >> 3);
            a_off[j] = ((uint32_t)(row0 + (r < m ? r : 0)) * (uint32_t)ldh + (((lane & 7) ^ (r & 7)) << 3)) * 2u;
        }
#pragma unroll
        for (int j = 0; j < kBDma; ++j) {
            if constexpr (W8) {   // 16 rows of 64 code bytes per DMA, chunk (lane % 4) ^ ((r / 4) % 4)
                const int r = 16 * (wave * 2 + j) + (lane >> 2);
                b_off[j] = (uint32_t)(o0 + r) * (uint32_t)K + ((((lane & 3) ^ (r >> 2)) & 3) << 4);
            } else {              // 8 rows of 128 bytes per DMA, chunk (lane % 8) ^ (r % 8)
                const int r = 8 * (wave * kBPer + j) + (lane >> 3);
                b_off[j] = ((uint32_t)(o0 + r) * (uint32_t)K + (((lane & 7) ^ (r & 7)) << 3)) * 2u;
            }
        }
    };
    int gf = 0;   // stages fetched so far
    auto fetch_next = [&]() {
        if (!fvalid) return;
        uint8_t *buf = smem + fbuf * kStage;
        if constexpr (BLK) {
            if (fkt == 0 && wave == 0)   // lanes past the count re-read value 0 (never used)
                dma4s(s_base, lane < s_cnt ? lane * 4 : 0, smem + NB * kStage + (fq & (kSlots - 1)) * 1024);
        } else if constexpr (W8) {
            if (fkt == 0 && wave == 0) dma16s(s_base, lane * 16, smem + NB * kStage + (fq & (kSlots - 1)) * 1024);
        }
        const uint16_t *sa = H + fkt * kBK;
        const uint8_t *sb = b_base + fkt * kBK * kWs;
#pragma unroll
        for (int j = 0; j < kAPer; ++j) dma16s(sa, a_off[j], buf + (wave * kAPer + j) * 1024);
#pragma unroll
        for (int j = 0; j < kBDma; ++j) dma16s(sb, b_off[j], buf + kBM * kDmaRowB + (wave * kBDma + j) * 1024);
        fbuf = fbuf == NB - 1 ? 0 : fbuf + 1;
        ++gf;
        if (++fkt == fnk) {
            fkt = 0;
            ++fq;
            load_fetch_item();
        }
    };
    // until at most `later` stages of this wave's DMAs are in flight
    auto wait_stages = [&](int later) {
        if (later >= 2) __builtin_amdgcn_s_waitcnt(FGS_VMCNT(2 * G));
        else if (later == 1) __builtin_amdgcn_s_waitcnt(FGS_VMCNT(G));
        else __builtin_amdgcn_s_waitcnt(FGS_VMCNT(0));
    };
    // this lane's fragment addresses in buffer 0 per 32-wide K half h: A row
    // wm*64 + lane%16, B row wn*64 + lane%16 (the wave's columns are 64
    // contiguous ones of the item), K chunk 4 h + lane/16 (the other rows of
    // the wave differ by multiples of 16 rows: constant offsets)
    const uint32_t s0 = (uint32_t)(uintptr_t)(lds_void_t *)smem;
    uint32_t la[2], lb[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int c = 4 * h + fg;
        la[h] = s0 + (wm * 64 + fr) * kDmaRowB + ((c ^ (fr & 7)) << 4);
        if constexpr (W8)
            lb[h] = s0 + kBM * kDmaRowB + (wn * 64 + fr) * kW8RowB + ((((c >> 1) ^ (fr >> 2)) & 3) << 4) + ((c & 1) << 3);
        else
            lb[h] = s0 + kBM * kDmaRowB + (wn * 64 + fr) * kDmaRowB + ((c ^ (fr & 7)) << 4);
    }
    constexpr int kBRowB = W8 ? kW8RowB : kDmaRowB;

    load_fetch_item();
    if (!fvalid) return;
#pragma unroll
    for (int i = 0; i < NB - 1; ++i) fetch_next();
    wait_stages(gf - 1);   // stage 0 landed
    lds_barrier();
    fetch_next();
    __builtin_amdgcn_sched_barrier(0);

    int gs = 0;   // stage being computed
    for (int q = 0;; ++q) {
        const int item = xcd_map(blockIdx.x + q * G_wg, B);
        if (item >= n_items) break;
        const int u = item / gx;
        const int g = tiles[2 * u], m0 = tiles[2 * u + 1];
        const bool shared = g == E;
        const int nk = (shared ? fs : f) / kBK;
        const int o0 = (item % gx) * kBN;
        const int row0 = offsets[g] + m0, m = min(kBM, offsets[g + 1] - row0);

        auto run = [&](auto live_c) {
            constexpr int LV = decltype(live_c)::value;
            constexpr int R = LV > 0 ? 4 + LV : 0;
            f32x4_t acc[4][4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            auto read_half = [&](uint32_t bo, int h, uint4 (&af)[4], uint4 (&bf)[4]) {
                if constexpr (LV > 0) {
                    const uint32_t pa = la[h] + bo, pb = lb[h] + bo;
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni) {
                        const uint32_t rb = ni * 16 * kBRowB;
                        if constexpr (W8) bf[ni] = e4m3x8_to_bf16x8(lds_read8(pb + rb));
                        else bf[ni] = lds_read16(pb + rb);
                    }
#pragma unroll
                    for (int mi = 0; mi < LV; ++mi) af[mi] = lds_read16(pa + mi * 16 * kDmaRowB);
                }
            };
            auto mma_half = [&](const uint4 (&af)[4], const uint4 (&bf)[4]) {
#pragma unroll
                for (int mi = 0; mi < LV; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = mfma_bf16(bf[ni], af[mi], acc[mi][ni]);
            };
            // this wave's DMAs of stage gs + 1 landed; the later fetched stages stay in flight
            auto wait_next = [&]() { wait_stages(gf - gs - 2); };
            if constexpr (BLK) {
                // 128 x 128 block scales: the products of every 64-wide stage (its two
                // K halves, on the same double-buffered fragment schedule as below) go
                // into fresh accumulators that are folded into the sum times the scale
                // of the stage's K block (kt / 2) and output block (waves 0-1: the
                // item's first 128 columns, 2-3: the next 128), as tile_mma_dma_w8b does
                const uint32_t slot = s0 + NB * kStage + (q & (kSlots - 1)) * 1024;
                const int nkbk = nk / 2;
                f32x4_t pr[4][4];
                auto mma_into = [&](const uint4 (&af)[4], const uint4 (&bf)[4], bool first) {
#pragma unroll
                    for (int mi = 0; mi < LV; ++mi)
#pragma unroll
                        for (int ni = 0; ni < 4; ++ni)
                            pr[mi][ni] = mfma_bf16(bf[ni], af[mi], first ? f32x4_t{0.f, 0.f, 0.f, 0.f} : pr[mi][ni]);
                };
                auto fold = [&](int kt) {
                    const float c = lds_read_f32(slot + (uint32_t)((wn < 2 ? 0 : nkbk) + (kt >> 1)) * 4u);
#pragma unroll
                    for (int mi = 0; mi < LV; ++mi)
#pragma unroll
                        for (int ni = 0; ni < 4; ++ni) {
#pragma unroll
                            for (int qq = 0; qq < 4; ++qq) acc[mi][ni][qq] = fmaf(pr[mi][ni][qq], c, acc[mi][ni][qq]);
                        }
                };
                uint4 fa0[4], fb0[4], fa1[4], fb1[4];
                int cb = gs % NB;
                read_half(cb * kStage, 0, fa0, fb0);
#pragma nounroll
                for (int kt = 0; kt + 1 < nk; ++kt) {
                    const int nb = cb == NB - 1 ? 0 : cb + 1;
                    __builtin_amdgcn_sched_barrier(0);
                    read_half(cb * kStage, 1, fa1, fb1);
                    mma_into(fa0, fb0, true);
                    interleave_mfma_reads<R, 4 * LV>();
                    __builtin_amdgcn_sched_barrier(0);
                    wait_next();
                    lds_barrier();
                    fetch_next();
                    __builtin_amdgcn_sched_barrier(0);
                    read_half(nb * kStage, 0, fa0, fb0);
                    mma_into(fa1, fb1, false);
                    interleave_mfma_reads<R, 4 * LV>();
                    __builtin_amdgcn_sched_barrier(0);
                    fold(kt);
                    __builtin_amdgcn_sched_barrier(0);
                    ++gs;
                    cb = nb;
                }
                __builtin_amdgcn_sched_barrier(0);
                read_half(cb * kStage, 1, fa1, fb1);
                mma_into(fa0, fb0, true);
                __builtin_amdgcn_sched_barrier(0);
                const bool more = gf > gs + 1;
                if (more) {
                    wait_next();
                    lds_barrier();
                }
                __builtin_amdgcn_sched_barrier(0);
                mma_into(fa1, fb1, false);
                fold(nk - 1);
                __builtin_amdgcn_sched_barrier(0);
                const uint32_t ob = s0 + kOut + wave * 2048;
                const uint32_t lane_off = ((uint32_t)(lane >> 3) * (uint32_t)d + (uint32_t)(lane & 7) * 8u) * 2u;
                const float one[4] = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
                for (int mi = 0; mi < LV; ++mi) {
                    const int rb = wm * 64 + mi * 16;
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni) stage_bf16x4(ob, ni, lane, acc[mi][ni], one);
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        if (rb + 8 * h + (lane >> 3) < m)
                            store_staged(ob, h, lane, Y + (size_t)(row0 + rb + 8 * h) * d + o0 + wn * 64, lane_off);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (more) fetch_next();
                ++gs;
                return;
            }
            uint4 fa0[4], fb0[4], fa1[4], fb1[4];
            int cb = gs % NB;
            read_half(cb * kStage, 0, fa0, fb0);
            // every stage but the item's last: stage gs + NB goes into buffer cb
#pragma nounroll
            for (int kt = 0; kt + 1 < nk; ++kt) {
                const int nb = cb == NB - 1 ? 0 : cb + 1;
                __builtin_amdgcn_sched_barrier(0);
                read_half(cb * kStage, 1, fa1, fb1);
                mma_half(fa0, fb0);
                interleave_mfma_reads<R, 4 * LV>();
                __builtin_amdgcn_sched_barrier(0);
                wait_next();
                lds_barrier();
                fetch_next();
                __builtin_amdgcn_sched_barrier(0);
                read_half(nb * kStage, 0, fa0, fb0);
                mma_half(fa1, fb1);
                interleave_mfma_reads<R, 4 * LV>();
                __builtin_amdgcn_sched_barrier(0);
                ++gs;
                cb = nb;
            }
            // the last stage: wait for the next item's first stage (if any), finish,
            // store, then fetch stage gs + NB
            __builtin_amdgcn_sched_barrier(0);
            read_half(cb * kStage, 1, fa1, fb1);
            mma_half(fa0, fb0);
            __builtin_amdgcn_sched_barrier(0);
            const bool more = gf > gs + 1;
            if (more) {
                wait_next();
                lds_barrier();
            }
            __builtin_amdgcn_sched_barrier(0);
            mma_half(fa1, fb1);
            __builtin_amdgcn_sched_barrier(0);
            // lane: row wm*64 + mi*16 + lane%16, columns o0 + wn*64 + 16 ni + 4 (lane/16) .. +3,
            // staged per sub-tile row and stored 16 bytes per lane
            const uint32_t ob = s0 + kOut + wave * 2048;
            const uint32_t lane_off = ((uint32_t)(lane >> 3) * (uint32_t)d + (uint32_t)(lane & 7) * 8u) * 2u;
            float sc[4][4];
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) {
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) sc[ni][qq] = 1.f;
                if constexpr (W8) slot_scales(s0 + NB * kStage + (q & (kSlots - 1)) * 1024, wn * 64 + ni * 16, lane, sc[ni]);
            }
#pragma unroll
            for (int mi = 0; mi < LV; ++mi) {
                const int rb = wm * 64 + mi * 16;
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) stage_bf16x4(ob, ni, lane, acc[mi][ni], sc[ni]);
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    if (rb + 8 * h + (lane >> 3) < m)
                        store_staged(ob, h, lane, Y + (size_t)(row0 + rb + 8 * h) * d + o0 + wn * 64, lane_off);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (more) fetch_next();
            ++gs;
        };
        const int live = min(4, max(0, (m - wm * 64 + 15) / 16));
        switch (live) {
            case 4: run(Live<4>{}); break;
            case 3: run(Live<3>{}); break;
            case 2: run(Live<2>{}); break;
            case 1: run(Live<1>{}); break;
            default: run(Live<0>{}); break;
        }
    }
}

// ---- persistent wide down product: 256 x 256 items (the wide gate/up's
// 256-row tile list), 16 waves of 64 x 64, bf16 H with bf16 weights (W8
// false) or E4M3 weights with per-channel scales (W8 true), d a multiple of
// 256.  One workgroup per CU walks its XCD's items as down_gemm_persist_kernel
// does, with the wide tile's two rings: NA activation buffers and NB weight
// buffers of one stage each (bf16: 2 and 3 of 32 KB; E4M3: 3 of 32 KB and 3
// of 16 KB).  At the barrier that ends stage s the activations of stage s + NA
// and the weights of stage s + NB are fetched into the buffers stage s used,
// by two cursors that cross item boundaries on their own.  The wave waits
// before that barrier leave only the newest fetch group in flight; an item's
// stores are issued after the barrier of its last stage and before that
// stage's fetches, so the next wait covers them and no prefetch is waited
// for early.  A quarter fewer operand bytes per flop than the 128 x 256 item
// and one weight slice per expert and column block where an expert has at
// most 256 rows.
template <bool W8>
__global__ __launch_bounds__(1024) void down_gemm_wide_persist_kernel(
    const uint16_t *__restrict__ H, int ldh, const uint8_t *__restrict__ wd, const float *__restrict__ sd,
    const uint8_t *__restrict__ wsd, const float *__restrict__ ssd, const int32_t *__restrict__ tiles,
    const int32_t *__restrict__ n_tiles, const int32_t *__restrict__ offsets, uint16_t *__restrict__ Y, int d, int E,
    int f, int fs) {
    using WG = Wide<4>;
    static_assert(WG::kWaves == 16 && WG::kDma == 2, "16 waves, two 1 KB DMAs per wave and operand stage");
    constexpr int kAPerW = WG::kDma;               // 256 rows x 128 bytes = 32 DMAs of 1 KB
    constexpr int kBPerW = W8 ? 1 : WG::kDma;      // 256 rows x 128 (bf16) or 64 (E4M3) bytes
    constexpr int kWs = W8 ? 1 : 2;                // bytes per weight
    constexpr int kBRowB = W8 ? kW8RowB : kDmaRowB;
    constexpr int NA = W8 ? 3 : 2, NB = 3;
    constexpr int kABuf = kWideBufB, kBBuf = W8 ? kWideW8BufB : kWideBufB;
    constexpr int kBOff = 0, kAOff = NB * kBBuf;   // weight ring first, then the activation ring
    // E4M3: 4 slots of 256 column scales after the rings (the weight cursor runs at most NB items ahead)
    constexpr int kSOff = kAOff + NA * kABuf, kSlotB = W8 ? 4 * 1024 : 0;
    static_assert(NB * kBBuf + NA * kABuf + kSlotB <= 160 * 1024, "the rings must fit one CU's LDS");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[NB * kBBuf + NA * kABuf + kSlotB];
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = w / kWN, wn = w % kWN, fr = lane & 15, fg = lane >> 4;
    const int gx = d / kBN, B = kXcdTiles * gx;
    const int n_items = *n_tiles * gx;
    const int G_wg = gridDim.x;

    // activation cursor: next stage to fetch (item slot qa, stage kta of nka)
    int qa = 0, kta = 0, nka = 0, fab = 0, gfa = 0;
    bool va = false;
    uint32_t a_off[kAPerW];
    // rows past the group end read row 0 of the tile (never stored)
    auto set_a_off = [&](int row0, int m) {
#pragma unroll
        for (int j = 0; j < kAPerW; ++j) {
            const int r = 8 * (w * kAPerW + j) + (lane >> 3);
            a_off[j] = ((uint32_t)(row0 + (r < m ? r : 0)) * (uint32_t)ldh + (((lane & 7) ^ (r & 7)) << 3)) * 2u;
        }
    };
    auto load_a = [&]() {
        const int item = xcd_map(blockIdx.x + qa * G_wg, B);
        va = item < n_items;
        if (!va) return;
        const int u = item / gx;
        const int g = tiles[2 * u], m0 = tiles[2 * u + 1];
        nka = (g == E ? fs : f) / kBK;
        const int row0 = offsets[g] + m0;
        set_a_off(row0, min(kBMW, offsets[g + 1] - row0));
    };
    // A DMAs of the stage `kt` into ring buffer `buf`
    auto dma_a = [&](int kt, int buf) {
        const uint16_t *sa = H + kt * kBK;
#pragma unroll
        for (int j = 0; j < kAPerW; ++j) dma16s(sa, a_off[j], smem + kAOff + buf * kABuf + (w * kAPerW + j) * 1024);
    };
    auto fetch_a = [&]() {   // bf16 only
        if (!va) return;
        dma_a(kta, fab);
        fab = fab == NA - 1 ? 0 : fab + 1;
        ++gfa;
        if (++kta == nka) { kta = 0; ++qa; load_a(); }
    };
    // weight cursor
    int qb = 0, ktb = 0, nkb = 0, fbb = 0, gfb = 0;
    bool vb = false;
    uint32_t b_off[kBPerW];
    const uint8_t *b_base = wd;
    const float *s_base = sd;   // the weight cursor item's 256 column scales (E4M3)
    auto load_b = [&]() {
        const int item = xcd_map(blockIdx.x + qb * G_wg, B);
        vb = item < n_items;
        if (!vb) return;
        const int u = item / gx;
        const int g = tiles[2 * u];
        const bool shared = g == E;
        const int K = shared ? fs : f;
        nkb = K / kBK;
        const int o0 = (item % gx) * kBN;
        b_base = shared ? wsd : wd + (size_t)g * d * K * kWs;
        if constexpr (W8) {   // this cursor fetches the activations too
            const int row0 = offsets[g] + tiles[2 * u + 1];
            set_a_off(row0, min(kBMW, offsets[g + 1] - row0));
        }
        if constexpr (W8) s_base = shared ? ssd + o0 : sd + (size_t)g * d + o0;
#pragma unroll
        for (int j = 0; j < kBPerW; ++j) {
            if constexpr (W8) {   // 16 rows of 64 code bytes per DMA, chunk (lane % 4) ^ ((r / 4) % 4)
                const int r = 16 * w + (lane >> 2);
                b_off[j] = (uint32_t)(o0 + r) * (uint32_t)K + ((((lane & 3) ^ (r >> 2)) & 3) << 4);
            } else {              // 8 rows of 128 bytes per DMA, chunk (lane % 8) ^ (r % 8)
                const int r = 8 * (w * kBPerW + j) + (lane >> 3);
                b_off[j] = ((uint32_t)(o0 + r) * (uint32_t)K + (((lane & 7) ^ (r & 7)) << 3)) * 2u;
            }
        }
    };
    auto fetch_b = [&]() {
        if (!vb) return;
        const uint8_t *sb = b_base + ktb * kBK * kWs;
        if constexpr (W8) dma_a(ktb, fbb);
#pragma unroll
        for (int j = 0; j < kBPerW; ++j) dma16s(sb, b_off[j], smem + kBOff + fbb * kBBuf + (w * kBPerW + j) * 1024);
        fbb = fbb == NB - 1 ? 0 : fbb + 1;
        ++gfb;
        if (++ktb == nkb) { ktb = 0; ++qb; load_b(); }
    };
    // one fetch group: an item's column scales when the weight cursor starts it
    // (first, so a wait that leaves the group's operand DMAs in flight covers it),
    // then the activation and the weight stage
    auto fetch_group = [&](bool a) {
        if constexpr (W8)
            if (vb && ktb == 0 && w == 0) dma16s(s_base, lane * 16, smem + kSOff + (qb & 3) * 1024);
        if (!W8 && a) fetch_a();
        fetch_b();
    };
    // fetched stages (both operands): the activation cursor trails with bf16
    auto fetched = [&]() { return W8 ? gfb : gfa; };

    // this lane's fragment addresses in buffer 0 per 32-wide K half h: activation
    // row wm*64 + lane%16, weight row wn*64 + lane%16 (the wave's 64 columns are
    // contiguous), K chunk 4 h + lane/16
    const uint32_t s0 = (uint32_t)(uintptr_t)(lds_void_t *)smem;
    uint32_t la[2], lb[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int c = 4 * h + fg;
        la[h] = s0 + kAOff + (wm * 64 + fr) * kDmaRowB + ((c ^ (fr & 7)) << 4);
        if constexpr (W8)
            lb[h] = s0 + kBOff + (wn * 64 + fr) * kW8RowB + ((((c >> 1) ^ (fr >> 2)) & 3) << 4) + ((c & 1) << 3);
        else
            lb[h] = s0 + kBOff + (wn * 64 + fr) * kDmaRowB + ((c ^ (fr & 7)) << 4);
    }

    if constexpr (!W8) load_a();
    load_b();
    if (!vb) return;
    // prologue, in the steady state's issue order: activations of stages 0 .. NA-1,
    // weights of stages 0 .. NB-1; all of it lands before the first stage
#pragma unroll
    for (int i = 0; i < NB; ++i) fetch_group(i < NA);
    __builtin_amdgcn_s_waitcnt(FGS_VMCNT(0));
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);

    int gs = 0;   // stage being computed
    for (int q = 0;; ++q) {
        const int item = xcd_map(blockIdx.x + q * G_wg, B);
        if (item >= n_items) break;
        const int u = item / gx;
        const int g = tiles[2 * u], m0 = tiles[2 * u + 1];
        const bool shared = g == E;
        const int nk = (shared ? fs : f) / kBK;
        const int o0 = (item % gx) * kBN;
        const int row0 = offsets[g] + m0, m = min(kBMW, offsets[g + 1] - row0);

        auto run = [&](auto live_c) {
            constexpr int LV = decltype(live_c)::value;
            f32x4_t acc[4][4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            int ca = gs % NA, cbw = gs % NB;
            // the products of one stage from activation buffer ca and weight buffer cbw
            auto compute = [&]() {
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (LV > 0) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const uint32_t pa = la[h] + ca * kABuf, pb = lb[h] + cbw * kBBuf;
                        uint4 bf[4];
#pragma unroll
                        for (int ni = 0; ni < 4; ++ni) {
                            const uint32_t rb = ni * 16 * kBRowB;
                            if constexpr (W8) bf[ni] = e4m3x8_to_bf16x8(lds_read8(pb + rb));
                            else bf[ni] = lds_read16(pb + rb);
                        }
                        if constexpr (W8) {   // one activation fragment at a time: 128 registers a wave
#pragma unroll
                            for (int mi = 0; mi < LV; ++mi) {
                                const uint4 a = lds_read16(pa + mi * 16 * kDmaRowB);
#pragma unroll
                                for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = mfma_bf16(bf[ni], a, acc[mi][ni]);
                            }
                        } else {              // the next fragment requested before this one's MFMAs
                            uint4 a = lds_read16(pa);
#pragma unroll
                            for (int mi = 0; mi < LV; ++mi) {
                                const uint4 an = mi + 1 < LV ? lds_read16(pa + (mi + 1) * 16 * kDmaRowB) : a;
#pragma unroll
                                for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = mfma_bf16(bf[ni], a, acc[mi][ni]);
                                a = an;
                            }
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            };
            // this wave's DMAs of stage gs + 1 landed; only the newest fetch group
            // (weights of gs + 2 with bf16, both operands of gs + 2 with E4M3) may remain
            auto wait_next = [&]() {
                if constexpr (W8) {
                    if (gfb >= gs + 3) __builtin_amdgcn_s_waitcnt(FGS_VMCNT(kAPerW + kBPerW));
                    else __builtin_amdgcn_s_waitcnt(FGS_VMCNT(0));
                } else {
                    if (gfb >= gs + 3) __builtin_amdgcn_s_waitcnt(FGS_VMCNT(kBPerW));
                    else __builtin_amdgcn_s_waitcnt(FGS_VMCNT(0));
                }
            };
            auto advance = [&]() {
                ++gs;
                ca = ca == NA - 1 ? 0 : ca + 1;
                cbw = cbw == NB - 1 ? 0 : cbw + 1;
            };
            // every stage but the item's last (stage gs + 1 is this item's)
#pragma nounroll
            for (int kt = 0; kt + 1 < nk; ++kt) {
                compute();
                wait_next();
                lds_barrier();
                fetch_group(true);   // activations of stage gs + NA into buffer ca, weights of gs + NB into cbw
                __builtin_amdgcn_sched_barrier(0);
                advance();
            }
            // the last stage: products, then (if a later stage exists) its wait and
            // barrier, the stores, and only then the fetches of this barrier
            compute();
            const bool more = fetched() > gs + 1;
            if (more) wait_next();
            // every wave is past its reads of buffers ca and cbw (refilled, or here
            // lending this wave's own 2 KB of activation buffer ca to the output staging)
            lds_barrier();
            __builtin_amdgcn_sched_barrier(0);
            // lane: row wm*64 + mi*16 + lane%16, columns o0 + wn*64 + 16 ni + 4 (lane/16) .. +3,
            // staged per sub-tile row and stored 16 bytes per lane (the lane index recomputed
            // here rather than kept live through the K loop)
            const int ln = (int)__lane_id();
            const uint32_t ob = s0 + kAOff + ca * kABuf + w * kAPerW * 1024;
            const uint32_t lane_off = ((uint32_t)(ln >> 3) * (uint32_t)d + (uint32_t)(ln & 7) * 8u) * 2u;
#pragma unroll
            for (int mi = 0; mi < LV; ++mi) {
                const int rb = wm * 64 + mi * 16;
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) {
                    float sc[4] = {1.f, 1.f, 1.f, 1.f};
                    if constexpr (W8) slot_scales(s0 + kSOff + (q & 3) * 1024, wn * 64 + ni * 16, ln, sc);
                    stage_bf16x4(ob, ni, ln, acc[mi][ni], sc);
                }
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    if (rb + 8 * h + (ln >> 3) < m)
                        store_staged(ob, h, ln, Y + (size_t)(row0 + rb + 8 * h) * d + o0 + wn * 64, lane_off);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (more) fetch_group(true);
            __builtin_amdgcn_sched_barrier(0);
            advance();
        };
        const int live = min(4, max(0, (m - wm * 64 + 15) / 16));
        switch (live) {
            case 4: run(Live<4>{}); break;
            case 3: run(Live<3>{}); break;
            case 2: run(Live<2>{}); break;
            case 1: run(Live<1>{}); break;
            default: run(Live<0>{}); break;
        }
    }
}

// ---------------------------------------------------------------- FP8 x FP8
// 1 x 128 activation quantisation ("Inside Kolibri 1", section "The FP8 path
// is explicitly mixed precision"): A holds E4M3 codes of activations with one
// FP32 scale per row and 128 columns, B the E4M3 weights.  A stage is one
// 128-wide K block, i.e. 128 bytes per tile row, the same bytes as a bf16
// stage, so the loader and the LDS layout (rows of 128 bytes padded to 160)
// are those of the bf16 tile.  Each 16 x 16 sub-tile takes one
// v_mfma_f32_16x16x128_f8f6f4 per stage (a lane supplies 32 consecutive K
// bytes of its row: half the LDS bytes per flop of bf16), and the stage's
// products are added into the running sum times (activation scale of the row)
// x (weight scale of the column block).

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4_t mfma_f8(const uint4 &a0, const uint4 &a1, const uint4 &b0, const uint4 &b1) {
    const i32x8_t a = {(int32_t)a0.x, (int32_t)a0.y, (int32_t)a0.z, (int32_t)a0.w,
                       (int32_t)a1.x, (int32_t)a1.y, (int32_t)a1.z, (int32_t)a1.w};
    const i32x8_t b = {(int32_t)b0.x, (int32_t)b0.y, (int32_t)b0.z, (int32_t)b0.w,
                       (int32_t)b1.x, (int32_t)b1.y, (int32_t)b1.z, (int32_t)b1.w};
    // formats 0/0: both operands E4M3; scale operands 0 select the unscaled form
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
}

constexpr int kLdsRowB = 2 * kLdsStride;   // 160-byte LDS rows

struct StageF8 {
    uint4 a[kAPer];
    uint4 b[kBPer];
};

// sa[mi]: this lane's activation-scale row for sub-tile mi (row wm*64 + mi*16
// + lane%16), indexed by K block.  BLKW: column fragments ni < 2 use weight
// scale sw_lo[kb], ni >= 2 sw_hi[kb]; otherwise the weight scale is applied by
// the caller (per output channel).
// b_base[j] is the same for every lane (one expert's matrix); b_off[j] < 2^32.
template <bool BLKW>
__device__ __forceinline__ void tile_mma_f8(const uint8_t *a_base, const size_t (&a_off)[kAPer],
                                            const bool (&a_ok)[kAPer], const uint8_t *const (&b_base)[kBPer],
                                            const uint32_t (&b_off)[kBPer], int K, const float *sa_base,
                                            const uint32_t (&sa_off)[4], const float *sw_lo, const float *sw_hi,
                                            int m, uint8_t *lds, f32x4_t (&acc)[4][4]) {
    constexpr int kRowStep = kThreads / 8;
    constexpr int kAB = kBM * kLdsRowB, kStageB = (kBM + kBN) * kLdsRowB;
    // the wave index is uniform: in a scalar register, the live-row tests are scalar branches
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / kWN, wn = wave % kWN;
    const int chunk = (tid & 7) * 16;
    const int r0 = tid >> 3;
    uint8_t *const As[2] = {lds, lds + kStageB};
    uint8_t *const Bs[2] = {lds + kAB, lds + kStageB + kAB};
    const int fr = lane & 15, fk = (lane >> 4) * 32;
    const int live = min(4, max(0, (m - wm * 64 + 15) / 16));

    auto fetch = [&](StageF8 &st, int k0) {
#pragma unroll
        for (int j = 0; j < kAPer; ++j) st.a[j] = *reinterpret_cast<const uint4 *>(a_base + a_off[j] + k0 + chunk);
#pragma unroll
        for (int j = 0; j < kBPer; ++j) st.b[j] = *reinterpret_cast<const uint4 *>(b_base[j] + b_off[j] + k0 + chunk);
    };
    auto stash = [&](const StageF8 &st, int buf) {
#pragma unroll
        for (int j = 0; j < kAPer; ++j)
            *reinterpret_cast<uint4 *>(As[buf] + (r0 + kRowStep * j) * kLdsRowB + chunk) =
                a_ok[j] ? st.a[j] : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < kBPer; ++j)
            *reinterpret_cast<uint4 *>(Bs[buf] + (r0 + kRowStep * j) * kLdsRowB + chunk) = st.b[j];
    };
    // scales of K block kb: the activation scale of each sub-tile row of this
    // lane, and the weight scales of the two column halves (wave-uniform)
    struct Sc { float a[4], wlo, whi; };
    auto scales = [&](int kb, Sc &sc) {
        sc.wlo = 1.f;
        sc.whi = 1.f;
        if (BLKW) { sc.wlo = sw_lo[kb]; sc.whi = sw_hi[kb]; }
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) sc.a[mi] = sa_base[sa_off[mi] + kb];
    };
    // The products of sub-tile row mi are folded while those of mi+1 are in
    // the matrix core, so at most two rows of products (32 registers) live.
    auto compute = [&](int buf, const Sc &sc) {
        uint4 bf[4][2];
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
            const uint8_t *bp = Bs[buf] + (b_row_of(wn, ni) + fr) * kLdsRowB + fk;
            bf[ni][0] = *reinterpret_cast<const uint4 *>(bp);
            bf[ni][1] = *reinterpret_cast<const uint4 *>(bp + 16);
        }
        auto products = [&](int mi, f32x4_t (&pr)[4]) {
            const uint8_t *ap = As[buf] + (wm * 64 + mi * 16 + fr) * kLdsRowB + fk;
            const uint4 a0 = *reinterpret_cast<const uint4 *>(ap), a1 = *reinterpret_cast<const uint4 *>(ap + 16);
            // B fragment first: transposed result, a lane holds 4 consecutive columns of one row
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) pr[ni] = mfma_f8(bf[ni][0], bf[ni][1], a0, a1);
        };
        auto fold = [&](int mi, const f32x4_t (&pr)[4]) {
            const float clo = sc.a[mi] * sc.wlo, chi = sc.a[mi] * sc.whi;
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) {
                const float c = ni < 2 ? clo : chi;
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[mi][ni][q] = fmaf(pr[ni][q], c, acc[mi][ni][q]);
            }
        };
        f32x4_t p0[4], p1[4];
        if (live > 0) products(0, p0);
        if (live > 1) products(1, p1);
        if (live > 0) fold(0, p0);
        if (live > 2) products(2, p0);
        if (live > 1) fold(1, p1);
        if (live > 3) products(3, p1);
        if (live > 2) fold(2, p0);
        if (live > 3) fold(3, p1);
    };

    const int nk = K / 128;
    StageF8 s0, s1;
    Sc c0, c1;
    fetch(s0, 0);
    if (nk > 1) fetch(s1, 128);
    stash(s0, 0);
    lds_barrier();
    int kt = 0;
    for (; kt + 3 < nk; kt += 2) {
        scales(kt, c0);
        fetch(s0, (kt + 2) * 128);
        __builtin_amdgcn_sched_barrier(0);
        compute(0, c0);
        __builtin_amdgcn_sched_barrier(0);
        stash(s1, 1);
        lds_barrier();
        scales(kt + 1, c1);
        fetch(s1, (kt + 3) * 128);
        __builtin_amdgcn_sched_barrier(0);
        compute(1, c1);
        __builtin_amdgcn_sched_barrier(0);
        stash(s0, 0);
        lds_barrier();
    }
    // tail: 1, 2 or 3 stages left (stage kt in LDS buffer 0, stage kt+1 in s1)
    const int left = nk - kt;
    if (left == 3) fetch(s0, (kt + 2) * 128);
    scales(kt, c0);
    compute(0, c0);
    if (left >= 2) {
        stash(s1, 1);
        lds_barrier();
        scales(kt + 1, c1);
        compute(1, c1);
        if (left == 3) {
            stash(s0, 0);
            lds_barrier();
            scales(kt + 2, c0);
            compute(0, c0);
        }
    }
}

// ---- FP8 x FP8 with both operand tiles fetched straight into LDS: the
// bf16 direct-to-LDS tile's three stages and swizzled 128-byte rows, one
// 128-wide K block per stage.  A lane's 32 K bytes are chunks 2 (lane / 16)
// and 2 (lane / 16) + 1 of its row, two 16-byte reads.  The activation scales
// of the tile's rows and the weight block scales of the whole K range go to
// LDS once, before the loop (loads the compiler tracks must not follow the
// DMAs it cannot see: its waits for them would also wait for every DMA), so K
// is limited to kF8DmaMaxKb blocks.
static_assert(3 * kDmaStageB + kF8DmaMaxKb * (kBM + 2) * 4 + kBM * 4 * 4 <= 160 * 1024,
              "stages, scales and the epilogue's row maxima must fit one CU's LDS");

// sa_row[j]: activation scales (one per K block) of this lane's DMA row j
// (clamped to the group); BLKW: sw_lo / sw_hi the weight block scales of the
// two column halves.  Same accumulation order as tile_mma_f8.
template <bool BLKW>
__device__ __forceinline__ void tile_mma_dma_f8(const uint8_t *const (&a_src)[kAPer],
                                                const uint8_t *const (&b_src)[kBPer],
                                                const float *const (&sa_row)[kAPer], const float *sw_lo,
                                                const float *sw_hi, int K, int m, f32x4_t (&acc)[4][4]) {
    static_assert(kAPer == 2 && kBPer == 4, "six DMAs per wave and stage");
    __shared__ __attribute__((aligned(16))) uint8_t L0[kDmaStageB];
    __shared__ __attribute__((aligned(16))) uint8_t L1[kDmaStageB];
    __shared__ __attribute__((aligned(16))) uint8_t L2[kDmaStageB];
    __shared__ float sa_l[kF8DmaMaxKb][kBM];
    __shared__ float sw_l[2][kF8DmaMaxKb];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / kWN, wn = wave % kWN;
    const int fr = lane & 15, fg = lane >> 4;
    const int nk = K / 128;
    auto fetch = [&](int kt, uint8_t *buf) {
        const int k0 = kt * 128;
#pragma unroll
        for (int j = 0; j < kAPer; ++j) dma16(a_src[j] + k0, buf + (wave * kAPer + j) * 1024);
#pragma unroll
        for (int j = 0; j < kBPer; ++j) dma16(b_src[j] + k0, buf + kBM * kDmaRowB + (wave * kBPer + j) * 1024);
    };
    auto frag = [&](const uint8_t *base, int r, int c) {
        return *reinterpret_cast<const uint4 *>(base + r * kDmaRowB + ((c ^ (r & 7)) << 4));
    };
    auto wait_own = [&](int kt) {
        if (kt + 1 < nk) __builtin_amdgcn_s_waitcnt(FGS_VMCNT(kAPer + kBPer));
        else __builtin_amdgcn_s_waitcnt(FGS_VMCNT(0));
    };

    fetch(0, L0);
    if (nk > 1) fetch(1, L1);
    // scales: the 8 lanes that fetch a row split its K blocks (block 8 q + lane % 8)
    const int pos = lane & 7;
    float sv[kAPer][3];
#pragma unroll
    for (int j = 0; j < kAPer; ++j)
#pragma unroll
        for (int q = 0; q < 3; ++q) sv[j][q] = pos + 8 * q < nk ? sa_row[j][pos + 8 * q] : 0.f;
    const float wv = (BLKW && tid < 2 * nk) ? (tid < nk ? sw_lo[tid] : sw_hi[tid - nk]) : 0.f;
    wait_own(0);
#pragma unroll
    for (int j = 0; j < kAPer; ++j) {
        const int r = 8 * (wave * kAPer + j) + (lane >> 3);
#pragma unroll
        for (int q = 0; q < 3; ++q)
            if (pos + 8 * q < nk) sa_l[pos + 8 * q][r] = sv[j][q];
    }
    if (BLKW && tid < 2 * nk) sw_l[tid / nk][tid % nk] = wv;
    lds_barrier();
    if (nk > 2) fetch(2, L2);
    __builtin_amdgcn_sched_barrier(0);

    const int live = min(4, max(0, (m - wm * 64 + 15) / 16));
    auto compute = [&](int kt, const uint8_t *cur) {
        uint4 bf[4][2];
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
            const int r = b_row_of(wn, ni) + fr;
            bf[ni][0] = frag(cur + kBM * kDmaRowB, r, 2 * fg);
            bf[ni][1] = frag(cur + kBM * kDmaRowB, r, 2 * fg + 1);
        }
        const float wlo = BLKW ? sw_l[0][kt] : 1.f, whi = BLKW ? sw_l[1][kt] : 1.f;
        auto products = [&](int mi, f32x4_t (&pr)[4]) {
            const int r = wm * 64 + mi * 16 + fr;
            const uint4 a0 = frag(cur, r, 2 * fg), a1 = frag(cur, r, 2 * fg + 1);
            // B fragment first: transposed result, a lane holds 4 consecutive columns of one row
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) pr[ni] = mfma_f8(bf[ni][0], bf[ni][1], a0, a1);
        };
        auto fold = [&](int mi, const f32x4_t (&pr)[4]) {
            const float sa = sa_l[kt][wm * 64 + mi * 16 + fr];
            const float clo = sa * wlo, chi = sa * whi;
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) {
                const float c = ni < 2 ? clo : chi;
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[mi][ni][q] = fmaf(pr[ni][q], c, acc[mi][ni][q]);
            }
        };
        f32x4_t p0[4], p1[4];
        if (live > 0) products(0, p0);
        if (live > 1) products(1, p1);
        if (live > 0) fold(0, p0);
        if (live > 2) products(2, p0);
        if (live > 1) fold(1, p1);
        if (live > 3) products(3, p1);
        if (live > 2) fold(2, p0);
        if (live > 3) fold(3, p1);
    };
    // stage kt: wait for own stage-kt DMAs, barrier, fetch stage kt + 2 into
    // the buffer of stage kt - 1, multiply
    auto step = [&](int kt, const uint8_t *cur, uint8_t *next2) {
        wait_own(kt);
        lds_barrier();
        if (kt + 2 < nk) fetch(kt + 2, next2);
        __builtin_amdgcn_sched_barrier(0);
        compute(kt, cur);
        __builtin_amdgcn_sched_barrier(0);
    };
    int kt = 0;
    for (; kt + 3 <= nk; kt += 3) {   // stage s uses buffer s % 3
        step(kt, L0, L2);
        step(kt + 1, L1, L0);
        step(kt + 2, L2, L1);
    }
    if (kt < nk) step(kt, L0, L2);
    if (kt + 1 < nk) step(kt + 1, L1, L0);
}

// grid: (ceil(max(f, fs) / 128), tile capacity); block 512; LDS kGemmLds.
// A = E4M3 codes of x rows gathered through pair_of_row, scales xs [N][d/128].
// The epilogue quantises each row's 128 H columns of the tile (one 1 x 128
// group) to hq / hs.
template <bool BLKW, bool DMA>
__global__ __launch_bounds__(kThreads) void gate_up_gemm_f8_kernel(
    const uint8_t *__restrict__ xq, const float *__restrict__ xs, const void *__restrict__ wg,
    const void *__restrict__ wu, const float *__restrict__ sg, const float *__restrict__ su,
    const void *__restrict__ wsg, const void *__restrict__ wsu, const float *__restrict__ ssg,
    const float *__restrict__ ssu, const int32_t *__restrict__ tiles, const int32_t *__restrict__ n_tiles,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ por, uint8_t *__restrict__ hq,
    float *__restrict__ hs, int ldh, int d, int E, int k, int f, int fs) {
    extern __shared__ uint8_t ldsb[];
    int item;
    if (!xcd_item(*n_tiles * (int)gridDim.x, item)) return;
    const int u = item / gridDim.x;
    const int g = tiles[2 * u], m0 = tiles[2 * u + 1];
    const bool shared = g == E;
    const int fg = shared ? fs : f;
    constexpr int kHalf = kBN / 2;
    const int c0 = (item % gridDim.x) * kHalf;
    if (c0 >= fg) return;
    const int gstart = offsets[g];
    const int row0 = gstart + m0, m = min(kBM, offsets[g + 1] - row0);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 2, wn = wave & 3;
    const int nkb = d / 128;

    auto token_of = [&](int r) { return shared ? (row0 + r - gstart) : por[row0 + r] / k; };
    size_t a_off[kAPer];
    uint32_t b_off[kBPer];
    bool a_ok[kAPer];
    const uint8_t *b_base[kBPer];
    const size_t wrow0 = shared ? 0 : (size_t)g * f;
#pragma unroll
    for (int j = 0; j < kAPer; ++j) {
        const int r = (tid >> 3) + 64 * j;
        a_ok[j] = r < m;
        a_off[j] = (size_t)token_of(a_ok[j] ? r : 0) * d;
    }
    // loader rows tid/8 + 64 j: j < 2 are gate rows c0.., j >= 2 the matching up rows
    const uint8_t *gbase = (const uint8_t *)(shared ? wsg : wg) + (wrow0 + c0) * (size_t)d;
    const uint8_t *ubase = (const uint8_t *)(shared ? wsu : wu) + (wrow0 + c0) * (size_t)d;
#pragma unroll
    for (int j = 0; j < kBPer; ++j) {
        const int r = (tid >> 3) + 64 * j;
        b_base[j] = j * 64 >= kHalf ? ubase : gbase;
        b_off[j] = (uint32_t)((r & (kHalf - 1)) * d);   // f_g is a multiple of 128
    }
    uint32_t sa_off[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        const int r = wm * 64 + mi * 16 + (lane & 15);
        sa_off[mi] = (uint32_t)(token_of(r < m ? r : 0) * nkb);
    }
    const float *sw_lo = nullptr, *sw_hi = nullptr;
    if (BLKW) {
        const size_t sb = ((shared ? 0 : (size_t)g * (f / 128)) + c0 / 128) * (size_t)nkb;
        sw_lo = (shared ? ssg : sg) + sb;
        sw_hi = (shared ? ssu : su) + sb;
    }
    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float *red;   // [128 rows][4 column waves] for the epilogue's row maxima
    if constexpr (DMA) {
        // direct-to-LDS: lane i of DMA j of wave w fetches tile row 8 (w n + j) + i / 8
        // into chunk position i % 8 (source chunk (i % 8) ^ (row & 7))
        __shared__ float red_l[kBM * 4];
        red = red_l;
        const int pos = lane & 7;
        const uint8_t *a_src[kAPer], *b_src[kBPer];
        const float *sa_row[kAPer];
#pragma unroll
        for (int j = 0; j < kAPer; ++j) {
            const int r = 8 * (wave * kAPer + j) + (lane >> 3);
            const int t = token_of(r < m ? r : 0);
            a_src[j] = xq + (size_t)t * d + ((pos ^ (r & 7)) << 4);
            sa_row[j] = xs + (size_t)t * nkb;
        }
#pragma unroll
        for (int j = 0; j < kBPer; ++j) {
            const int r = 8 * (wave * kBPer + j) + (lane >> 3);
            b_src[j] = (r >= kHalf ? ubase : gbase) + (size_t)(r & (kHalf - 1)) * d + ((pos ^ (r & 7)) << 4);
        }
        tile_mma_dma_f8<BLKW>(a_src, b_src, sa_row, sw_lo, sw_hi, d, m, acc);
    } else {
        red = reinterpret_cast<float *>(ldsb);
        tile_mma_f8<BLKW>(xq, a_off, a_ok, b_base, b_off, d, xs, sa_off, sw_lo, sw_hi, m, ldsb, acc);
    }

    // SwiGLU: hv[mi][ni][q] is row wm*64 + mi*16 + lane%16, H column
    // c0 + wn*32 + ni*16 + 4*(lane/16) + q
    float hv[4][2][4];
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
        const int col = c0 + wn * 32 + ni * 16 + (lane >> 4) * 4;
        float gs[4] = {1.f, 1.f, 1.f, 1.f}, us[4] = {1.f, 1.f, 1.f, 1.f};
        if (!BLKW) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                gs[q] = shared ? ssg[col + q] : sg[wrow0 + col + q];
                us[q] = shared ? ssu[col + q] : su[wrow0 + col + q];
            }
        }
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int q = 0; q < 4; ++q) hv[mi][ni][q] = silu(acc[mi][ni][q] * gs[q]) * (acc[mi][ni + 2][q] * us[q]);
    }
    // row maxima over the tile's 128 columns: this wave's 32, then across the 4 column waves in LDS
    float amax[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        float mx = 0.f;
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int q = 0; q < 4; ++q) mx = fmaxf(mx, fabsf(hv[mi][ni][q]));
        mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        amax[mi] = mx;
    }
    lds_barrier();   // every wave is done reading the operand tiles
    if (lane < 16) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) red[(wm * 64 + mi * 16 + lane) * 4 + wn] = amax[mi];
    }
    lds_barrier();
    const int nhb = ldh / 128;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        const int r = wm * 64 + mi * 16 + (lane & 15);
        const float4 rm = *reinterpret_cast<const float4 *>(red + r * 4);
        const float mx = fmaxf(fmaxf(rm.x, rm.y), fmaxf(rm.z, rm.w));
        const float sc = mx > 0.f ? mx / 448.0f : 1.0f;
        if (r < m) {
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) {
                const int col = c0 + wn * 32 + ni * 16 + (lane >> 4) * 4;
                float v[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) v[q] = fminf(fmaxf(hv[mi][ni][q] / sc, -448.f), 448.f);
                uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
                w = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], w, true);
                *reinterpret_cast<uint32_t *>(hq + (size_t)(row0 + r) * ldh + col) = w;
            }
            if (wn == 0 && lane < 16) hs[(size_t)(row0 + r) * nhb + c0 / 128] = sc;
        }
    }
}

// grid: (ceil(d / 256), tile capacity); block 512; LDS kGemmLds.
// A = E4M3 codes of the group's hidden rows (contiguous), scales hs.
template <bool BLKW, bool DMA>
__global__ __launch_bounds__(kThreads) void down_gemm_f8_kernel(
    const uint8_t *__restrict__ hq, const float *__restrict__ hs, int ldh, const void *__restrict__ wd,
    const float *__restrict__ sd, const void *__restrict__ wsd, const float *__restrict__ ssd,
    const int32_t *__restrict__ tiles, const int32_t *__restrict__ n_tiles, const int32_t *__restrict__ offsets,
    uint16_t *__restrict__ Y, int d, int E, int f, int fs) {
    extern __shared__ uint8_t ldsb[];
    int item;
    if (!xcd_item(*n_tiles * (int)gridDim.x, item)) return;
    const int u = item / gridDim.x;
    const int g = tiles[2 * u], m0 = tiles[2 * u + 1];
    const bool shared = g == E;
    const int fg = shared ? fs : f;
    const int o0 = (item % gridDim.x) * kBN;
    const int row0 = offsets[g] + m0, m = min(kBM, offsets[g + 1] - row0);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 2, wn = wave & 3;
    const uint8_t *base = (const uint8_t *)(shared ? wsd : wd);
    const size_t obase = shared ? 0 : (size_t)g * d;
    const int nhb = ldh / 128;

    size_t a_off[kAPer];
    uint32_t b_off[kBPer];
    bool a_ok[kAPer];
    const uint8_t *b_base[kBPer];
#pragma unroll
    for (int j = 0; j < kAPer; ++j) {
        const int r = (tid >> 3) + 64 * j;
        a_ok[j] = r < m;
        a_off[j] = (size_t)(row0 + (a_ok[j] ? r : 0)) * ldh;
    }
    const uint8_t *ebase = base + obase * (size_t)fg;   // this expert's [d][f_g] matrix
#pragma unroll
    for (int j = 0; j < kBPer; ++j) {
        const int r = (tid >> 3) + 64 * j;
        b_base[j] = ebase;
        b_off[j] = (uint32_t)((o0 + r < d ? o0 + r : 0) * fg);   // rows past d: never stored
    }
    uint32_t sa_off[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        const int r = wm * 64 + mi * 16 + (lane & 15);
        sa_off[mi] = (uint32_t)((row0 + (r < m ? r : 0)) * nhb);
    }
    const float *sw_lo = nullptr, *sw_hi = nullptr;
    if (BLKW) {
        const int nkb = fg / 128, nob = d / 128, ob = o0 / 128;
        const float *sp = shared ? ssd : sd + (size_t)g * nob * nkb;
        sw_lo = sp + (size_t)ob * nkb;
        sw_hi = sp + (size_t)(ob + 1 < nob ? ob + 1 : ob) * nkb;
    }
    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if constexpr (DMA) {
        // direct-to-LDS (see the gate/up kernel for the lane -> row map)
        const int pos = lane & 7;
        const uint8_t *a_src[kAPer], *b_src[kBPer];
        const float *sa_row[kAPer];
#pragma unroll
        for (int j = 0; j < kAPer; ++j) {
            const int r = 8 * (wave * kAPer + j) + (lane >> 3);
            const size_t row = (size_t)row0 + (r < m ? r : 0);
            a_src[j] = hq + row * ldh + ((pos ^ (r & 7)) << 4);
            sa_row[j] = hs + row * nhb;
        }
#pragma unroll
        for (int j = 0; j < kBPer; ++j) {
            const int r = 8 * (wave * kBPer + j) + (lane >> 3);
            b_src[j] = ebase + (size_t)(o0 + r < d ? o0 + r : 0) * fg + ((pos ^ (r & 7)) << 4);
        }
        tile_mma_dma_f8<BLKW>(a_src, b_src, sa_row, sw_lo, sw_hi, fg, m, acc);
    } else {
        tile_mma_f8<BLKW>(hq, a_off, a_ok, b_base, b_off, fg, hs, sa_off, sw_lo, sw_hi, m, ldsb, acc);
    }

#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
        const int o = o0 + b_row_of(wn, ni) + (lane >> 4) * 4;
        if (o >= d) continue;
        float sc[4] = {1.f, 1.f, 1.f, 1.f};
        if (!BLKW) {
#pragma unroll
            for (int q = 0; q < 4; ++q) sc[q] = shared ? ssd[o + q] : sd[obase + o + q];
        }
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const int r = wm * 64 + mi * 16 + (lane & 15);
            if (r < m)
                *reinterpret_cast<uint2 *>(Y + (size_t)(row0 + r) * d + o) =
                    make_uint2(pack_bf16x2(acc[mi][ni][0] * sc[0], acc[mi][ni][1] * sc[1]),
                               pack_bf16x2(acc[mi][ni][2] * sc[2], acc[mi][ni][3] * sc[3]));
        }
    }
}

// ---------------------------------------------------------------- router
// "Inside Kolibri 1" (flozi.net), section "Routing: selection bias and
// mixture weights are separate": FP32 logits [N, 384] from the flattened
// tokens.  For larger batches the router is one bf16 GEMM: each FP32 router
// weight is split exactly into three bf16 terms (hi and mid by truncation,
// lo = the rest, at most 8 significant bits) laid side by side along K,
// W3[e] = [hi(W_r[e]) | mid(W_r[e]) | lo(W_r[e])], and the A loader reads x
// three times along K.  Products of bf16 values are exact in FP32 and all 3d
// terms of a logit accumulate in one FP32 accumulator.

// grid: E (one workgroup per router row); block 256.  Also writes flags[e] =
// whether any mid or lo term of row e is nonzero (bf16-representable router
// weights, as in the pages' checkpoint, have none).
__global__ __launch_bounds__(256) void router_split_kernel(const float *__restrict__ rw, uint16_t *__restrict__ w3,
                                                           int32_t *__restrict__ flags, int E, int d) {
    const int e = blockIdx.x;
    uint16_t *row = w3 + (size_t)e * 3 * d;
    const float4 *src = reinterpret_cast<const float4 *>(rw + (size_t)e * d);
    int any = 0;
    // four weights per thread and pass (d is a multiple of 64): one 16-byte
    // load, three 8-byte stores
    for (int q = threadIdx.x; q < d / 4; q += blockDim.x) {
        const float4 v4 = src[q];
        const float v[4] = {v4.x, v4.y, v4.z, v4.w};
        uint32_t hw[2] = {0, 0}, mw[2] = {0, 0}, lw[2] = {0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t uh = __float_as_uint(v[i]) & 0xFFFF0000u;
            const float r1 = v[i] - __uint_as_float(uh);
            const uint32_t um = __float_as_uint(r1) & 0xFFFF0000u;
            const float r2 = r1 - __uint_as_float(um);
            const uint32_t m = um >> 16, l = f32_to_bf16_rne(r2);
            hw[i >> 1] |= (uh >> 16) << (16 * (i & 1));
            mw[i >> 1] |= m << (16 * (i & 1));
            lw[i >> 1] |= l << (16 * (i & 1));
            any |= ((m | l) & 0x7FFF) != 0;   // a -0 term contributes nothing either
        }
        *reinterpret_cast<uint2 *>(row + 4 * q) = make_uint2(hw[0], hw[1]);
        *reinterpret_cast<uint2 *>(row + d + 4 * q) = make_uint2(mw[0], mw[1]);
        *reinterpret_cast<uint2 *>(row + 2 * d + 4 * q) = make_uint2(lw[0], lw[1]);
    }
    any = __syncthreads_or(any);
    if (threadIdx.x == 0) flags[e] = any;
}

// The product runs on the direct-to-LDS tile: 128 tokens x 256 experts per
// workgroup, x and W3 rows fetched straight into three LDS stages (the
// register-staged 128 x 128 tile took 46 us at N = 8192 against 30 us).
// grid: (ceil(E / 256), ceil(N / 128), ks); block 512; static LDS.
// Slice z covers GEMM columns [z*3d/ks, (z+1)*3d/ks) (never two terms, so
// its x columns are that range modulo d) and writes partial[z].
__global__ __launch_bounds__(kThreads) void router_gemm_dma_kernel(const uint16_t *__restrict__ x,
                                                                   const uint16_t *__restrict__ w3,
                                                                   const int32_t *__restrict__ flags,
                                                                   float *__restrict__ partial, int N, int d, int E) {
    const int t0 = blockIdx.y * kBM, e0 = blockIdx.x * kBN;
    const int tid = threadIdx.x;
    if ((int)blockIdx.z >= (int)gridDim.z / 3) {   // mid or lo slice: skipped when all its experts' terms are zero
        const int e = e0 + tid;
        const int any = __syncthreads_or(tid < kBN && e < E ? flags[e] : 0);
        if (!any) return;
    }
    const int m = min(kBM, N - t0);
    const int kslice = 3 * d / (int)gridDim.z;
    const int kz = (int)blockIdx.z * kslice, ka = kz % d;
    // lane i of DMA j of wave w fills tile row 8 (w n + j) + i / 8 at swizzled chunk i % 8
    const int lane = tid & 63, w = tid >> 6, pos = lane & 7;
    const uint16_t *a_src[kAPer], *b_src[kBPer];
#pragma unroll
    for (int j = 0; j < kAPer; ++j) {
        const int r = 8 * (w * kAPer + j) + (lane >> 3);
        a_src[j] = x + (size_t)(t0 + (r < m ? r : 0)) * d + ka + ((pos ^ (r & 7)) << 3);
    }
#pragma unroll
    for (int j = 0; j < kBPer; ++j) {
        const int r = 8 * (w * kBPer + j) + (lane >> 3);
        // rows past E re-read row 0; never stored
        b_src[j] = w3 + (size_t)(e0 + r < E ? e0 + r : 0) * 3 * d + kz + ((pos ^ (r & 7)) << 3);
    }
    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    tile_mma_dma(a_src, b_src, kslice, m, acc);

    float *logits = partial + (size_t)blockIdx.z * N * E;
    const int wave = tid >> 6, wm = wave / kWN, wn = wave % kWN;
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
        const int e = e0 + b_row_of(wn, ni) + (lane >> 4) * 4;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const int r = wm * 64 + mi * 16 + (lane & 15);
            if (r >= m) continue;
            float *dst = logits + (size_t)(t0 + r) * E + e;
            if (e + 3 < E && (E & 3) == 0) {
                *reinterpret_cast<float4 *>(dst) = make_float4(acc[mi][ni][0], acc[mi][ni][1], acc[mi][ni][2], acc[mi][ni][3]);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (e + q < E) dst[q] = acc[mi][ni][q];
            }
        }
    }
}

hipError_t launch_router_gemm(const Plan &p, uint16_t *w3) {
    hipLaunchKernelGGL(router_split_kernel, dim3(p.E), dim3(256), 0, p.stream, p.rw, w3, p.rflags, p.E, p.d);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid((p.E + kBN - 1) / kBN, (p.N + kBM - 1) / kBM, p.ks);
    hipLaunchKernelGGL(router_gemm_dma_kernel, grid, dim3(kThreads), 0, p.stream, (const uint16_t *)p.x, w3,
                       p.rflags, p.partial, p.N, p.d, p.E);
    return hipGetLastError();
}

template <typename K>
static hipError_t allow_lds(K kernel, size_t bytes = kGemmLds) {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)bytes);
}

hipError_t gemm_kernels_init() {
    hipError_t e;
    if ((e = allow_lds(gate_up_gemm_kernel<kWBf16, true>)) != hipSuccess) return e;
    if ((e = allow_lds(gate_up_gemm_kernel<kWFp8Row, true>)) != hipSuccess) return e;
    if ((e = allow_lds(gate_up_gemm_kernel<kWFp8Blk, false>)) != hipSuccess) return e;
    if ((e = allow_lds(gate_up_gemm_kernel<kWFp8Blk, true>)) != hipSuccess) return e;
    if ((e = allow_lds(down_gemm_kernel<kWFp8Blk>)) != hipSuccess) return e;
    if ((e = allow_lds(gate_up_gemm_f8_kernel<true, false>)) != hipSuccess) return e;
    if ((e = allow_lds(gate_up_gemm_f8_kernel<false, false>)) != hipSuccess) return e;
    if ((e = allow_lds(down_gemm_f8_kernel<true, false>)) != hipSuccess) return e;
    if ((e = allow_lds(down_gemm_f8_kernel<false, false>)) != hipSuccess) return e;
    // the direct-to-LDS kernels (bf16 x with bf16 or FP8 weights, FP8 x FP8
    // within 24 K blocks, the router GEMM) use static LDS only
    return hipSuccess;
}

// FP8 x FP8 products with every K range within kF8DmaMaxKb blocks run the
// direct-to-LDS tile (its scales live in LDS for the whole K range)
static bool w8b_dma(const Plan &p) {   // block-scaled FP8 weights, bf16 activations: the same K bound
    return p.d / 128 <= kF8DmaMaxKb && p.f / 128 <= kF8DmaMaxKb && p.fs / 128 <= kF8DmaMaxKb;
}

// ---- the wide FP8 x FP8 gate/up tile (1 x 128 activation quantisation, from
// 8192 tokens): 256 x 256 items (256 rows; 128 gate columns and the matching
// 128 up columns), 8 waves in 2 (rows) x 4 (columns), each 128 x 64 with 128
// accumulator registers (two waves per SIMD), one 128-wide K block per
// stage.  Per stage the activation codes (32 KB), the weight codes (32 KB)
// and the 256 rows' activation scales of that K block arrive by DMA (one
// dword DMA per wave: rows 32 w .. 32 w + 31), two stages of each in LDS;
// with block scales the tile's gate and up K-block weight scales come once,
// before the loop.  Every stage's products are formed per 16-row sub-tile
// (one v_mfma_f32_16x16x128_f8f6f4 per 16 x 16 block) and folded into the
// FP32 sums times (row's activation scale) x (column block's weight scale),
// in the order tile_mma_dma_f8 uses, so H matches the 128-row kernel bit for
// bit.  The SwiGLU epilogue quantises each row's 128 H values of the tile (the
// row maximum crosses the 4 column waves through LDS).  Twice the flops per
// operand byte of the 128 x 256 FP8 tile.
constexpr int kF8WRows = 256;
constexpr int kF8WOp = kF8WRows * 128;    // one operand tile of one stage (32 KB)
constexpr int kF8WScl = 8 * 256;          // one stage's row scales: 64 slots per wave, 32 used
template <bool BLKW>
__global__ __launch_bounds__(512) void gate_up_gemm_f8_wide_kernel(
    const uint8_t *__restrict__ xq, const float *__restrict__ xs, const void *__restrict__ wg,
    const void *__restrict__ wu, const float *__restrict__ sg, const float *__restrict__ su,
    const void *__restrict__ wsg, const void *__restrict__ wsu, const float *__restrict__ ssg,
    const float *__restrict__ ssu, const int32_t *__restrict__ tiles, const int32_t *__restrict__ n_tiles,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ por, uint8_t *__restrict__ hq,
    float *__restrict__ hs, int ldh, int d, int E, int k, int f, int fs) {
    // LDS: activations A0 A1, weights B0 B1, row scales S0 S1, the weight block scales
    // (gate, then up: 256 bytes each, what one 64-lane dword DMA writes)
    constexpr int kA = 0, kB = 2 * kF8WOp, kS = 4 * kF8WOp, kWsc = kS + 2 * kF8WScl;
    constexpr int kAPerW = 4, kBPerW = 4;   // 1 KB DMAs per wave and operand stage
    constexpr int G = kAPerW + kBPerW + 1;  // DMAs per wave and stage
    // a 64-lane dword DMA writes 256 bytes: one row-scale region per wave, one block-scale region each
    static_assert(kF8WScl == 8 * 256 && kWsc + 2 * 256 <= 160 * 1024, "DMA regions");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kWsc + 512];
    int item;
    if (!xcd_item(*n_tiles * (int)gridDim.x, item)) return;
    const int u = item / gridDim.x;
    const int g = tiles[2 * u], m0 = tiles[2 * u + 1];
    const bool shared = g == E;
    const int fg = shared ? fs : f;
    const int c0 = (item % gridDim.x) * 128;
    if (c0 >= fg) return;
    const int gstart = offsets[g];
    const int row0 = gstart + m0, m = min(kF8WRows, offsets[g + 1] - row0);
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), pos = lane & 7;
    const int wm = w >> 2, wn = w & 3;
    const int fr = lane & 15, fq = lane >> 4;
    const int nk = d / 128;
    auto token_row = [&](int r) { return shared ? (row0 + r - gstart) : por[row0 + r] / k; };

    // DMA sources (byte offsets at K = 0): rows past the group end read row 0 (never stored)
    uint32_t a_off[kAPerW], b_off[kBPerW], s_off;
#pragma unroll
    for (int j = 0; j < kAPerW; ++j) {
        const int r = 8 * (w * kAPerW + j) + (lane >> 3);
        a_off[j] = (uint32_t)token_row(r < m ? r : 0) * (uint32_t)d + (uint32_t)((pos ^ (r & 7)) << 4);
    }
    const size_t wrow0 = shared ? 0 : (size_t)g * f;
    // weight rows 0..127 are gate rows c0.., 128..255 the matching up rows: waves 0-3 fetch gate rows
    const uint8_t *b_base = uniform_ptr((const uint8_t *)(w < 4 ? (shared ? wsg : wg) : (shared ? wsu : wu)) +
                                        (wrow0 + c0) * (size_t)d);
#pragma unroll
    for (int j = 0; j < kBPerW; ++j) {
        const int r = 8 * (w * kBPerW + j) + (lane >> 3);
        b_off[j] = (uint32_t)(r & 127) * (uint32_t)d + (uint32_t)((pos ^ (r & 7)) << 4);
    }
    {
        const int r = 32 * w + (lane & 31);
        s_off = (uint32_t)token_row(r < m ? r : 0) * (uint32_t)nk * 4u;
    }
    const uint32_t s0 = (uint32_t)(uintptr_t)(lds_void_t *)smem;
    auto fetch = [&](int kt, int buf) __attribute__((always_inline)) {
        const uint8_t *sa = xq + kt * 128, *sb = b_base + kt * 128;
#pragma unroll
        for (int j = 0; j < kAPerW; ++j) dma16s(sa, a_off[j], smem + kA + buf * kF8WOp + (w * kAPerW + j) * 1024);
#pragma unroll
        for (int j = 0; j < kBPerW; ++j) dma16s(sb, b_off[j], smem + kB + buf * kF8WOp + (w * kBPerW + j) * 1024);
        dma4s(xs + kt, s_off, smem + kS + buf * kF8WScl + w * 256);
    };
    if constexpr (BLKW) {   // the tile's K-block weight scales: gate (wave 0) and up (wave 1)
        if (w < 2) {
            const size_t sb = ((shared ? 0 : (size_t)g * (f / 128)) + c0 / 128) * (size_t)nk;
            const float *src = (w == 0 ? (shared ? ssg : sg) : (shared ? ssu : su)) + sb;
            dma4s(src, lane < nk ? lane * 4 : 0, smem + kWsc + w * 256);
        }
    }
    fetch(0, 0);
    if (nk > 1) fetch(1, 1);
    if (nk > 1) __builtin_amdgcn_s_waitcnt(FGS_VMCNT(G));
    else __builtin_amdgcn_s_waitcnt(FGS_VMCNT(0));
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);

    // fragment addresses in buffer 0: activation row wm*128 + lane%16 (+16 mi), weight row
    // b_row_of(wn, ni) + lane%16; a lane's 32 K bytes are chunks 2 (lane/16) and 2 (lane/16) + 1
    uint32_t la[2], lb[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int ch = 2 * fq + c;
        la[c] = s0 + kA + (wm * 128 + fr) * 128 + ((ch ^ (fr & 7)) << 4);
        lb[c] = s0 + kB + (wn * 32 + fr) * 128 + ((ch ^ (fr & 7)) << 4);
    }
    // this lane's row scale slot for sub-tile mi: row wm*128 + mi*16 + lane%16 -> (row / 32) * 64 + row % 32
    const uint32_t ls = s0 + kS + (uint32_t)(((wm * 128 + fr) >> 5) * 64 + ((wm * 128 + fr) & 31)) * 4u;

    f32x4_t acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto run = [&](auto live_c) __attribute__((always_inline)) {
        constexpr int LV = decltype(live_c)::value;   // live 16-row sub-tiles (rounded up to even)
        auto stage = [&](int kt, auto p_c) __attribute__((always_inline)) {
            constexpr int P = decltype(p_c)::value;   // buffer kt % 2
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (LV > 0) {
                uint4 bf[4][2];
#pragma unroll
                for (int ni = 0; ni < 4; ++ni)
#pragma unroll
                    for (int c = 0; c < 2; ++c)
                        bf[ni][c] = lds_read16(lb[c] + P * kF8WOp + (ni < 2 ? ni * 16 : 128 + (ni - 2) * 16) * 128);
                const float wlo = BLKW ? lds_read_f32(s0 + kWsc + kt * 4) : 1.f;
                const float whi = BLKW ? lds_read_f32(s0 + kWsc + 256 + kt * 4) : 1.f;
                uint4 a0 = lds_read16(la[0] + P * kF8WOp), a1 = lds_read16(la[1] + P * kF8WOp);
                // the products of sub-tile mi are folded while those of mi + 1 are formed
                // (two product sets alternate), so the matrix core and the FP32 folds overlap
                f32x4_t p0[4], p1[4];
                float sp0 = 0.f, sp1 = 0.f;   // the row scale of the products in p0 / p1
                auto fold = [&](int mi, const f32x4_t (&pr)[4], float sa) __attribute__((always_inline)) {
                    const float clo = sa * wlo, chi = sa * whi;
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni) {
                        const float c = ni < 2 ? clo : chi;
#pragma unroll
                        for (int q = 0; q < 4; ++q) acc[mi][ni][q] = fmaf(pr[ni][q], c, acc[mi][ni][q]);
                    }
                    // the empty statements take the sums as operands: the fold happens here,
                    // not at the end of the stage (which would keep every product live)
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni) asm volatile("" : "+v"(acc[mi][ni]));
                };
#pragma unroll
                for (int mi = 0; mi < LV; ++mi) {
                    // the next sub-tile's fragments requested before this one's MFMAs
                    uint4 n0 = a0, n1 = a1;
                    if (mi + 1 < LV) {
                        n0 = lds_read16(la[0] + P * kF8WOp + (mi + 1) * 16 * 128);
                        n1 = lds_read16(la[1] + P * kF8WOp + (mi + 1) * 16 * 128);
                    }
                    // sub-tile mi's rows are 16 consecutive rows: slot offset (mi*16 / 32) * 64 + (mi & 1) * 16
                    const float sa = lds_read_f32(ls + P * kF8WScl + (uint32_t)((mi >> 1) * 64 + (mi & 1) * 16) * 4u);
                    if (mi & 1) {
#pragma unroll
                        for (int ni = 0; ni < 4; ++ni) p1[ni] = mfma_f8(bf[ni][0], bf[ni][1], a0, a1);
                        sp1 = sa;
                        fold(mi - 1, p0, sp0);
                    } else {
#pragma unroll
                        for (int ni = 0; ni < 4; ++ni) p0[ni] = mfma_f8(bf[ni][0], bf[ni][1], a0, a1);
                        sp0 = sa;
                        if (mi > 0) fold(mi - 1, p1, sp1);
                    }
                    a0 = n0;
                    a1 = n1;
                    __builtin_amdgcn_sched_barrier(0);
                }
                if ((LV - 1) & 1) fold(LV - 1, p1, sp1);
                else fold(LV - 1, p0, sp0);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (kt + 1 < nk) {
                // own DMAs of stage kt+1 landed and every wave is done with buffer P: refill it
                __builtin_amdgcn_s_waitcnt(FGS_VMCNT(0));
                lds_barrier();
                if (kt + 2 < nk) fetch(kt + 2, P);
            }
        };
        int kt = 0;
        for (; kt + 2 <= nk; kt += 2) {
            stage(kt, Live<0>{});
            stage(kt + 1, Live<1>{});
        }
        if (kt < nk) stage(kt, Live<0>{});
    };
    const int live = min(8, max(0, (m - wm * 128 + 15) / 16));
    switch ((live + 1) & ~1) {
        case 8: run(Live<8>{}); break;
        case 6: run(Live<6>{}); break;
        case 4: run(Live<4>{}); break;
        case 2: run(Live<2>{}); break;
        default: run(Live<0>{}); break;
    }

    // SwiGLU into acc[mi][0..1]: row wm*128 + mi*16 + lane%16, H column c0 + wn*32 + ni*16 + 4 (lane/16) + q
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
        const int col = c0 + wn * 32 + ni * 16 + fq * 4;
        float gs[4] = {1.f, 1.f, 1.f, 1.f}, us[4] = {1.f, 1.f, 1.f, 1.f};
        if (!BLKW) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                gs[q] = shared ? ssg[col + q] : sg[wrow0 + col + q];
                us[q] = shared ? ssu[col + q] : su[wrow0 + col + q];
            }
        }
#pragma unroll
        for (int mi = 0; mi < 8; ++mi)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[mi][ni][q] = silu(acc[mi][ni][q] * gs[q]) * (acc[mi][ni + 2][q] * us[q]);
    }
    // row maxima over the tile's 128 H columns: this wave's 32, then across the 4 column
    // waves through LDS (the first activation buffer, free once every wave is done)
    float amax[8];
#pragma unroll
    for (int mi = 0; mi < 8; ++mi) {
        float mx = 0.f;
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int q = 0; q < 4; ++q) mx = fmaxf(mx, fabsf(acc[mi][ni][q]));
        mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        amax[mi] = mx;
    }
    lds_barrier();
    float *red = reinterpret_cast<float *>(smem + kA);   // [256 rows][4 column waves]
    if (lane < 16) {
#pragma unroll
        for (int mi = 0; mi < 8; ++mi) red[(wm * 128 + mi * 16 + lane) * 4 + wn] = amax[mi];
    }
    lds_barrier();
    const int nhb = ldh / 128;
#pragma unroll
    for (int mi = 0; mi < 8; ++mi) {
        const int r = wm * 128 + mi * 16 + fr;
        const float4 rm = *reinterpret_cast<const float4 *>(red + r * 4);
        const float mx = fmaxf(fmaxf(rm.x, rm.y), fmaxf(rm.z, rm.w));
        const float sc = mx > 0.f ? mx / 448.0f : 1.0f;
        if (r < m) {
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) {
                const int col = c0 + wn * 32 + ni * 16 + fq * 4;
                float v[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) v[q] = fminf(fmaxf(acc[mi][ni][q] / sc, -448.f), 448.f);
                uint32_t wv = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
                wv = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], wv, true);
                *reinterpret_cast<uint32_t *>(hq + (size_t)(row0 + r) * ldh + col) = wv;
            }
            if (wn == 0 && lane < 16) hs[(size_t)(row0 + r) * nhb + c0 / 128] = sc;
        }
    }
}

// ---- persistent FP8 x FP8 down product (1 x 128 quantised H, E4M3 weights with
// per-channel or 128 x 128 block scales), K (f and f_s) at most 4 blocks of 128,
// d a multiple of 256.  The ring and the item walk of down_gemm_persist_kernel
// with 128-wide K stages of E4M3 codes (48 KB: 128 H rows and 256 weight rows
// of 128 bytes).  With an item's first stage every wave fetches one quarter
// of its activation scales (K block w / 2, rows 64 (w % 2) ..: 512 values in
// an LDS slot) and wave 0 its weight scales (both output blocks' K-block
// scales, or 256 column scales), all ahead of the stage's own DMAs.  All of a
// stage's fragments are read before its barrier; each 16 x 16 product (one
// v_mfma_f32_16x16x128_f8f6f4) is folded into the FP32 sum times (row scale)
// x (block scale) one sub-tile behind the MFMAs, as tile_mma_dma_f8 orders
// them, so Y matches the one-item kernel bit for bit.
constexpr int kF8PSlot = 3 * 1024;   // 2 KB activation scales + 1 KB weight scales
template <bool BLKW>
__global__ __launch_bounds__(kThreads) void down_gemm_f8_persist_kernel(
    const uint8_t *__restrict__ hq, const float *__restrict__ hs, int ldh, const uint8_t *__restrict__ wd,
    const float *__restrict__ sd, const uint8_t *__restrict__ wsd, const float *__restrict__ ssd,
    const int32_t *__restrict__ tiles, const int32_t *__restrict__ n_tiles, const int32_t *__restrict__ offsets,
    uint16_t *__restrict__ Y, int d, int E, int f, int fs) {
    static_assert(kAPer == 2 && kBPer == 4, "six operand DMAs per wave and stage");
    constexpr int NB = 3, kStage = kDmaStageB, G = kAPer + kBPer, kSlots = 4;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[NB * kStage + kSlots * kF8PSlot];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / kWN, wn = wave % kWN, fr = lane & 15, fg = lane >> 4, pos = lane & 7;
    const int gx = d / kBN, B = kXcdTiles * gx;
    const int n_items = *n_tiles * gx;
    const int G_wg = gridDim.x;
    const int nhb = ldh / 128;
    const uint32_t s0 = (uint32_t)(uintptr_t)(lds_void_t *)smem;
    constexpr int kSlotBase = NB * kStage;

    // fetch cursor
    int fq = 0, fkt = 0, fnk = 0, fbuf = 0, gf = 0;
    bool fvalid = false;
    uint32_t a_off[kAPer], b_off[kBPer], sa_off;
    const uint8_t *b_base = wd;
    const float *w_scale = sd;   // block scales (2 K-block runs) or 256 column scales of the item
    int w_cnt = 0;
    auto load_fetch_item = [&]() {
        const int item = xcd_map(blockIdx.x + fq * G_wg, B);
        fvalid = item < n_items;
        if (!fvalid) return;
        const int u = item / gx;
        const int g = tiles[2 * u], m0 = tiles[2 * u + 1];
        const bool shared = g == E;
        const int K = shared ? fs : f;
        const int o0 = (item % gx) * kBN;
        const int row0 = offsets[g] + m0, m = min(kBM, offsets[g + 1] - row0);
        const int nkb = K / 128;
        fnk = nkb;
        b_base = (shared ? wsd : wd + (size_t)g * d * K);
        if constexpr (BLKW) {   // [E][d/128][K/128]: output blocks o0/128 and o0/128 + 1 are adjacent
            w_scale = (shared ? ssd : sd + (size_t)g * (d / 128) * nkb) + (size_t)(o0 / 128) * nkb;
            w_cnt = 2 * nkb;
        } else {
            w_scale = shared ? ssd + o0 : sd + (size_t)g * d + o0;
        }
#pragma unroll
        for (int j = 0; j < kAPer; ++j) {
            const int r = 8 * (wave * kAPer + j) + (lane >> 3);
            a_off[j] = (uint32_t)(row0 + (r < m ? r : 0)) * (uint32_t)ldh + (uint32_t)((pos ^ (r & 7)) << 4);
        }
#pragma unroll
        for (int j = 0; j < kBPer; ++j) {
            const int r = 8 * (wave * kBPer + j) + (lane >> 3);
            b_off[j] = (uint32_t)(o0 + r) * (uint32_t)K + (uint32_t)((pos ^ (r & 7)) << 4);
        }
        // this wave's quarter of the activation scales: K block wave / 2, rows 64 (wave % 2) + lane
        const int kb = (wave >> 1) < nkb ? (wave >> 1) : 0, r = 64 * (wave & 1) + lane;
        sa_off = ((uint32_t)(row0 + (r < m ? r : 0)) * (uint32_t)nhb + (uint32_t)kb) * 4u;
    };
    auto fetch_next = [&]() {
        if (!fvalid) return;
        if (fkt == 0) {   // the item's scales, ahead of the stage's own DMAs
            uint8_t *slot = smem + kSlotBase + (fq & (kSlots - 1)) * kF8PSlot;
            dma4s(hs, sa_off, slot + wave * 256);
            if (wave == 0) {
                if constexpr (BLKW) dma4s(w_scale, lane < w_cnt ? lane * 4 : 0, slot + 2048);
                else dma16s(w_scale, lane * 16, slot + 2048);
            }
        }
        uint8_t *buf = smem + fbuf * kStage;
        const uint8_t *sa = hq + fkt * 128, *sb = b_base + fkt * 128;
#pragma unroll
        for (int j = 0; j < kAPer; ++j) dma16s(sa, a_off[j], buf + (wave * kAPer + j) * 1024);
#pragma unroll
        for (int j = 0; j < kBPer; ++j) dma16s(sb, b_off[j], buf + kBM * kDmaRowB + (wave * kBPer + j) * 1024);
        fbuf = fbuf == NB - 1 ? 0 : fbuf + 1;
        ++gf;
        if (++fkt == fnk) {
            fkt = 0;
            ++fq;
            load_fetch_item();
        }
    };
    auto wait_stages = [&](int later) {
        if (later >= 1) __builtin_amdgcn_s_waitcnt(FGS_VMCNT(G));
        else __builtin_amdgcn_s_waitcnt(FGS_VMCNT(0));
    };
    // fragment addresses in buffer 0: H row wm*64 + lane%16, weight row wn*64 + lane%16 (+ 16 per
    // column fragment: the wave's 64 columns are contiguous), K chunks 2 (lane/16) and 2 (lane/16) + 1
    uint32_t la[2], lb[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int ch = 2 * fg + c;
        la[c] = s0 + (wm * 64 + fr) * kDmaRowB + ((ch ^ (fr & 7)) << 4);
        lb[c] = s0 + kBM * kDmaRowB + (wn * 64 + fr) * kDmaRowB + ((ch ^ (fr & 7)) << 4);
    }

    load_fetch_item();
    if (!fvalid) return;
    fetch_next();
    fetch_next();
    wait_stages(gf - 1);   // stage 0 (and the first item's scales) landed
    lds_barrier();
    fetch_next();
    __builtin_amdgcn_sched_barrier(0);

    int gs = 0;
    for (int q = 0;; ++q) {
        const int item = xcd_map(blockIdx.x + q * G_wg, B);
        if (item >= n_items) break;
        const int u = item / gx;
        const int g = tiles[2 * u], m0 = tiles[2 * u + 1];
        const bool shared = g == E;
        const int nk = (shared ? fs : f) / 128;
        const int o0 = (item % gx) * kBN;
        const int row0 = offsets[g] + m0, m = min(kBM, offsets[g + 1] - row0);
        const uint32_t slot = s0 + kSlotBase + (q & (kSlots - 1)) * kF8PSlot;

        auto run = [&](auto live_c) __attribute__((always_inline)) {
            constexpr int LV = decltype(live_c)::value;
            f32x4_t acc[4][4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            int cb = gs % NB;
#pragma nounroll
            for (int kt = 0; kt < nk; ++kt) {
                const int nb = cb == NB - 1 ? 0 : cb + 1;
                uint4 bf[4][2], af[4][2];
                float sa[4] = {0.f, 0.f, 0.f, 0.f};
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (LV > 0) {
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
                        for (int c = 0; c < 2; ++c)
                            bf[ni][c] = lds_read16(lb[c] + cb * kStage + ni * 16 * kDmaRowB);
#pragma unroll
                    for (int mi = 0; mi < LV; ++mi) {
#pragma unroll
                        for (int c = 0; c < 2; ++c) af[mi][c] = lds_read16(la[c] + cb * kStage + mi * 16 * kDmaRowB);
                        sa[mi] = lds_read_f32(slot + (uint32_t)(kt * kBM + wm * 64 + mi * 16 + fr) * 4u);
                    }
                }
                // the wave's 64 columns lie in one 128-column output block
                const float wsc = BLKW ? lds_read_f32(slot + 2048 + ((wn < 2 ? 0 : nk) + kt) * 4) : 1.f;
                __builtin_amdgcn_sched_barrier(0);
                const bool last = kt + 1 == nk;
                const bool more = gf > gs + 1;
                if (more) wait_stages(gf - gs - 2);   // stage gs + 1 landed; a later one may stay in flight
                // every wave has read buffer cb: it may be refilled, or at the item's end
                // take the output staging
                if (more || last) lds_barrier();
                if (!last) fetch_next();   // stage gs + NB into buffer cb
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (LV > 0) {
                    f32x4_t p0[4], p1[4];
                    auto fold = [&](int mi, const f32x4_t (&pr)[4]) __attribute__((always_inline)) {
                        const float c = sa[mi] * wsc;
#pragma unroll
                        for (int ni = 0; ni < 4; ++ni) {
#pragma unroll
                            for (int qq = 0; qq < 4; ++qq) acc[mi][ni][qq] = fmaf(pr[ni][qq], c, acc[mi][ni][qq]);
                        }
#pragma unroll
                        for (int ni = 0; ni < 4; ++ni) asm volatile("" : "+v"(acc[mi][ni]));
                    };
#pragma unroll
                    for (int mi = 0; mi < LV; ++mi) {
                        if (mi & 1) {
#pragma unroll
                            for (int ni = 0; ni < 4; ++ni) p1[ni] = mfma_f8(bf[ni][0], bf[ni][1], af[mi][0], af[mi][1]);
                            fold(mi - 1, p0);
                        } else {
#pragma unroll
                            for (int ni = 0; ni < 4; ++ni) p0[ni] = mfma_f8(bf[ni][0], bf[ni][1], af[mi][0], af[mi][1]);
                            if (mi > 0) fold(mi - 1, p1);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    if ((LV - 1) & 1) fold(LV - 1, p1);
                    else fold(LV - 1, p0);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (last) {
                    // stage the output through this wave's own 2 KB of buffer cb (its activation
                    // chunks: every fragment of the stage was read before the barrier, and only
                    // this wave's next fetch, issued after these stores, writes there again)
                    const uint32_t ob = s0 + cb * kStage + wave * kAPer * 1024;
                    const uint32_t lane_off = ((uint32_t)(lane >> 3) * (uint32_t)d + (uint32_t)(lane & 7) * 8u) * 2u;
                    float sc[4][4];
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni) {
#pragma unroll
                        for (int qq = 0; qq < 4; ++qq) sc[ni][qq] = 1.f;
                        if constexpr (!BLKW) slot_scales(slot + 2048, wn * 64 + ni * 16, lane, sc[ni]);
                    }
#pragma unroll
                    for (int mi = 0; mi < LV; ++mi) {
                        const int rb = wm * 64 + mi * 16;
#pragma unroll
                        for (int ni = 0; ni < 4; ++ni) stage_bf16x4(ob, ni, lane, acc[mi][ni], sc[ni]);
#pragma unroll
                        for (int h = 0; h < 2; ++h)
                            if (rb + 8 * h + (lane >> 3) < m)
                                store_staged(ob, h, lane, Y + (size_t)(row0 + rb + 8 * h) * d + o0 + wn * 64, lane_off);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    if (more) fetch_next();
                }
                __builtin_amdgcn_sched_barrier(0);
                ++gs;
                cb = nb;
            }
        };
        const int live = min(4, max(0, (m - wm * 64 + 15) / 16));
        switch (live) {
            case 4: run(Live<4>{}); break;
            case 3: run(Live<3>{}); break;
            case 2: run(Live<2>{}); break;
            case 1: run(Live<1>{}); break;
            default: run(Live<0>{}); break;
        }
    }
}

static bool f8_dma(const Plan &p) {
    return p.d / 128 <= kF8DmaMaxKb && p.f / 128 <= kF8DmaMaxKb && p.fs / 128 <= kF8DmaMaxKb;
}

hipError_t launch_gate_up_gemm(const Plan &p) {
    const int fmax = p.f > p.fs ? p.f : p.fs;
    // spare tile rows: the XCD-aware order needs n + 8 * kXcdTiles * gx launch slots
    const int gx = (fmax + kBN / 2 - 1) / (kBN / 2);
    dim3 grid(gx, p.max_tiles + kXcds * kXcdTiles), block(kThreads);
    if (p.bm == kGemmBMWide && p.aq) {   // 1 x 128 activation quantisation, 256-row tiles (gemm_bm)
        hipError_t e = launch_quant_groups(p.x, 1, p.d, p.N, p.d, p.xq, p.d, p.xs, p.d / 128, p.stream);
        if (e != hipSuccess) return e;
#define FGS_GUFW(B)                                                                                              \
    hipLaunchKernelGGL((gate_up_gemm_f8_wide_kernel<B>), grid, dim3(512), 0, p.stream, p.xq, p.xs, p.W.w_gate,      \
                       p.W.w_up, p.W.s_gate, p.W.s_up, p.W.ws_gate, p.W.ws_up, p.W.ss_gate, p.W.ss_up, p.tiles,      \
                       p.n_tiles, p.offsets, p.por, p.hq, p.hs, p.ldh, p.d, p.E, p.k, p.f, p.fs)
        if (p.flags & MOE_FLAG_FP8_BLOCK128) FGS_GUFW(true); else FGS_GUFW(false);
#undef FGS_GUFW
        return hipGetLastError();
    }
    if (p.bm == kGemmBMWide) {   // bf16 activations, bf16 or per-channel E4M3 weights, 256-row tiles (gemm_bm)
#define FGS_GUW(W8)                                                                                            \
    hipLaunchKernelGGL((gate_up_gemm_wide_kernel<kWideWMW, W8>), grid, dim3(Wide<kWideWMW>::kThreads), 0, p.stream, \
                       (const uint16_t *)p.x, p.W.w_gate, p.W.w_up, p.W.s_gate, p.W.s_up, p.W.ws_gate, p.W.ws_up,   \
                       p.W.ss_gate, p.W.ss_up, p.tiles, p.n_tiles, p.offsets, p.por, p.H, p.ldh, p.d, p.E, p.k, p.f, \
                       p.fs)
        if (p.wdt == MOE_DTYPE_FP8_E4M3) FGS_GUW(true); else FGS_GUW(false);
#undef FGS_GUW
        return hipGetLastError();
    }
    if (p.aq) {
        hipError_t e = launch_quant_groups(p.x, 1, p.d, p.N, p.d, p.xq, p.d, p.xs, p.d / 128, p.stream);
        if (e != hipSuccess) return e;
#define FGS_GUF(B, D)                                                                                         \
    hipLaunchKernelGGL((gate_up_gemm_f8_kernel<B, D>), grid, block, D ? 0 : kGemmLds, p.stream, p.xq, p.xs,        \
                       p.W.w_gate, p.W.w_up, p.W.s_gate, p.W.s_up, p.W.ws_gate, p.W.ws_up, p.W.ss_gate, p.W.ss_up,  \
                       p.tiles, p.n_tiles, p.offsets, p.por, p.hq, p.hs, p.ldh, p.d, p.E, p.k, p.f, p.fs)
        const bool blk = (p.flags & MOE_FLAG_FP8_BLOCK128) != 0;
        if (f8_dma(p)) { if (blk) FGS_GUF(true, true); else FGS_GUF(false, true); }
        else { if (blk) FGS_GUF(true, false); else FGS_GUF(false, false); }
#undef FGS_GUF
        return hipGetLastError();
    }
#define FGS_GUG(WM, XF)                                                                                         \
    hipLaunchKernelGGL((gate_up_gemm_kernel<WM, XF>), grid, block,                                               \
                       ((WM == kWBf16 || WM == kWFp8Row || WM == kWFp8BlkDma) && !XF) ? 0 : kGemmLds, p.stream, p.x,    \
                       p.W.w_gate, p.W.w_up,                                                                           \
                       p.W.s_gate, p.W.s_up, p.W.ws_gate, p.W.ws_up, p.W.ss_gate, p.W.ss_up, p.tiles, p.n_tiles,  \
                       p.offsets, p.por, p.H, p.ldh, p.d, p.E, p.k, p.f, p.fs)
    const bool xf32 = p.xdt == MOE_DTYPE_F32;
    if (p.wdt != MOE_DTYPE_FP8_E4M3) { if (xf32) FGS_GUG(kWBf16, true); else FGS_GUG(kWBf16, false); }
    else if (p.flags & MOE_FLAG_FP8_BLOCK128) {
        if (xf32) FGS_GUG(kWFp8Blk, true);
        else if (w8b_dma(p)) FGS_GUG(kWFp8BlkDma, false);
        else FGS_GUG(kWFp8Blk, false);
    }
    else { if (xf32) FGS_GUG(kWFp8Row, true); else FGS_GUG(kWFp8Row, false); }
#undef FGS_GUG
    return hipGetLastError();
}

// compute units of the current device, rounded down to whole XCD groups (cached per device)
static hipError_t cu_count(int *out) {
    static std::atomic<int> cache[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        v = v / kXcds * kXcds;
        if (v < kXcds) v = kXcds;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    *out = v;
    return hipSuccess;
}

hipError_t launch_down_gemm(const Plan &p) {
    const int gx = (p.d + kBN - 1) / kBN;
    dim3 grid(gx, p.max_tiles + kXcds * kXcdTiles), block(kThreads);
    uint16_t *Y = reinterpret_cast<uint16_t *>(p.Y);
    // the down product (K = f, 8 stages at f = 512) keeps 128-row tiles: with wide
    // gate/up tiles the dispatch writes it a list of its own (a 256-row down tile was
    // slower at prefill size, 341 against 320 us: short K loop, idle row waves; taking
    // each wide entry as two 128-row items cost 15-23 us against the plain list)
    const int32_t *tiles = p.bm == kGemmBMWide ? p.tiles2 : p.tiles;
    const int32_t *n_tiles = p.bm == kGemmBMWide ? p.n_tiles2 : p.n_tiles;
    grid.y = (p.bm == kGemmBMWide ? p.max_tiles2 : p.max_tiles) + kXcds * kXcdTiles;
#if FGS_DOWN_PERSIST && FGS_DOWN_F8P
    if (p.aq && p.d % kBN == 0 && p.f <= 512 && p.fs <= 512 && p.f % 128 == 0 && p.fs % 128 == 0 &&
        ((long)p.N * p.k + p.N) * p.ldh < (1L << 32) && (long)p.d * (p.f > p.fs ? p.f : p.fs) < (1L << 32)) {
        int cus = 0;
        hipError_t e = cu_count(&cus);
        if (e != hipSuccess) return e;
        if (p.flags & MOE_FLAG_FP8_BLOCK128)
            hipLaunchKernelGGL(down_gemm_f8_persist_kernel<true>, dim3(cus), block, 0, p.stream, p.hq, p.hs, p.ldh,
                               (const uint8_t *)p.W.w_down, p.W.s_down, (const uint8_t *)p.W.ws_down, p.W.ss_down,
                               tiles, n_tiles, p.offsets, Y, p.d, p.E, p.f, p.fs);
        else
            hipLaunchKernelGGL(down_gemm_f8_persist_kernel<false>, dim3(cus), block, 0, p.stream, p.hq, p.hs, p.ldh,
                               (const uint8_t *)p.W.w_down, p.W.s_down, (const uint8_t *)p.W.ws_down, p.W.ss_down,
                               tiles, n_tiles, p.offsets, Y, p.d, p.E, p.f, p.fs);
        return hipGetLastError();
    }
#endif
    if (p.aq) {
#define FGS_DNF(B, D)                                                                                          \
    hipLaunchKernelGGL((down_gemm_f8_kernel<B, D>), grid, block, D ? 0 : kGemmLds, p.stream, p.hq, p.hs, p.ldh,     \
                       p.W.w_down, p.W.s_down, p.W.ws_down, p.W.ss_down, tiles, n_tiles, p.offsets, Y, p.d, p.E, \
                       p.f, p.fs)
        const bool blk = (p.flags & MOE_FLAG_FP8_BLOCK128) != 0;
        if (f8_dma(p)) { if (blk) FGS_DNF(true, true); else FGS_DNF(false, true); }
        else { if (blk) FGS_DNF(true, false); else FGS_DNF(false, false); }
#undef FGS_DNF
        return hipGetLastError();
    }
#if FGS_DOWN_PERSIST
    // the persistent kernel: bf16 or per-channel E4M3 weights, whole 256-column
    // blocks, 32-bit offsets into H and into one expert's matrix
    const long h_bytes = ((long)p.N * p.k + p.N) * p.ldh * 2;
    const bool w8 = p.wdt == MOE_DTYPE_FP8_E4M3 && !(p.flags & MOE_FLAG_FP8_BLOCK128);
    // 128 x 128 block scales: both output blocks' K-block scales of an item in one 64-lane DMA
    const bool w8b = p.wdt == MOE_DTYPE_FP8_E4M3 && (p.flags & MOE_FLAG_FP8_BLOCK128) && p.f <= 4096 &&
                     p.fs <= 4096 && p.d % kBN == 0 && h_bytes < (1L << 32);
    if (w8b) {
        int cus = 0;
        hipError_t e = cu_count(&cus);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((down_gemm_persist_kernel<true, true>), dim3(cus), block, 0, p.stream, p.H, p.ldh,
                           (const uint8_t *)p.W.w_down, p.W.s_down, (const uint8_t *)p.W.ws_down, p.W.ss_down,
                           tiles, n_tiles, p.offsets, Y, p.d, p.E, p.f, p.fs);
        return hipGetLastError();
    }
    if ((p.wdt == MOE_DTYPE_BF16 || w8) && p.d % kBN == 0 && p.f % kBK == 0 && p.fs % kBK == 0 &&
        h_bytes < (1L << 32) &&
        (long)p.d * (p.f > p.fs ? p.f : p.fs) * 2 < (1L << 32)) {
        int cus = 0;
        hipError_t e = cu_count(&cus);
        if (e != hipSuccess) return e;
#if FGS_DOWN_WIDE
        // 256 x 256 items (the gate/up's 256-row tile list) where the routed experts
        // average at least 256 rows; one MI355X, d = 2560, E = 384, top-6: all-hot
        // probe down 433 -> 403 us, Zipf 458 -> 443, but prefill (about 150 rows per
        // expert) 315 -> 319, so it keeps the 128-row items
        if (p.bm == kGemmBMWide && (long)p.N * p.k >= 256L * p.E) {
            if (w8)
                hipLaunchKernelGGL(down_gemm_wide_persist_kernel<true>, dim3(cus), dim3(1024), 0, p.stream, p.H,
                                   p.ldh, (const uint8_t *)p.W.w_down, p.W.s_down, (const uint8_t *)p.W.ws_down,
                                   p.W.ss_down, p.tiles, p.n_tiles, p.offsets, Y, p.d, p.E, p.f, p.fs);
            else
                hipLaunchKernelGGL(down_gemm_wide_persist_kernel<false>, dim3(cus), dim3(1024), 0, p.stream, p.H,
                                   p.ldh, (const uint8_t *)p.W.w_down, p.W.s_down, (const uint8_t *)p.W.ws_down,
                                   p.W.ss_down, p.tiles, p.n_tiles, p.offsets, Y, p.d, p.E, p.f, p.fs);
            return hipGetLastError();
        }
#endif
        if (w8)
            hipLaunchKernelGGL((down_gemm_persist_kernel<true, false>), dim3(cus), block, 0, p.stream, p.H, p.ldh,
                               (const uint8_t *)p.W.w_down, p.W.s_down, (const uint8_t *)p.W.ws_down, p.W.ss_down,
                               tiles, n_tiles, p.offsets, Y, p.d, p.E, p.f, p.fs);
        else
            hipLaunchKernelGGL((down_gemm_persist_kernel<false, false>), dim3(cus), block, 0, p.stream, p.H, p.ldh,
                               (const uint8_t *)p.W.w_down, p.W.s_down, (const uint8_t *)p.W.ws_down, p.W.ss_down,
                               tiles, n_tiles, p.offsets, Y, p.d, p.E, p.f, p.fs);
        return hipGetLastError();
    }
#endif
#define FGS_DNG(WM)                                                                                       \
    hipLaunchKernelGGL((down_gemm_kernel<WM>), grid, block,                                                       \
                       (WM == kWBf16 || WM == kWFp8Row || WM == kWFp8BlkDma) ? 0 : kGemmLds, p.stream, p.H,             \
                       p.ldh, p.W.w_down, p.W.s_down,                                                                \
                       p.W.ws_down, p.W.ss_down, tiles, n_tiles, p.offsets, Y, p.d, p.E, p.f, p.fs)
    if (p.wdt != MOE_DTYPE_FP8_E4M3) FGS_DNG(kWBf16);
    else if (p.flags & MOE_FLAG_FP8_BLOCK128) {
        if (w8b_dma(p)) FGS_DNG(kWFp8BlkDma);
        else FGS_DNG(kWFp8Blk);
    }
    else FGS_DNG(kWFp8Row);
#undef FGS_DNG
    return hipGetLastError();
}

}  // namespace fgs
