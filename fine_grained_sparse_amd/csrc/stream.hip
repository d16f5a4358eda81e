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
// those rows in registers (coalesced non-temporal loads: consecutive lanes
// read consecutive chunks of a row), and dot them against that expert's token
// rows, which each lane reads straight from L2 with the next token's row in
// flight (no LDS, no barrier).  Cross-lane sums use a butterfly
// reduce-scatter: at each halving step a lane keeps half of its partial sums
// and trades the other half with its partner, so V sums over 64 lanes cost
// about V shuffles.
//
// Work list: one tile per non-empty group (routed experts, and the shared
// expert as group E with all N tokens), written by the dispatch scan.
//
// FP8 weights are decoded to bf16 (exact) before the dot products: in the
// gate/up kernel per token (a wave holds twice as many FP8 rows, too many to
// keep converted), in the down kernel once after the loads land.  Scales
// ("Inside Kolibri 1", section "The FP8 path is explicitly mixed precision"):
// a per-output-channel scale is applied to the finished dot product; with
// 128 x 128 block scales every 8-element partial product is scaled by its own
// block's scale before the cross-lane sum.  With 1 x 128 activation
// quantisation (AQ) the token rows arrive as E4M3 codes plus one FP32 scale
// per 128 values; codes are exact in bf16, so the same dot products run on
// them and each 8-element partial is multiplied by its group's activation
// scale (times the weight block scale).  The gate/up kernel then writes FP32
// hidden values, which are quantised in 1 x 128 groups before the down
// kernel reads them.
#include "moe_common.h"
#include "moe_plan.h"

namespace fgs {

template <bool FP8> struct WChunk;            // 8 weights of one row
template <> struct WChunk<false> { typedef uint4 T; };
template <> struct WChunk<true> { typedef uint2 T; };

template <bool FP8>
__device__ __forceinline__ typename WChunk<FP8>::T load_chunk(const void *base, size_t elem_off) {
    if constexpr (FP8) return ld_stream8((const uint8_t *)base + elem_off);
    else return ld_stream16((const uint16_t *)base + elem_off);
}
// 8 weights as bfloat16: the E4M3 -> bf16 conversion is exact
// (v_cvt_scalef32_pk_bf16_fp8 with scale 1)
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_bf16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
template <bool FP8>
__device__ __forceinline__ uint4 chunk_bf16(const typename WChunk<FP8>::T &w) {
    if constexpr (FP8)
        return make_uint4(e4m3x2_bf16x2<false>(w.x), e4m3x2_bf16x2<true>(w.x), e4m3x2_bf16x2<false>(w.y),
                          e4m3x2_bf16x2<true>(w.y));
    else
        return w;
}

// weight modes: bfloat16, FP8 with per-channel scales, FP8 with 128x128 block scales
enum { kWBf16 = 0, kWFp8Row = 1, kWFp8Blk = 2 };

// 8 activations -> bfloat16 x 8 (FP32 x is rounded to nearest even)
__device__ __forceinline__ uint4 load_x8(const void *x, int xdt, size_t elem_off) {
    if (xdt == MOE_DTYPE_BF16) return *reinterpret_cast<const uint4 *>((const uint16_t *)x + elem_off);
    const float4 *p = reinterpret_cast<const float4 *>((const float *)x + elem_off);
    float4 a = p[0], b = p[1];
    return make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y), pack_bf16x2(b.z, b.w));
}

// H columns per wave: 2 with bf16 weights, 4 with FP8 weights (rows of
// E4M3 codes are half the bytes, so a wave holds twice as many to keep as many
// bytes in flight)
template <bool FP8> constexpr int gu_cols_per_wave() { return FP8 ? 4 : 2; }
template <bool FP8> constexpr int gu_cols_per_block() { return 4 * gu_cols_per_wave<FP8>(); }

template <int CPL>
__device__ __forceinline__ void load_x_row(uint4 (&xv)[CPL], const void *x, int xdt, int t, int d, int lane,
                                           int nch) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int ch = lane + 64 * i;
        xv[i] = ch < nch ? load_x8(x, xdt, (size_t)t * d + (size_t)ch * 8) : make_uint4(0, 0, 0, 0);
    }
}

// AQ token row: 8 E4M3 codes per chunk and the scale of the chunk's 128-group
// (lanes past the row end get zero codes and a valid scale)
template <int CPL>
__device__ __forceinline__ void load_xq_row(uint2 (&xv)[CPL], float (&sv)[CPL], const uint8_t *xq, const float *xs,
                                            int t, int d, int lane, int nch) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int ch = lane + 64 * i;
        const bool ok = ch < nch;
        xv[i] = ok ? *reinterpret_cast<const uint2 *>(xq + (size_t)t * d + (size_t)ch * 8) : make_uint2(0, 0);
        sv[i] = xs[(size_t)t * (d / 128) + ((ok ? ch : 0) >> 4)];
    }
}

// grid: (ceil(max(f, fs) / gu_cols_per_block) column blocks, tile list capacity); block 256.
// Column blocks run fastest, so the workgroups in flight together cover a few
// experts' matrices completely (page and DRAM-row locality).  No LDS and no
// barrier: each lane reads its slice of a token row straight from L2, with
// the next token's row in flight while the current one is reduced.
// AQ: x is the E4M3 codes [N][d] with scales xs [N][d/128]; the output goes to
// the FP32 buffer Hf instead of H.
template <int CPL, int WM, bool AQ>
__global__ __launch_bounds__(256) void gate_up_stream_kernel(
    const void *__restrict__ x, int xdt, const float *__restrict__ xs, const void *__restrict__ wg,
    const void *__restrict__ wu, const float *__restrict__ sg, const float *__restrict__ su,
    const void *__restrict__ wsg, const void *__restrict__ wsu, const float *__restrict__ ssg,
    const float *__restrict__ ssu, const int32_t *__restrict__ tiles, const int32_t *__restrict__ n_tiles,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ por, uint16_t *__restrict__ H,
    float *__restrict__ Hf, int ldh, int d, int E, int k, int f, int fs, int bm) {
    constexpr bool FP8 = WM != kWBf16, BLK = WM == kWFp8Blk;
    constexpr int RP = gu_cols_per_wave<FP8>(), NR = 2 * RP;   // H columns, weight rows per wave
    const int u = blockIdx.y;
    if (u >= *n_tiles) return;
    const int g = tiles[2 * u], m0 = tiles[2 * u + 1];
    const bool shared = g == E;
    const int fg = shared ? fs : f;
    if ((int)blockIdx.x * gu_cols_per_block<FP8>() >= fg) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c0 = blockIdx.x * gu_cols_per_block<FP8>() + wave * RP;
    const int nch = d / 8;

    // this wave's NR weight rows: gate c0 .. c0+RP-1, then up c0 .. c0+RP-1 (issued first)
    const void *gbase = shared ? wsg : wg;
    const void *ubase = shared ? wsu : wu;
    const size_t rbase = shared ? 0 : (size_t)g * f;
    // lanes past the row end read chunk 0 again (finite weights) and are
    // multiplied by a zero activation chunk; no select on loaded values, so
    // nothing waits for these loads before the token rows are requested
    typename WChunk<FP8>::T wr[NR][CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int ch = lane + 64 * i;
        const int chc = ch < nch ? ch : 0;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const void *b = r < RP ? gbase : ubase;
            wr[r][i] = load_chunk<FP8>(b, (rbase + c0 + (r % RP)) * (size_t)d + (size_t)chc * 8);
        }
    }
    // block scales: chunk ch covers input columns [8ch, 8ch+8), in K block ch/16;
    // rows c0 .. c0+RP-1 share one output block
    float bsc[2][CPL];
    if (BLK) {
        const int nkb = d / 128;
        const size_t sb = ((shared ? 0 : (size_t)g * (f / 128)) + c0 / 128) * nkb;
        const float *gs = (shared ? ssg : sg) + sb, *us = (shared ? ssu : su) + sb;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int ch = lane + 64 * i;
            const int kb = (ch < nch ? ch : 0) >> 4;
            bsc[0][i] = gs[kb];
            bsc[1][i] = us[kb];
        }
    }

    const int gstart = offsets[g];
    const int row0 = gstart + m0, m = min(bm, offsets[g + 1] - row0);
    // lane j holds the token of row row0 + j (m <= 64)
    int tok = 0;
    if (lane < m) tok = shared ? (m0 + lane) : por[row0 + lane] / k;

    // after the reduction the value index of a lane is its top log2(NR) bits:
    // gate column c0 + j sits on the lanes with bit 5 clear and value j, the
    // matching up column on the same lanes with bit 5 set
    constexpr int kLb = 6 - (NR == 8 ? 3 : 2);   // lowest value bit
    const int r_out = (lane >> kLb) & (RP - 1);
    float gsc = 1.f, usc = 1.f;
    if (WM == kWFp8Row) {
        const float *gs = shared ? ssg : sg + (size_t)g * f;
        const float *us = shared ? ssu : su + (size_t)g * f;
        gsc = gs[c0 + r_out];
        usc = us[c0 + r_out];
    }

    uint4 xa[CPL], xb[CPL];
    uint2 qa[CPL], qb[CPL];
    float sa[CPL], sb[CPL];
    if (AQ) load_xq_row<CPL>(qa, sa, (const uint8_t *)x, xs, __shfl(tok, 0, kWave), d, lane, nch);
    else load_x_row<CPL>(xa, x, xdt, __shfl(tok, 0, kWave), d, lane, nch);
    // bf16 rows are used as loaded; E4M3 rows are converted per token (held
    // converted they would need twice the registers)
    for (int t = 0; t < m; ++t) {
        if (t + 1 < m) {
            if (AQ) load_xq_row<CPL>(qb, sb, (const uint8_t *)x, xs, __shfl(tok, t + 1, kWave), d, lane, nch);
            else load_x_row<CPL>(xb, x, xdt, __shfl(tok, t + 1, kWave), d, lane, nch);
        }
        float acc[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) acc[r] = 0.f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const uint4 xc = AQ ? chunk_bf16<true>(qa[i]) : xa[i];
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const int gu = r / RP;   // 0 gate, 1 up
                typename WChunk<FP8>::T raw = wr[r][i];
                if constexpr (FP8) {
                    // an empty asm makes the codes opaque per token, so the
                    // conversion is not hoisted out of the token loop (which
                    // would hold every row converted: twice the registers)
                    asm volatile("" : "+v"(raw.x), "+v"(raw.y));
                }
                const uint4 wv = chunk_bf16<FP8>(raw);
                if (AQ) acc[r] = fmaf(dot8_bf16(wv, xc, 0.f), BLK ? sa[i] * bsc[gu][i] : sa[i], acc[r]);
                else if (BLK) acc[r] = fmaf(dot8_bf16(wv, xc, 0.f), bsc[gu][i], acc[r]);
                else acc[r] = dot8_bf16(wv, xc, acc[r]);
            }
        }
        butterfly_reduce<NR>(acc);
        const float upv = __shfl_xor(acc[0], 32, kWave);
        if ((lane & (32 | ((1 << kLb) - 1))) == 0) {  // one lane per gate column
            const float hv = silu(acc[0] * gsc) * (upv * usc);
            if (AQ) Hf[(size_t)(row0 + t) * ldh + c0 + r_out] = hv;
            else H[(size_t)(row0 + t) * ldh + c0 + r_out] = (uint16_t)f32_to_bf16_rne(hv);
        }
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            if (AQ) { qa[i] = qb[i]; sa[i] = sb[i]; }
            else xa[i] = xb[i];
        }
    }
}

// output rows per wave: 4 KB of weights per wave in both formats (4 bf16 rows
// of 512, 8 E4M3 rows).  Measured at decode size, 2, 8 and 16 bf16 rows and
// 4 or 16 FP8 rows are slower: fewer, larger waves leave more of the machine
// idle behind each one's index loads and at the grid's tail.  32 rows per
// workgroup in both formats: eight bf16 waves (decode N=32: 62.8 against
// 64.1 us with four waves, 64.8 with sixteen), four FP8 waves (eight: 37.7
// against 37.2 us, with 1 x 128 activations 44.2 against 41.3).
template <bool FP8> constexpr int dn_waves() { return FP8 ? 4 : 8; }
template <bool FP8> constexpr int dn_rows_per_wave() { return FP8 ? 8 : 4; }
template <bool FP8> constexpr int dn_rows_per_block() { return dn_waves<FP8>() * dn_rows_per_wave<FP8>(); }

// grid: (d / dn_rows_per_block, tile list capacity); block 64 * dn_waves.  Needs f, fs <= 512.
// AQ: H is the E4M3 codes [rows][ldh] (as bytes) with scales hs [rows][ldh/128].
template <int WM, bool AQ>
__global__ __launch_bounds__(64 * dn_waves<WM != kWBf16>()) void down_stream_kernel(
    const uint16_t *__restrict__ H, const float *__restrict__ hs, int ldh, const void *__restrict__ wd,
    const float *__restrict__ sd,
    const void *__restrict__ wsd, const float *__restrict__ ssd, const int32_t *__restrict__ tiles,
    const int32_t *__restrict__ n_tiles, const int32_t *__restrict__ offsets, float *__restrict__ Y, int d, int E,
    int f, int fs, int bm) {
    constexpr bool FP8 = WM != kWBf16, BLK = WM == kWFp8Blk;
    constexpr int kDnRW = dn_rows_per_wave<FP8>();
    const int u = blockIdx.y;
    if (u >= *n_tiles) return;
    const int g = tiles[2 * u], m0 = tiles[2 * u + 1];
    const bool shared = g == E;
    const int fg = shared ? fs : f;
    const int nch = fg / 8;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int o0 = blockIdx.x * dn_rows_per_block<FP8>() + wave * kDnRW;

    const void *base = shared ? wsd : wd;
    const size_t obase = shared ? 0 : (size_t)g * d;
    const bool ok = lane < nch;  // masked lanes: chunk 0 again, times a zero H chunk
    typename WChunk<FP8>::T wr[kDnRW];
#pragma unroll
    for (int r = 0; r < kDnRW; ++r)
        wr[r] = load_chunk<FP8>(base, (obase + o0 + r) * (size_t)fg + (size_t)(ok ? lane : 0) * 8);
    const int myrow = butterfly_index<kDnRW>(lane);
    float scl = 1.f;
    if (WM == kWFp8Row) scl = shared ? ssd[o0 + myrow] : sd[obase + o0 + myrow];
    // block scales: the wave's 8 rows lie in output block o0/128; lane's chunk
    // covers inputs [8 lane, 8 lane + 8), in K block lane/16
    float lsc = 1.f;
    if (BLK) {
        const int nkb = fg / 128;
        const float *sp = shared ? ssd : sd + (size_t)g * (d / 128) * nkb;
        lsc = sp[(size_t)(o0 / 128) * nkb + ((ok ? lane : 0) >> 4)];
    }

    const int row0 = offsets[g] + m0, m = min(bm, offsets[g + 1] - row0);
    const uint16_t *hp = H + (size_t)row0 * ldh + (size_t)(ok ? lane : 0) * 8;
    const uint8_t *qp = (const uint8_t *)H + (size_t)row0 * ldh + (size_t)(ok ? lane : 0) * 8;
    const float *sp = AQ ? hs + (size_t)row0 * (ldh / 128) + ((ok ? lane : 0) >> 4) : nullptr;
    uint4 ha = make_uint4(0, 0, 0, 0);
    float hsa = 0.f;
    if (AQ) {
        if (ok) ha = chunk_bf16<true>(*reinterpret_cast<const uint2 *>(qp));
        hsa = sp[0];
    } else if (ok) {
        ha = *reinterpret_cast<const uint4 *>(hp);
    }
    uint4 w[kDnRW];
#pragma unroll
    for (int r = 0; r < kDnRW; ++r) w[r] = chunk_bf16<FP8>(wr[r]);
    for (int t = 0; t < m; ++t) {
        uint4 hb = make_uint4(0, 0, 0, 0);
        uint2 hqb = make_uint2(0, 0);
        float hsb = 0.f;
        if (t + 1 < m) {
            if (AQ) {
                if (ok) hqb = *reinterpret_cast<const uint2 *>(qp + (size_t)(t + 1) * ldh);
                hsb = sp[(size_t)(t + 1) * (ldh / 128)];
            } else if (ok) {
                hb = *reinterpret_cast<const uint4 *>(hp + (size_t)(t + 1) * ldh);
            }
        }
        const float psc = AQ ? (BLK ? hsa * lsc : hsa) : lsc;
        float p[kDnRW];
#pragma unroll
        for (int r = 0; r < kDnRW; ++r) {
            p[r] = dot8_bf16(w[r], ha, 0.f);
            if (AQ || BLK) p[r] *= psc;
        }
        butterfly_reduce<kDnRW>(p);
        if ((lane & (64 / kDnRW - 1)) == 0) Y[(size_t)(row0 + t) * d + o0 + myrow] = p[0] * scl;
        if (AQ) { ha = chunk_bf16<true>(hqb); hsa = hsb; }
        else ha = hb;
    }
}

hipError_t launch_gate_up(const Plan &p) {
    const int fmax = p.f > p.fs ? p.f : p.fs;
    const int cb = p.wdt == MOE_DTYPE_FP8_E4M3 ? gu_cols_per_block<true>() : gu_cols_per_block<false>();
    dim3 grid((fmax + cb - 1) / cb, p.max_tiles), block(256);
    const size_t lds = 0;
    const int cpl = (p.d / 8 + 63) / 64;
    const int wm = p.wdt != MOE_DTYPE_FP8_E4M3 ? kWBf16 : (p.flags & MOE_FLAG_FP8_BLOCK128) ? kWFp8Blk : kWFp8Row;
    if (p.aq) {  // the experts' input in 1 x 128 groups
        hipError_t e = launch_quant_groups(p.x, 1, p.d, p.N, p.d, p.xq, p.d, p.xs, p.d / 128, p.stream);
        if (e != hipSuccess) return e;
    }
    const void *xin = p.aq ? (const void *)p.xq : p.x;
#define FGS_GU(C, WM, AQ)                                                                                        \
    hipLaunchKernelGGL((gate_up_stream_kernel<C, WM, AQ>), grid, block, lds, p.stream, xin, p.xdt, p.xs,        \
                       p.W.w_gate, p.W.w_up, p.W.s_gate, p.W.s_up, p.W.ws_gate, p.W.ws_up, p.W.ss_gate, p.W.ss_up, \
                       p.tiles, p.n_tiles, p.offsets, p.por, p.H, p.hf, p.ldh, p.d, p.E, p.k, p.f, p.fs, p.bm)
#define FGS_GU_C(C)                                                                  \
    do {                                                                             \
        if (wm == kWFp8Blk) { if (p.aq) FGS_GU(C, kWFp8Blk, true); else FGS_GU(C, kWFp8Blk, false); } \
        else if (wm == kWFp8Row) { if (p.aq) FGS_GU(C, kWFp8Row, true); else FGS_GU(C, kWFp8Row, false); } \
        else FGS_GU(C, kWBf16, false);                                               \
    } while (0)
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
    const int rb = p.wdt == MOE_DTYPE_FP8_E4M3 ? dn_rows_per_block<true>() : dn_rows_per_block<false>();
    const int waves = p.wdt == MOE_DTYPE_FP8_E4M3 ? dn_waves<true>() : dn_waves<false>();
    dim3 grid(p.d / rb, p.max_tiles), block(64 * waves);
    const long rows = (long)p.N * p.k + p.N;
    if (p.aq) {  // hidden activations in 1 x 128 groups (every row of H, routed and shared)
        hipError_t e = launch_quant_groups(p.hf, 0, p.ldh, rows, p.ldh, p.hq, p.ldh, p.hs, p.ldh / 128, p.stream);
        if (e != hipSuccess) return e;
    }
    const uint16_t *hin = p.aq ? (const uint16_t *)p.hq : p.H;
#define FGS_DN(WM, AQ)                                                                                         \
    hipLaunchKernelGGL((down_stream_kernel<WM, AQ>), grid, block, 0, p.stream, hin, p.hs, p.ldh, p.W.w_down,    \
                       p.W.s_down, p.W.ws_down, p.W.ss_down, p.tiles, p.n_tiles, p.offsets, p.Y, p.d, p.E, p.f, \
                       p.fs, p.bm)
    if (p.wdt != MOE_DTYPE_FP8_E4M3) FGS_DN(kWBf16, false);
    else if (p.flags & MOE_FLAG_FP8_BLOCK128) { if (p.aq) FGS_DN(kWFp8Blk, true); else FGS_DN(kWFp8Blk, false); }
    else { if (p.aq) FGS_DN(kWFp8Row, true); else FGS_DN(kWFp8Row, false); }
#undef FGS_DN
    return hipGetLastError();
}

}  // namespace fgs
