"""CPU oracle for the fine-grained MoE feed-forward layer (test infrastructure).

This is test infrastructure, not a product path: only the tests, the smoke
check and the benchmark's CPU-baseline leg may import it.  It shares no code
with the HIP library and never calls it.

It is a plain, slow statement of what the layer computes, in float64 numpy,
step by step in the order the pages give:

  * "Inside Kolibri 1: Hybrid RNoPE Attention, Sparse MoE, and FP8 Serving"
    (flozi.net), section "Routing: selection bias and mixture weights are
    separate": a router maps the flattened tokens [N, 2560] to FP32 logits
    [N, 384]; a learned expert-correction bias is added to the logits and the
    six largest ids are selected (rule step 1); the *unbiased* logits of those
    ids go through a sigmoid and are used as mixture weights, with no
    renormalisation to sum one (rule step 2).  Routing is token-choice top-k
    with no per-expert capacity.  Each routed or shared expert is a SwiGLU MLP:
    SiLU(gate) x up from two 2560 -> 512 projections, then 512 -> 2560.
  * same page, section "The released stack": every MoE evaluates one shared
    expert besides the six routed ones.
  * same page, section "The FP8 path is explicitly mixed precision": FP8 E4M3
    weights carry FP32 scales that must be used exactly (never rounded to
    powers of two); the router logits stay FP32.
  * "Kolibri 1 Deep Dive" (abrarakhunji.com), "Mathematical Routing & Load
    Balancing Formulation": the layer output is the gate-weighted sum of the
    selected experts' SwiGLU outputs (its residual term belongs to the caller).

Readings taken where the pages are silent (each is listed in the design notes):
  * logits: the FP32 logit is the float64 dot product rounded once to float32;
    the selection score is the float32 sum of that logit and the float32 bias;
  * ties in the selection score go to the lower expert id; the selected ids
    are stored in ascending order (slot j = j-th smallest selected id);
  * the shared expert has coefficient 1 and no gate; no expert linear has a
    bias term; no routed scaling factor (1.0);
  * FP8 is OCP E4M3FN (bias 7, max 448, NaN at S.1111.111, no infinities) and
    a dequantised weight is code value x scale;
  * everything after the logits is computed in float64; the output is rounded
    once to the output dtype (float32 or bfloat16, round to nearest even);
  * optional 1 x 128 activation quantisation (the FP8 section's dynamic
    groups): per group scale = float32(amax / 448), codes = E4M3 nearest-even
    of float32(v / scale); applied to x and to each expert's hidden
    activations (rounded to float32 first), never to the router's input.

Parity status: every function below is pinned by the CPU tests (brute-force
selection, library sorts and decoders, dense compute-every-expert formulation,
closed-form worked example, page arithmetic).  There is no worked numerical
example of the layer on the pages, so the output values themselves are pinned
only through those reductions.
"""
from __future__ import annotations

import math
from itertools import combinations
from typing import Dict, Optional, Sequence

import numpy as np

__all__ = [
    "decode_bf16", "decode_e4m3fn", "dequant_weight", "router_logits",
    "select_topk", "mixture_weights", "dispatch", "swiglu_expert",
    "combine", "moe_forward", "token_outputs", "brute_force_topk",
    "expert_param_counts", "round_to_bf16_bits", "rms_norm", "block_forward",
    "encode_e4m3fn", "quantize_groups", "dequantize_groups", "fake_quant",
]


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------

def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64.

    A bfloat16 is the upper half of an IEEE binary32: shifting the 16 bits to
    the top of a 32-bit word gives the same number as a float32, exactly.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3FN codes (uint8) -> float64, from the format's fields.

    1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
    is subnormal (m/8 * 2^-6); the all-ones exponent with mantissa 111 is NaN;
    there is no infinity, so S.1111.000..110 are ordinary numbers up to 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = (m / 8.0) * 2.0 ** (1 - 7)
    v = np.where(e == 0, subnormal, normal) * sign
    v = np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, v)
    return v


def round_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 bits, round to nearest, ties to even (via float32).

    Used only to express the layer output in a bfloat16 output dtype.  The
    float64 value is first rounded to float32 (exact for every value that is
    not a tie at float32 precision), then the 16 low bits are rounded off.
    """
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return u.astype(np.uint16)


def dequant_weight(w: np.ndarray, scale: Optional[np.ndarray], w_dtype: str) -> np.ndarray:
    """Stored expert weight -> float64 [out, in].

    bfloat16: exact widening.  FP8: decoded code times its FP32 scale, used as
    stored (never rounded to a power of two).  `scale` holds one value per
    output channel ([..., out]) or one per block of the matrix ([..., out/b,
    in/b], the released checkpoint's 128 x 128 blocks, "Inside Kolibri 1",
    section "The FP8 path is explicitly mixed precision").
    """
    if w_dtype == "bf16":
        return decode_bf16(w)
    if w_dtype == "fp8":
        q = decode_e4m3fn(w)
        s = np.asarray(scale, dtype=np.float32).astype(np.float64)
        if s.ndim == q.ndim:
            # one scale per (out/b, in/b) block: expand each scale over its block
            bo, bi = q.shape[-2] // s.shape[-2], q.shape[-1] // s.shape[-1]
            return q * np.repeat(np.repeat(s, bo, axis=-2), bi, axis=-1)
        return q * s[..., :, None]
    raise ValueError(w_dtype)


E4M3_MAX = 448.0


def encode_e4m3fn(r: np.ndarray) -> np.ndarray:
    """float32 values with |r| <= 448 -> OCP E4M3FN codes, nearest value, ties to even.

    The non-negative finite values are the codes 0x00..0x7E in increasing
    order; each |r| goes to the closer of its two neighbours in that list, and
    an exact midpoint to the code whose mantissa (lowest bit) is even.  The
    sign bit is copied, so -0.0 gives 0x80.
    """
    r = np.asarray(r, dtype=np.float32)
    if np.any(np.abs(r) > E4M3_MAX) or not np.all(np.isfinite(r)):
        raise ValueError("encode_e4m3fn needs finite |r| <= 448")
    table = decode_e4m3fn(np.arange(0x7F, dtype=np.uint8))
    a = np.abs(r.astype(np.float64))
    hi = np.searchsorted(table, a, side="left")      # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - table[lo], table[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return code | np.where(np.signbit(r), 0x80, 0).astype(np.uint8)


def quantize_groups(v32: np.ndarray, group: int = 128):
    """Dynamic FP8 quantisation of activations in 1 x `group` groups.

    "Inside Kolibri 1", section "The FP8 path is explicitly mixed precision":
    activations are quantised on the fly in groups of 1 x 128.  Per group of
    `group` consecutive values of a row: scale = float32(amax / 448) (1 for an
    all-zero group), code = E4M3 of float32(v / scale) clamped to +-448 (the
    clamp only catches the amax element when the division rounds above 448).
    Every step is a float32 operation, as the kernels do it.  Returns codes
    [rows, cols] uint8 and scales [rows, cols/group] float32.
    """
    v = np.asarray(v32, dtype=np.float32)
    rows, cols = v.shape
    if cols % group:
        raise ValueError("cols must be a multiple of the group size")
    vg = v.reshape(rows, cols // group, group)
    amax = np.abs(vg).max(axis=2)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    r = (vg / scale[..., None]).astype(np.float32)
    r = np.clip(r, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return encode_e4m3fn(r).reshape(rows, cols), scale


def dequantize_groups(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """codes [rows, cols] times their group's scale, float64 (exact)."""
    q = decode_e4m3fn(codes)
    g = q.shape[1] // scale.shape[1]
    return q * np.repeat(np.asarray(scale, dtype=np.float32).astype(np.float64), g, axis=1)


def fake_quant(v: np.ndarray) -> np.ndarray:
    """Rows rounded to float32, quantised in 1 x 128 groups and decoded again (float64)."""
    return dequantize_groups(*quantize_groups(np.asarray(v, dtype=np.float64).astype(np.float32)))


def _x_to_f64(x: np.ndarray) -> np.ndarray:
    if x.dtype == np.uint16:
        return decode_bf16(x)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# routing
# --------------------------------------------------------------------------

def router_logits(x64: np.ndarray, router_w: np.ndarray) -> np.ndarray:
    """FP32 logits h[t, e] = sum_i x[t, i] * W_r[e, i].

    The sum is taken in float64 and rounded once to float32 (the pages keep the
    router's output logits in FP32).
    """
    w64 = np.asarray(router_w, dtype=np.float32).astype(np.float64)
    return (x64 @ w64.T).astype(np.float32)


def select_topk(h32: np.ndarray, bias: np.ndarray, k: int):
    """Rule step 1: add the correction bias, keep the k best expert ids.

    Score s = float32(h + b).  Order is (s descending, id ascending), so equal
    scores go to the lower id.  Returns (ids [N, k] int32 in ascending id
    order, gap [N] float64 = s of the k-th pick minus s of the (k+1)-th, +inf
    when every expert is selected, s [N, E] float32).
    """
    h32 = np.asarray(h32, dtype=np.float32)
    b32 = np.asarray(bias, dtype=np.float32)
    s = (h32 + b32[None, :]).astype(np.float32)
    n, n_exp = s.shape
    if not 1 <= k <= n_exp:
        raise ValueError("need 1 <= k <= n_experts")
    # a stable sort of -s keeps lower ids first among equal scores
    order = np.argsort(-s.astype(np.float64), axis=1, kind="stable")
    chosen = order[:, :k]
    ids = np.sort(chosen, axis=1).astype(np.int32)
    rows = np.arange(n)
    s_k = s[rows, order[:, k - 1]].astype(np.float64)
    if k < n_exp:
        gap = s_k - s[rows, order[:, k]].astype(np.float64)
    else:
        gap = np.full(n, np.inf)
    return ids, gap, s


def mixture_weights(h32: np.ndarray, ids: np.ndarray, renormalize: bool = False) -> np.ndarray:
    """Rule step 2: sigmoid of the *unbiased* logits of the chosen ids.

    w[t, j] = 1 / (1 + exp(-h[t, ids[t, j]])), float64, not renormalised.

    With `renormalize` the weights follow the other page's gate instead ("Kolibri
    1 Deep Dive", "Mathematical Routing & Load Balancing Formulation"): the
    exponentials of the selected logits divided by their sum over the selected
    set, so they sum to one.  Still computed from the unbiased logits.
    """
    h = np.take_along_axis(np.asarray(h32, dtype=np.float32), ids.astype(np.int64), axis=1)
    h = h.astype(np.float64)
    if renormalize:
        z = np.exp(h - h.max(axis=1, keepdims=True))
        return z / z.sum(axis=1, keepdims=True)
    return 1.0 / (1.0 + np.exp(-h))


def dispatch(ids: np.ndarray, n_experts: int):
    """Token-choice dispatch with no capacity: a stable counting sort.

    Pairs are (token t, slot j), flattened as t*k + j.  Returns
      counts [E]        pairs routed to each expert (0 is allowed),
      offsets [E+1]     exclusive prefix sum of counts,
      pair_of_row [N*k] the pair stored at each row of the expert-sorted buffer,
      row_of_pair [N*k] the inverse map.
    Within an expert, rows follow increasing token index (slot order breaks no
    ties, since a token selects an expert at most once).
    """
    ids = np.asarray(ids)
    n, k = ids.shape
    counts = np.zeros(n_experts, dtype=np.int64)
    for t in range(n):
        for j in range(k):
            counts[ids[t, j]] += 1
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    for e in range(n_experts):
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = np.zeros(n_experts, dtype=np.int64)
    pair_of_row = np.empty(n * k, dtype=np.int64)
    row_of_pair = np.empty(n * k, dtype=np.int64)
    for t in range(n):
        for j in range(k):
            e = ids[t, j]
            p = offsets[e] + cursor[e]
            cursor[e] += 1
            pair_of_row[p] = t * k + j
            row_of_pair[t * k + j] = p
    return (counts.astype(np.int32), offsets.astype(np.int32),
            pair_of_row.astype(np.int32), row_of_pair.astype(np.int32))


# --------------------------------------------------------------------------
# experts and combine
# --------------------------------------------------------------------------

def _sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


def swiglu_expert(x64: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray,
                  act_quant: bool = False) -> np.ndarray:
    """One SwiGLU expert on rows of x: W_d (SiLU(W_g x) * (W_u x)).

    x64 [m, d]; wg, wu [f, d]; wd [d, f]; all float64; no bias terms.
    SiLU(z) = z * sigmoid(z).  With `act_quant` the hidden activations, the
    down projection's input, are rounded to float32 and quantised in 1 x 128
    groups first (the caller quantises x the same way).
    """
    a = x64 @ wg.T
    u = x64 @ wu.T
    hidden = a * _sigmoid(a) * u
    if act_quant:
        hidden = fake_quant(hidden)
    return hidden @ wd.T


def combine(ys: np.ndarray, y_rows: np.ndarray, w: np.ndarray, row_of_pair: np.ndarray) -> np.ndarray:
    """out[t] = ys[t] + w[t,0] Y[row(t,0)] + ... + w[t,k-1] Y[row(t,k-1)], left to right."""
    n, k = w.shape
    out = ys.copy()
    for j in range(k):
        out = out + w[:, j:j + 1] * y_rows[row_of_pair.reshape(n, k)[:, j]]
    return out


def _expert_weights(inp: Dict[str, np.ndarray], e: int, w_dtype: str):
    sc = (lambda key: inp.get(key)[e] if inp.get(key) is not None else None)
    wg = dequant_weight(inp["w_gate"][e], sc("s_gate"), w_dtype)
    wu = dequant_weight(inp["w_up"][e], sc("s_up"), w_dtype)
    wd = dequant_weight(inp["w_down"][e], sc("s_down"), w_dtype)
    return wg, wu, wd


def _shared_weights(inp: Dict[str, np.ndarray], w_dtype: str):
    return (dequant_weight(inp["ws_gate"], inp.get("ss_gate"), w_dtype),
            dequant_weight(inp["ws_up"], inp.get("ss_up"), w_dtype),
            dequant_weight(inp["ws_down"], inp.get("ss_down"), w_dtype))


def _finish(out64: np.ndarray, x_dtype: str, residual: Optional[np.ndarray]):
    if residual is not None:
        out64 = out64 + _x_to_f64(residual)
    if x_dtype == "bf16":
        return out64, round_to_bf16_bits(out64)
    return out64, out64.astype(np.float32)


def moe_forward(inp: Dict[str, np.ndarray], top_k: int, w_dtype: str, x_dtype: str,
                residual: Optional[np.ndarray] = None, renormalize: bool = False,
                act_quant: bool = False) -> Dict[str, np.ndarray]:
    """The whole layer for every token.

    `inp` holds numpy arrays as produced by moe_inputs.to_numpy.  With
    `residual` the old output is added before the single rounding (the
    caller's residual add, done in place).  With `act_quant` the inputs of
    every expert matmul (x, and each expert's hidden activations) are
    quantised dynamically in 1 x 128 groups (quantize_groups); the router
    still sees x unquantised.  Returns routing, layout, per-row expert
    outputs and the output (float64 and rounded to the output dtype).
    """
    x64 = _x_to_f64(inp["x"])
    n = x64.shape[0]
    n_exp = inp["router_w"].shape[0]
    h32 = router_logits(x64, inp["router_w"])
    ids, gap, s = select_topk(h32, inp["router_b"], top_k)
    w = mixture_weights(h32, ids, renormalize)
    counts, offsets, pair_of_row, row_of_pair = dispatch(ids, n_exp)

    d = x64.shape[1]
    xe = fake_quant(x64) if act_quant else x64   # the experts' input
    y_rows = np.zeros((n * top_k, d), dtype=np.float64)
    for e in range(n_exp):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if lo == hi:
            continue
        tokens = pair_of_row[lo:hi] // top_k
        wg, wu, wd = _expert_weights(inp, e, w_dtype)
        y_rows[lo:hi] = swiglu_expert(xe[tokens], wg, wu, wd, act_quant)

    ys = swiglu_expert(xe, *_shared_weights(inp, w_dtype), act_quant)
    out64 = combine(ys, y_rows, w, row_of_pair)
    out64, out_cast = _finish(out64, x_dtype, residual)
    return dict(logits=h32, scores=s, ids=ids, gap=gap, w=w, counts=counts,
                offsets=offsets, pair_of_row=pair_of_row, row_of_pair=row_of_pair,
                y_rows=y_rows, ys=ys, out64=out64, out=out_cast)


def token_outputs(inp: Dict[str, np.ndarray], tokens: Sequence[int], top_k: int,
                  w_dtype: str, ids: Optional[np.ndarray] = None,
                  renormalize: bool = False, act_quant: bool = False) -> Dict[str, np.ndarray]:
    """Routing of every token, and the output of the listed tokens only.

    For full-size checks: the layer output of token t depends only on x[t],
    its own selection and the weights, so sampled tokens are evaluated one by
    one.  With `ids` given (e.g. another implementation's selection), those
    experts are used for the output instead of the oracle's own choice; the
    mixture weights still come from the oracle's unbiased logits.
    """
    x64 = _x_to_f64(inp["x"])
    h32 = router_logits(x64, inp["router_w"])
    own_ids, gap, _ = select_topk(h32, inp["router_b"], top_k)
    use_ids = own_ids if ids is None else np.asarray(ids)
    w = mixture_weights(h32, use_ids, renormalize)
    shared = _shared_weights(inp, w_dtype)
    cache: Dict[int, tuple] = {}
    outs = []
    for t in tokens:
        xt = x64[t:t + 1]
        if act_quant:   # groups lie within one row, so a row quantises on its own
            xt = fake_quant(xt)
        acc = swiglu_expert(xt, *shared, act_quant)[0]
        for j in range(top_k):
            e = int(use_ids[t, j])
            if e not in cache:
                cache[e] = _expert_weights(inp, e, w_dtype)
            acc = acc + w[t, j] * swiglu_expert(xt, *cache[e], act_quant)[0]
        outs.append(acc)
    return dict(logits=h32, ids=own_ids, gap=gap, w=w, out64=np.array(outs))


# --------------------------------------------------------------------------
# sandwich normalisation around the MoE sublayer
# --------------------------------------------------------------------------

def rms_norm(v64: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: v / sqrt(mean(v^2) + eps) * g, float64."""
    g64 = np.asarray(g, dtype=np.float32).astype(np.float64)
    return v64 / np.sqrt(np.mean(v64 * v64, axis=-1, keepdims=True) + eps) * g64


def block_forward(inp: Dict[str, np.ndarray], resid: np.ndarray, g_pre: np.ndarray, g_post: np.ndarray,
                  eps: float, top_k: int, w_dtype: str, x_dtype: str,
                  renormalize: bool = False, act_quant: bool = False) -> Dict[str, np.ndarray]:
    """The MoE sublayer of a sandwich-normalised block, residual stream updated.

    "Inside Kolibri 1" (flozi.net), section "The released stack": RMSNorm
    before and after the MoE, residual addition after the sublayer:
        x   = RMSNorm(r; g_pre), rounded to the activation type (the MoE input)
        y   = MoE(x)
        out = r + RMSNorm(y; g_post), rounded once to the activation type.
    """
    r64 = _x_to_f64(resid)
    xn = rms_norm(r64, g_pre, eps)
    xs = round_to_bf16_bits(xn) if x_dtype == "bf16" else xn.astype(np.float32)
    res = moe_forward(dict(inp, x=xs), top_k, w_dtype, x_dtype, renormalize=renormalize, act_quant=act_quant)
    z = rms_norm(res["out64"], g_post, eps)
    out64 = r64 + z
    out = round_to_bf16_bits(out64) if x_dtype == "bf16" else out64.astype(np.float32)
    res.update(x_norm=xs, y64=res["out64"], out64=out64, out=out)
    return res


# --------------------------------------------------------------------------
# independent formulations used as pins
# --------------------------------------------------------------------------

def brute_force_topk(s_row: np.ndarray, k: int) -> tuple:
    """Best k-subset of one token's scores by enumeration (small E only).

    The k largest scores form the subset with the largest score sum; among
    equal sums the lexicographically smallest ascending id tuple wins, which
    is the lower-id tie rule.
    """
    best, best_sum = None, -math.inf
    s64 = [float(v) for v in s_row]
    for sub in combinations(range(len(s64)), k):
        tot = math.fsum(s64[i] for i in sub)
        if tot > best_sum:
            best, best_sum = sub, tot
    return best


def expert_param_counts(d_model: int = 2560, d_ff: int = 512, n_routed: int = 384,
                        top_k: int = 6, n_shared: int = 1) -> Dict[str, int]:
    """Matrix weights per expert, per token-block and per block.

    Each expert holds two d->f projections and one f->d projection.
    """
    per_expert = 3 * d_model * d_ff
    return dict(per_expert=per_expert,
                per_token_block=(top_k + n_shared) * per_expert,
                per_block=(n_routed + n_shared) * per_expert)
