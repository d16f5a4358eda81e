"""Helpers for comparing the HIP library with the CPU oracle.

The criteria:
  * selected expert ids: bit-exact, except tokens whose oracle gap between the
    k-th and (k+1)-th biased score is below 1e-5 (counted, and checked to be a
    valid selection within that gap; their output is compared with the oracle
    evaluated on the GPU's ids);
  * dispatch layout (offsets, pair_of_row, row_of_pair): bit-exact against the
    oracle's dispatch applied to the GPU's ids;
  * logits and mixture weights: within float32 accumulation error;
  * output: max over tokens of ||y_gpu[t] - y_ref[t]||_inf / ||y_ref[t]||_inf
    within 2e-2 for bfloat16 weights and 6e-2 for FP8 weights.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np
import torch

import oracle.moe_oracle as O
from fine_grained_sparse_amd import binding as B
from moe_inputs import LayerConfig, to_numpy

NEAR_TIE = 1e-5
OUT_TOL = {"bf16": 2e-2, "fp8": 6e-2}
# |logit| ~ 1 summed over d = 2560 products in float32: a few 1e-6 at most
LOGIT_ATOL = 2e-5


def to_device(inputs: Dict[str, torch.Tensor], device="cuda") -> Dict[str, torch.Tensor]:
    return {k: v.to(device) for k, v in inputs.items()}


def run_gpu(cfg: LayerConfig, dev_inputs: Dict[str, torch.Tensor], residual: Optional[torch.Tensor] = None,
            n_tokens: Optional[int] = None, renormalize: bool = False, act_quant: bool = False) -> Dict[str, np.ndarray]:
    """One moe_forward call with every optional output requested."""
    x = dev_inputs["x"]
    n = x.shape[0] if n_tokens is None else n_tokens
    layer = B.MoeLayer(cfg.top_k, dev_inputs, max(n, 1), x.dtype)
    bufs = B.route_outputs(n, cfg.n_experts, cfg.top_k, x.device)
    aux = B.aux_struct(bufs)
    if residual is not None:
        out = residual.clone()
        layer.forward(x, out=out, accumulate=True, aux=aux, renormalize=renormalize, act_quant=act_quant)
    else:
        out = torch.full_like(x, float("nan"))
        layer.forward(x, out=out, aux=aux, renormalize=renormalize, act_quant=act_quant)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in bufs.items()}
    res["out"] = out.float().cpu().numpy().astype(np.float64)
    return res


def check_routing(cfg: LayerConfig, g: Dict[str, np.ndarray], ref: Dict[str, np.ndarray],
                  renormalize: bool = False, logit_atol: float = LOGIT_ATOL,
                  near_tie: float = NEAR_TIE) -> Dict[str, int]:
    """Compare logits, ids, weights and layout; returns counts for reporting."""
    n = g["topk_ids"].shape[0]
    k, E = cfg.top_k, cfg.n_experts
    assert np.allclose(g["logits"], ref["logits"], rtol=0, atol=logit_atol), \
        f"logits max err {np.abs(g['logits'] - ref['logits']).max()}"
    near = ref["gap"] < near_tie
    ids_eq = np.all(g["topk_ids"] == ref["ids"], axis=1)
    bad = ~ids_eq & ~near
    assert not bad.any(), f"{bad.sum()} tokens differ in selection with gap >= {near_tie}: {np.nonzero(bad)[0][:10]}"
    # differing near-tie tokens: the GPU's set must be a valid top-k within the gap
    for t in np.nonzero(~ids_eq)[0]:
        s = ref["scores"][t].astype(np.float64)
        gi = g["topk_ids"][t]
        assert len(set(gi.tolist())) == k and np.all(np.diff(gi) > 0)
        kth = np.sort(s)[::-1][k - 1]
        assert np.all(s[gi] >= kth - near_tie)
    # ids ascending, distinct, in range
    assert np.all(np.diff(g["topk_ids"], axis=1) > 0) and g["topk_ids"].min() >= 0 and g["topk_ids"].max() < E
    # weights = sigmoid of the unbiased logit at the GPU's ids
    w_ref = O.mixture_weights(ref["logits"], g["topk_ids"], renormalize)
    # |d sigmoid / dh| <= 1/4 (the softmax variant's weights move no more than that per logit change)
    w_atol = 2e-6 if logit_atol <= LOGIT_ATOL else 2e-6 + 0.5 * logit_atol
    assert np.allclose(g["topk_w"], w_ref, rtol=0, atol=w_atol), f"weights err {np.abs(g['topk_w'] - w_ref).max()}"
    # gap (diagnostic value) is close to the oracle's where the ids agree
    if k < E:
        assert np.allclose(g["gap"][ids_eq], ref["gap"][ids_eq], rtol=0, atol=4 * logit_atol)
    else:
        assert np.all(np.isinf(g["gap"]))
    # dispatch layout: bit-exact against the oracle's dispatch of the GPU's ids
    counts, offsets, por, rop = O.dispatch(g["topk_ids"], E)
    assert np.array_equal(g["expert_offsets"], offsets), "expert_offsets differ"
    assert np.array_equal(g["pair_of_row"], por), "pair_of_row differs"
    assert np.array_equal(g["row_of_pair"], rop), "row_of_pair differs"
    return dict(tokens=n, near_tie=int(near.sum()), differing_ids=int((~ids_eq).sum()))


def rel_err(out: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per token ||out - ref||_inf / ||ref||_inf."""
    num = np.abs(out - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    return num / np.maximum(den, 1e-30)


def check_output(cfg: LayerConfig, gpu_out: np.ndarray, ref_out: np.ndarray, tokens: Optional[Sequence[int]] = None):
    tol = OUT_TOL[cfg.w_dtype]
    assert np.all(np.isfinite(gpu_out)), "non-finite output"
    e = rel_err(gpu_out, ref_out)
    worst = float(e.max()) if e.size else 0.0
    assert worst <= tol, f"max relative error {worst:.3e} > {tol} (token {int(np.argmax(e))})"
    return worst


def full_check(cfg: LayerConfig, host_inputs: Dict[str, torch.Tensor], g: Dict[str, np.ndarray],
               residual: Optional[np.ndarray] = None, renormalize: bool = False,
               act_quant: bool = False) -> Dict[str, float]:
    """Whole-layer oracle on every token, at any size (routing, layout and every output row)."""
    npi = to_numpy(host_inputs)
    ref = O.moe_forward(npi, cfg.top_k, cfg.w_dtype, cfg.x_dtype, residual=residual, renormalize=renormalize,
                        act_quant=act_quant)
    stats = check_routing(cfg, g, ref, renormalize)
    ref_out = ref["out64"].copy()
    diff = np.nonzero(np.any(g["topk_ids"] != ref["ids"], axis=1))[0]
    if diff.size:
        alt = O.token_outputs(npi, diff, cfg.top_k, cfg.w_dtype, ids=g["topk_ids"], renormalize=renormalize,
                              act_quant=act_quant)["out64"]
        if residual is not None:
            alt = alt + (O.decode_bf16(residual[diff]) if residual.dtype == np.uint16 else residual[diff])
        ref_out[diff] = alt
    stats["max_rel_err"] = check_output(cfg, g["out"], ref_out)
    return stats


def block_run_and_check(cfg: LayerConfig, host_inputs: Dict[str, torch.Tensor], seed: int = 0,
                        renormalize: bool = False, eps: float = 1e-6, act_quant: bool = False) -> Dict[str, float]:
    """moe_block_forward (sandwich norms, residual in place) against the oracle, in two parts.

    1. The pre-norm on its own: the normalised input the GPU wrote (kept in the
       workspace) against RMSNorm(resid) rounded to the activation type.
    2. The layer and the post-norm on that same normalised input: the oracle's
       layer evaluated on the GPU's x_norm, so routing, dispatch and output are
       held to the plain rules of full_check (ids bit-exact except oracle gaps
       below 1e-5; differing near-tie tokens compared on the GPU's ids), and
       resid_out = resid + RMSNorm(y; g_post) is checked on every token.
    """
    g = torch.Generator().manual_seed(seed + 7)
    n, d = host_inputs["x"].shape
    xdt = host_inputs["x"].dtype
    resid = (torch.randn(n, d, generator=g) * 3.0).to(xdt)
    g_pre = (1.0 + 0.1 * torch.randn(d, generator=g)).to(torch.bfloat16).float()
    g_post = (1.0 + 0.1 * torch.randn(d, generator=g)).to(torch.bfloat16).float()
    dev = to_device(host_inputs)
    layer = B.MoeLayer(cfg.top_k, dev, max(n, 1), xdt)
    bufs = B.route_outputs(n, cfg.n_experts, cfg.top_k, "cuda")
    r_dev = resid.cuda()
    layer.block_forward(r_dev, g_pre.cuda(), g_post.cuda(), eps, aux=B.aux_struct(bufs), renormalize=renormalize,
                        act_quant=act_quant)
    torch.cuda.synchronize()
    gout = {k: v.cpu().numpy() for k, v in bufs.items()}
    gout["out"] = r_dev.float().cpu().numpy().astype(np.float64)
    # the normalised input the layer read: stored after the layer's own workspace
    off = B.workspace_size(layer.desc(n, B.MOE_FLAG_FP8_ACT_QUANT if act_quant else 0))
    nbytes = n * d * (2 if xdt == torch.bfloat16 else 4)
    xn_t = layer.workspace[off:off + nbytes].cpu().view(xdt).reshape(n, d)
    npi = to_numpy(host_inputs)
    if xdt == torch.bfloat16:
        r_np = resid.view(torch.int16).numpy().view(np.uint16)
        r64 = O.decode_bf16(r_np)
        xn_gpu_store = xn_t.view(torch.int16).numpy().view(np.uint16)
        xn_gpu = O.decode_bf16(xn_gpu_store)
    else:
        r_np = resid.numpy()
        r64 = r_np.astype(np.float64)
        xn_gpu_store = xn_t.numpy()
        xn_gpu = xn_gpu_store.astype(np.float64)

    # 1. pre-norm.  The normalised input is rounded to the activation type;
    # where the FP32 value lies next to a rounding boundary, FP32 summation
    # order can flip the rounding by one unit (bf16: 2^-7 relative, on a small
    # fraction of elements).  FP32 activations are not rounded again: every
    # element may differ by a few FP32 ulps of arithmetic order.
    xn64 = O.rms_norm(r64, g_pre.numpy(), eps)
    xn_ref = O.decode_bf16(O.round_to_bf16_bits(xn64)) if xdt == torch.bfloat16 else \
        xn64.astype(np.float32).astype(np.float64)
    ulp = 2.0 ** -7 if xdt == torch.bfloat16 else 2.0 ** -20
    dx = np.abs(xn_gpu - xn_ref)
    assert np.all(dx <= ulp * np.abs(xn_ref) + 1e-30), "normalised input differs by more than one unit"
    flips = int((dx > 0).sum())
    if xdt == torch.bfloat16:
        assert flips <= max(8, dx.size // 1000), f"{flips} elements of the normalised input differ"

    # 2. layer + post-norm + residual on the GPU's normalised input
    npx = dict(npi, x=xn_gpu_store)
    ref = O.moe_forward(npx, cfg.top_k, cfg.w_dtype, cfg.x_dtype, renormalize=renormalize, act_quant=act_quant)
    stats = check_routing(cfg, gout, ref, renormalize)
    y64 = ref["out64"].copy()
    diff = np.nonzero(np.any(gout["topk_ids"] != ref["ids"], axis=1))[0]
    if diff.size:
        y64[diff] = O.token_outputs(npx, diff, cfg.top_k, cfg.w_dtype, ids=gout["topk_ids"],
                                    renormalize=renormalize, act_quant=act_quant)["out64"]
    out_ref = r64 + O.rms_norm(y64, g_post.numpy(), eps)
    stats["xnorm_flips"] = flips
    stats["max_rel_err"] = check_output(cfg, gout["out"], out_ref)
    return stats
