"""Seeded synthetic inputs for the fine-grained MoE layer.

This module is shared by the CPU oracle (``oracle/``), the tests and the
benchmark.  It only draws and stores numbers: it holds none of the layer's
arithmetic (no router, no selection, no expert, no combine).  The FP8 weight
*encoding* below is part of the input recipe (it makes a synthetic FP8
checkpoint: E4M3 codes plus one FP32 scale per output channel); decoding those
codes is done separately by each side.

Shapes follow the layer described on "Inside Kolibri 1: Hybrid RNoPE Attention,
Sparse MoE, and FP8 Serving" (flozi.net): hidden size 2560, 384 routed experts,
top-6, one shared expert, SwiGLU experts 2560 -> 512 -> 2560, FP8 E4M3 weights
with FP32 scales.  The toy configuration is a scaled-down layer for tests.

Storage conventions (identical for both sides):
  x          [N, d]        float32 (toy) or bfloat16
  router_w   [E, d]        float32, values rounded to bfloat16-representable
  router_b   [E]           float32
  w_gate     [E, f, d]     bfloat16, or uint8 E4M3 codes + s_gate [E, f] float32
                           (or [E, f/128, d/128] with 128x128 block scales)
  w_up       [E, f, d]     as w_gate
  w_down     [E, d, f]     bfloat16, or uint8 codes + s_down [E, d] float32
  ws_gate    [f_s, d]      shared expert, same dtype rules (scales [f_s])
  ws_up      [f_s, d]
  ws_down    [d, f_s]      (scales [d])
All matrices are row-major [out][in].
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np
import torch

__all__ = ["LayerConfig", "CONFIGS", "get_config", "generate", "to_numpy",
           "TENSOR_ORDER", "zipf_bias"]

# Order of the per-tensor child seeds drawn from SeedSequence(seed).
TENSOR_ORDER = ("x", "router_w", "router_b", "w_gate", "w_up", "w_down",
                "ws_gate", "ws_up", "ws_down", "zipf_perm")


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    n_tokens: int
    d_model: int
    n_experts: int
    top_k: int
    d_ff: int
    d_ff_shared: int
    x_dtype: str          # "f32" | "bf16"  (the output has the same dtype)
    w_dtype: str          # "bf16" | "fp8"
    bias_kind: str        # "normal" | "zipf" | "hot"
    bias_std: float = 0.1
    zipf_s: float = 1.1
    x_std: float = 1.0
    w_std: float = 0.02
    router_std: float = 0.02
    scale_block: int = 0  # FP8 scales: 0 = one per output channel, 128 = one per 128x128 block

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)


_FULL = dict(d_model=2560, n_experts=384, top_k=6, d_ff=512, d_ff_shared=512)

CONFIGS: Dict[str, LayerConfig] = {
    # scaled-down layer used for exhaustive checks
    "toy": LayerConfig("toy", n_tokens=128, d_model=256, n_experts=32, top_k=6,
                       d_ff=64, d_ff_shared=64, x_dtype="f32", w_dtype="bf16",
                       bias_kind="normal", bias_std=0.1),
    # full layer shape, a decode batch
    "decode": LayerConfig("decode", n_tokens=32, x_dtype="bf16", w_dtype="bf16",
                          bias_kind="normal", bias_std=0.1, **_FULL),
    # full layer shape, a prefill chunk, near-uniform routing
    "prefill": LayerConfig("prefill", n_tokens=8192, x_dtype="bf16", w_dtype="bf16",
                           bias_kind="normal", bias_std=0.01, **_FULL),
    # FP8 E4M3 expert weights with one FP32 scale per output channel
    "fp8": LayerConfig("fp8", n_tokens=4096, x_dtype="bf16", w_dtype="fp8",
                       bias_kind="normal", bias_std=0.1, **_FULL),
    # FP8 E4M3 weights with one FP32 scale per 128x128 block (the released
    # checkpoint's granularity)
    "fp8block": LayerConfig("fp8block", n_tokens=4096, x_dtype="bf16", w_dtype="fp8", scale_block=128,
                            bias_kind="normal", bias_std=0.1, **_FULL),
    # FP8 weights, router bias = log of a Zipf(1.1) popularity over experts
    "zipf": LayerConfig("zipf", n_tokens=16384, x_dtype="bf16", w_dtype="fp8",
                        bias_kind="zipf", zipf_s=1.1, **_FULL),
    # compute-ceiling probe of the grouped GEMMs: a bias of +16 on experts
    # 0..top_k-1 routes every token to them, so every row tile is full and the
    # seven experts' weights are shared by all tiles (stay on chip)
    "hot": LayerConfig("hot", n_tokens=16384, x_dtype="bf16", w_dtype="bf16",
                       bias_kind="hot", bias_std=0.1, **_FULL),
}


def get_config(name: str, **overrides) -> LayerConfig:
    cfg = CONFIGS[name]
    return cfg.replace(**overrides) if overrides else cfg


def _child_seeds(seed: int) -> Dict[str, int]:
    kids = np.random.SeedSequence(seed).spawn(len(TENSOR_ORDER))
    return {name: int(k.generate_state(1, dtype=np.uint64)[0] & 0x7FFF_FFFF_FFFF_FFFF)
            for name, k in zip(TENSOR_ORDER, kids)}


def _randn(shape, std: float, seed: int, device: str) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
    return t.mul_(std)


def zipf_bias(n_experts: int, s: float, seed: int) -> torch.Tensor:
    """Router bias whose exponent is a Zipf(s) popularity share.

    b[e] = ln p[pi(e)], p[r] = r^-s / sum_r' r'^-s (r = 1..E), pi a seeded
    permutation.  Adding ln p to roughly unit-variance logits makes expert
    popularity heavy-tailed; many experts then receive no token at all.
    """
    r = np.arange(1, n_experts + 1, dtype=np.float64)
    p = r ** (-s)
    p /= p.sum()
    perm = np.random.Generator(np.random.PCG64(seed)).permutation(n_experts)
    return torch.from_numpy(np.log(p[perm]).astype(np.float32))


def _fp8_per_channel(w: torch.Tensor):
    """Encode float32 [..., out, in] as E4M3 codes + one FP32 scale per row.

    scale = amax(|row|) / 448 (448 is the largest finite E4M3 magnitude), codes
    = round-to-nearest-even(row / scale).  Part of the synthetic-checkpoint
    recipe, not of the layer.
    """
    amax = w.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax)).to(torch.float32)
    q = (w / scale.unsqueeze(-1)).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), scale


def _fp8_block(w: torch.Tensor, b: int):
    """Encode float32 [..., out, in] as E4M3 codes + one FP32 scale per b x b block.

    scale = amax(|block|) / 448, codes = round-to-nearest-even(w / scale); the
    scale tensor has shape [..., out/b, in/b].  Input recipe only.
    """
    *lead, o, i = w.shape
    wb = w.reshape(*lead, o // b, b, i // b, b)
    amax = wb.abs().amax(dim=(-3, -1))
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax)).to(torch.float32)
    q = (wb / scale.unsqueeze(-1).unsqueeze(-3)).to(torch.float8_e4m3fn)
    return q.reshape(*lead, o, i).view(torch.uint8), scale


def _encode(w: torch.Tensor, cfg: "LayerConfig"):
    if cfg.w_dtype == "fp8":
        return _fp8_block(w, cfg.scale_block) if cfg.scale_block else _fp8_per_channel(w)
    return w.to(torch.bfloat16), None


def _weight(shape, cfg: LayerConfig, seed: int, device: str, chunk_first_dim: bool):
    """bf16 tensor, or (uint8 codes, fp32 scales) for FP8.

    On the host the experts are drawn one at a time (bounded memory); on a GPU
    the whole tensor is drawn at once (a different, equally seeded stream).
    """
    if chunk_first_dim and len(shape) == 3 and not str(device).startswith("cuda"):
        # draw one expert at a time to bound peak host memory
        g = torch.Generator(device=device)
        g.manual_seed(seed)
        outs, scales = [], []
        for _ in range(shape[0]):
            w = torch.randn(shape[1:], generator=g, dtype=torch.float32, device=device)
            w.mul_(cfg.w_std)
            q, s = _encode(w, cfg)
            outs.append(q)
            if s is not None:
                scales.append(s)
        return torch.stack(outs), (torch.stack(scales) if scales else None)
    w = _randn(shape, cfg.w_std, seed, device)
    return _encode(w, cfg)


# Expert weights do not depend on the token count; the last few weight sets
# drawn are kept (read-only use) so that cases differing only in N reuse them.
_WEIGHT_CACHE: "Dict[tuple, Dict[str, torch.Tensor]]" = {}
_WEIGHT_CACHE_MAX = 2


def generate(cfg: LayerConfig, seed: int = 0, device: str = "cpu",
             n_tokens: Optional[int] = None, cache: bool = True) -> Dict[str, torch.Tensor]:
    """Draw every input of one layer call.  Returns torch tensors on `device`.

    Keys: x, router_w, router_b, w_gate, w_up, w_down, ws_gate, ws_up, ws_down
    and, for FP8 weights, s_gate, s_up, s_down, ss_gate, ss_up, ss_down.
    The weight tensors may be shared with earlier calls: do not modify them.
    """
    n = cfg.n_tokens if n_tokens is None else n_tokens
    seeds = _child_seeds(seed)
    d, E, f, fs = cfg.d_model, cfg.n_experts, cfg.d_ff, cfg.d_ff_shared
    out: Dict[str, torch.Tensor] = {}

    x = _randn((n, d), cfg.x_std, seeds["x"], device)
    out["x"] = x if cfg.x_dtype == "f32" else x.to(torch.bfloat16)

    rw = _randn((E, d), cfg.router_std, seeds["router_w"], device)
    out["router_w"] = rw.to(torch.bfloat16).to(torch.float32)

    if cfg.bias_kind == "zipf":
        out["router_b"] = zipf_bias(E, cfg.zipf_s, seeds["zipf_perm"]).to(device)
    elif cfg.bias_kind == "hot":
        b = _randn((E,), cfg.bias_std, seeds["router_b"], device)
        b[:cfg.top_k] += 16.0
        out["router_b"] = b
    else:
        out["router_b"] = _randn((E,), cfg.bias_std, seeds["router_b"], device)

    wkey = (d, E, f, fs, cfg.w_dtype, cfg.scale_block, cfg.w_std, seed, str(device))
    if cache and wkey in _WEIGHT_CACHE:
        out.update(_WEIGHT_CACHE[wkey])
        return out
    wts: Dict[str, torch.Tensor] = {}
    for key, shape in (("w_gate", (E, f, d)), ("w_up", (E, f, d)), ("w_down", (E, d, f)),
                       ("ws_gate", (fs, d)), ("ws_up", (fs, d)), ("ws_down", (d, fs))):
        w, s = _weight(shape, cfg, seeds[key], device, chunk_first_dim=True)
        wts[key] = w
        if s is not None:
            wts["s" + key[1:] if key.startswith("w_") else "ss" + key[2:]] = s
    if cache:
        while len(_WEIGHT_CACHE) >= _WEIGHT_CACHE_MAX:
            _WEIGHT_CACHE.pop(next(iter(_WEIGHT_CACHE)))
        _WEIGHT_CACHE[wkey] = wts
    out.update(wts)
    return out


def to_numpy(inputs: Dict[str, torch.Tensor]) -> Dict[str, np.ndarray]:
    """Host numpy views: bf16 tensors become their uint16 bit patterns."""
    res = {}
    for k, v in inputs.items():
        v = v.detach().cpu()
        if v.dtype == torch.bfloat16:
            res[k] = v.view(torch.int16).numpy().view(np.uint16)
        elif v.dtype == torch.uint8:
            res[k] = v.numpy()
        else:
            res[k] = v.numpy()
    return res
