"""Pins of the CPU oracle: checks against what the pages and mathematics fix.

Every pin takes the oracle module as its argument so that the mutation tests
can run the same pins against a copy of the oracle with a planted mistake and
show that some pin fails.  Nothing here calls the HIP library.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

from moe_inputs import generate, get_config, to_numpy

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _sig(z):
    return 1.0 / (1.0 + math.exp(-z))


def _bf16_bits(a):
    t = torch.tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------

def pin_bf16_decode(o):
    """Every non-NaN bfloat16 pattern decodes like torch's bfloat16 -> float32."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    got = o.decode_bf16(bits)
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok].astype(np.float64))
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def pin_e4m3_decode(o):
    """All 256 E4M3FN codes decode like torch.float8_e4m3fn -> float32."""
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = o.decode_e4m3fn(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok].astype(np.float64))
    # largest finite magnitude is 448 and there is no infinity
    assert np.nanmax(np.abs(got)) == 448.0


def pin_fp8_scale_exact(o):
    """A dequantised FP8 weight is code x the stored FP32 scale, unrounded.

    The pages require FP32 scales to be used exactly, never rounded to a power
    of two; with a non-power-of-two scale the two readings differ.
    """
    codes = np.array([[0x38, 0x40, 0xC4, 0x01]], dtype=np.uint8)   # 1, 2, -3, 2^-9
    scale = np.array([0.0123], dtype=np.float32)
    got = o.dequant_weight(codes, scale, "fp8")
    exact = np.array([[1.0, 2.0, -3.0, 2.0 ** -9]]) * float(scale[0])
    assert np.array_equal(got, exact)
    pow2 = 2.0 ** round(math.log2(float(scale[0])))
    assert not np.allclose(got, np.array([[1.0, 2.0, -3.0, 2.0 ** -9]]) * pow2)


def pin_fp8_block_scales(o):
    """128x128 block scales: every element of a block uses that block's scale."""
    rng = np.random.default_rng(12)
    q = rng.integers(0, 256, size=(256, 384), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x30  # no NaN codes
    s = (rng.random((2, 3)) * 0.01 + 1e-3).astype(np.float32)
    got = o.dequant_weight(q, s, "fp8")
    dec = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for bo in range(2):
        for bi in range(3):
            blk = got[bo * 128:(bo + 1) * 128, bi * 128:(bi + 1) * 128]
            assert np.array_equal(blk, dec[bo * 128:(bo + 1) * 128, bi * 128:(bi + 1) * 128] * float(s[bo, bi]))


def pin_e4m3_encoder(o):
    """E4M3 encoding: round trip of every code, and torch's float8_e4m3fn cast
    (nearest, ties to even) on random values, exact midpoints and -0.0."""
    codes = np.arange(256, dtype=np.uint8)
    finite = codes[(codes & 0x7F) != 0x7F]
    assert np.array_equal(o.encode_e4m3fn(o.decode_e4m3fn(finite).astype(np.float32)), finite)
    rng = np.random.default_rng(13)
    table = o.decode_e4m3fn(np.arange(0x7F, dtype=np.uint8))
    mids = ((table[:-1] + table[1:]) / 2).astype(np.float32)   # exact in float32
    r = np.concatenate([rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 2.0 ** rng.integers(-12, 6, 20000),
                        mids, -mids, [0.0, -0.0, 448.0, -448.0]]).astype(np.float32)
    ref = torch.from_numpy(r).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(o.encode_e4m3fn(r), ref)


def pin_group_quantisation(o):
    """1 x 128 activation groups: closed forms and the error bound."""
    # a hand-worked group: amax 7 gives scale 7/448 = 2^-6 exactly, so codes are of 64 v
    v = np.zeros((1, 128), np.float32)
    v[0, :4] = [1.0, -2.0, 0.5, 7.0]
    q, sc = o.quantize_groups(v)
    assert sc[0, 0] == np.float32(2.0 ** -6)
    assert q[0, :4].tolist() == [0x68, 0xF0, 0x60, 0x7E] and not q[0, 4:].any()
    # an all-zero group has scale 1 and zero codes
    q, sc = o.quantize_groups(np.zeros((2, 256), np.float32))
    assert np.all(sc == 1.0) and not q.any()
    rng = np.random.default_rng(14)
    v = (rng.standard_normal((40, 512)) * rng.uniform(1e-3, 1e3, (40, 1))).astype(np.float32)
    q, sc = o.quantize_groups(v)
    assert q.shape == v.shape and sc.shape == (40, 4)
    # each group's largest magnitude maps to +-448
    g = np.abs(v).reshape(40, 4, 128).argmax(axis=2)
    top = np.take_along_axis(q.reshape(40, 4, 128), g[..., None], axis=2)[..., 0]
    assert np.all((top & 0x7F) == 0x7E)
    # nearest value: error at most half a step (2^-4 relative, or 2^-10 scale in the subnormal range)
    err = np.abs(o.dequantize_groups(q, sc) - v.astype(np.float64))
    s_full = np.repeat(sc.astype(np.float64), 128, axis=1)
    assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(v), 2.0 ** -10 * s_full) * (1 + 1e-6))
    # scaling a row by a power of two scales its scales and keeps its codes
    q4, sc4 = o.quantize_groups(v * np.float32(4.0))
    assert np.array_equal(q4, q) and np.array_equal(sc4, sc * np.float32(4.0))


def pin_hidden_quantised(o):
    """With act_quant, the down projection sees hidden values on the E4M3 grid of their group."""
    rng = np.random.default_rng(15)
    x = rng.standard_normal((6, 128))
    wg, wu = rng.standard_normal((128, 128)) * 0.1, rng.standard_normal((128, 128)) * 0.1
    y = o.swiglu_expert(x, wg, wu, np.eye(128), act_quant=True)   # identity down: y = quantised hidden
    a = x @ wg.T
    plain = a / (1 + np.exp(-a)) * (x @ wu.T)
    s = np.abs(y).max(axis=1, keepdims=True) / 448.0
    r = y / s
    grid = o.decode_e4m3fn(o.encode_e4m3fn(np.clip(r, -448, 448).astype(np.float32)))
    assert np.allclose(r, grid, rtol=1e-6, atol=1e-9)
    assert not np.allclose(y, plain, rtol=1e-3) and np.allclose(y, plain, rtol=0.07, atol=1e-3 * np.abs(plain).max())


def pin_bf16_rounding(o):
    """Output rounding to bfloat16 agrees with torch's float32 -> bfloat16."""
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-8, 8, 20000),
                        [0.0, -0.0, 1.0, 1.00390625, 1.01171875, -65504.0]]).astype(np.float32)
    got = o.round_to_bf16_bits(v.astype(np.float64))
    assert np.array_equal(got, _bf16_bits(v))


# --------------------------------------------------------------------------
# router and selection
# --------------------------------------------------------------------------

def pin_logits_correctly_rounded(o):
    """Logits are the exact dot product rounded once to float32.

    Checked with exact rational arithmetic on a small case.
    """
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 24)).astype(np.float32)
    w = rng.standard_normal((7, 24)).astype(np.float32) * 0.02
    got = o.router_logits(x.astype(np.float64), w)
    assert got.dtype == np.float32
    for t in range(5):
        for e in range(7):
            exact = sum(Fraction(float(x[t, i])) * Fraction(float(w[e, i])) for i in range(24))
            # the float32 nearest to the exact value: compare both neighbours
            f = np.float32(float(exact))
            cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
            best = min(cands, key=lambda c: abs(Fraction(float(c)) - exact))
            assert got[t, e] == best, (t, e)


def pin_brute_force_selection(o):
    """For E <= 8 the selection equals the best k-subset found by enumeration."""
    rng = np.random.default_rng(3)
    for n_exp in (6, 7, 8):
        for k in range(1, n_exp + 1):
            h = rng.standard_normal((6, n_exp)).astype(np.float32)
            b = (rng.standard_normal(n_exp) * 0.5).astype(np.float32)
            ids, gap, s = o.select_topk(h, b, k)
            for t in range(h.shape[0]):
                want = o.brute_force_topk(s[t], k)
                assert tuple(ids[t]) == tuple(want), (n_exp, k, t)
                # independent: brute force on plain float32 sums, no oracle involved
                s_ind = (h[t] + b).astype(np.float32)
                best = max(_subsets(n_exp, k), key=lambda S: (math.fsum(float(s_ind[i]) for i in S),
                                                              [-i for i in S]))
                assert tuple(ids[t]) == best
            if k == n_exp:
                assert np.all(np.isinf(gap))


def _subsets(n, k):
    from itertools import combinations
    return list(combinations(range(n), k))


def pin_tie_break_lower_id(o):
    """Equal scores go to the lower expert id."""
    h = np.array([[1.0, 3.0, 3.0, 2.0, 3.0, 0.0]], dtype=np.float32)
    b = np.zeros(6, dtype=np.float32)
    ids, gap, _ = o.select_topk(h, b, 2)
    assert ids.tolist() == [[1, 2]]
    assert gap[0] == 0.0
    ids, gap, _ = o.select_topk(h, b, 4)
    assert ids.tolist() == [[1, 2, 3, 4]]
    assert gap[0] == 1.0


def pin_bias_forces_subset(o):
    """A large bias on a subset S makes every token select exactly S."""
    rng = np.random.default_rng(4)
    for n_exp, k in ((8, 3), (8, 6), (7, 1)):
        h = rng.standard_normal((10, n_exp)).astype(np.float32)
        S = sorted(rng.choice(n_exp, size=k, replace=False).tolist())
        b = np.zeros(n_exp, dtype=np.float32)
        b[S] = 1e4
        ids, _, _ = o.select_topk(h, b, k)
        assert all(row == S for row in ids.tolist())
        # the weights still come from the unbiased logits
        w = o.mixture_weights(h, ids)
        want = 1.0 / (1.0 + np.exp(-h[:, S].astype(np.float64)))
        assert np.allclose(w, want, rtol=0, atol=1e-15)


def pin_zero_bias_is_library_topk(o):
    """With b = 0 the selected set is torch.topk's set of the logits."""
    rng = np.random.default_rng(5)
    h = rng.standard_normal((50, 32)).astype(np.float32)
    ids, _, _ = o.select_topk(h, np.zeros(32, np.float32), 6)
    ref = torch.topk(torch.from_numpy(h), 6, dim=1).indices.sort(dim=1).values.numpy()
    assert np.array_equal(ids, ref)


def pin_weights_unbiased_unnormalised(o):
    """Weights are sigmoid(h) at the ids; the bias never scales them.

    Changing the bias without changing the selection leaves the weights
    bit-identical; the weights do not sum to one.
    """
    rng = np.random.default_rng(6)
    h = rng.standard_normal((40, 16)).astype(np.float32)
    b = (rng.standard_normal(16) * 0.1).astype(np.float32)
    ids, gap, _ = o.select_topk(h, b, 4)
    w = o.mixture_weights(h, ids)
    assert np.all((w > 0) & (w < 1))
    assert not np.allclose(w.sum(axis=1), 1.0)
    # shifting every bias by the same amount keeps the selection
    ids2, _, _ = o.select_topk(h, b + np.float32(0.5), 4)
    assert np.array_equal(ids, ids2)
    w2 = o.mixture_weights(h, ids2)
    assert np.array_equal(w, w2)
    # closed form at one entry
    t, j = 3, 2
    assert w[t, j] == 1.0 / (1.0 + math.exp(-float(h[t, ids[t, j]])))


# --------------------------------------------------------------------------
# dispatch
# --------------------------------------------------------------------------

def pin_dispatch_is_stable_sort(o):
    """The dispatch layout is a stable argsort of the flattened ids."""
    rng = np.random.default_rng(7)
    for n, n_exp, k in ((1, 8, 6), (37, 16, 6), (300, 32, 6), (64, 384, 6)):
        h = rng.standard_normal((n, n_exp)).astype(np.float32)
        ids, _, _ = o.select_topk(h, np.zeros(n_exp, np.float32), k)
        counts, offsets, por, rop = o.dispatch(ids, n_exp)
        assert np.array_equal(por, np.argsort(ids.ravel(), kind="stable"))
        assert np.array_equal(counts, np.bincount(ids.ravel(), minlength=n_exp))
        assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
        assert int(counts.sum()) == n * k
        assert np.array_equal(rop[por], np.arange(n * k))
        # permute then unpermute restores any per-pair payload bit for bit
        payload = rng.standard_normal((n * k, 3))
        assert np.array_equal(payload[por][rop], payload)
        # each token's ids are distinct and ascending
        assert np.all(np.diff(ids, axis=1) > 0)


# --------------------------------------------------------------------------
# experts and the whole layer
# --------------------------------------------------------------------------

def pin_textbook_expert(o):
    """The expert equals torch's float64 silu(x Wg^T) * (x Wu^T) Wd^T."""
    rng = np.random.default_rng(8)
    x = rng.standard_normal((9, 40))
    wg, wu = rng.standard_normal((12, 40)) * 0.1, rng.standard_normal((12, 40)) * 0.1
    wd = rng.standard_normal((40, 12)) * 0.1
    got = o.swiglu_expert(x, wg, wu, wd)
    T = lambda a: torch.from_numpy(a)
    ref = torch.nn.functional.linear(
        torch.nn.functional.silu(torch.nn.functional.linear(T(x), T(wg))) *
        torch.nn.functional.linear(T(x), T(wu)), T(wd)).numpy()
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-15)


def _small_layer(n=48, d=32, n_exp=8, k=2, f=12, w_dtype="bf16", x_dtype="f32", seed=0, scale_block=0):
    cfg = get_config("toy").replace(n_tokens=n, d_model=d, n_experts=n_exp, top_k=k, d_ff=f,
                                    d_ff_shared=f, w_dtype=w_dtype, x_dtype=x_dtype, scale_block=scale_block)
    return cfg, to_numpy(generate(cfg, seed=seed))


def _dense_form(o, inp, k, w_dtype, act_quant=False):
    """Compute every expert on every token, mask by the selection, sum by id."""
    x = o.decode_bf16(inp["x"]) if inp["x"].dtype == np.uint16 else inp["x"].astype(np.float64)
    xe = o.fake_quant(x) if act_quant else x
    n_exp = inp["router_w"].shape[0]
    w32 = inp["router_w"].astype(np.float64)
    h = (x @ w32.T).astype(np.float32)
    s = (h + inp["router_b"][None, :]).astype(np.float32)
    mask = np.zeros(h.shape)
    for t in range(x.shape[0]):
        top = sorted(range(n_exp), key=lambda e: (-float(s[t, e]), e))[:k]
        for e in top:
            mask[t, e] = 1.0 / (1.0 + math.exp(-float(h[t, e])))
    sc = lambda key: inp.get(key)
    out = o.swiglu_expert(xe, o.dequant_weight(inp["ws_gate"], sc("ss_gate"), w_dtype),
                          o.dequant_weight(inp["ws_up"], sc("ss_up"), w_dtype),
                          o.dequant_weight(inp["ws_down"], sc("ss_down"), w_dtype), act_quant)
    for e in range(n_exp):
        g = lambda key, skey: o.dequant_weight(inp[key][e], None if sc(skey) is None else sc(skey)[e], w_dtype)
        ye = o.swiglu_expert(xe, g("w_gate", "s_gate"), g("w_up", "s_up"), g("w_down", "s_down"), act_quant)
        out = out + mask[:, e:e + 1] * ye
    return out, mask


def pin_dense_formulation(o):
    """Routed output equals the dense compute-every-expert-then-mask form."""
    for w_dtype, x_dtype, n_exp, k, blk in (("bf16", "f32", 8, 2, 0), ("fp8", "bf16", 8, 6, 0),
                                            ("bf16", "bf16", 16, 6, 0), ("fp8", "bf16", 8, 3, 128)):
        cfg, inp = _small_layer(n_exp=n_exp, k=k, w_dtype=w_dtype, x_dtype=x_dtype, scale_block=blk,
                                d=256 if blk else 32, f=128 if blk else 12)
        for aq in ((False, True) if blk else (False,)):
            res = o.moe_forward(inp, k, w_dtype, x_dtype, act_quant=aq)
            dense, mask = _dense_form(o, inp, k, w_dtype, act_quant=aq)
            assert np.allclose(res["out64"], dense, rtol=1e-12, atol=1e-14)
            sel = np.zeros_like(mask, dtype=bool)
            np.put_along_axis(sel, res["ids"].astype(np.int64), True, axis=1)
            assert np.array_equal(sel, mask > 0)


def pin_all_selected(o):
    """k = E: every expert is used with weight sigmoid(h); gap is +inf."""
    cfg, inp = _small_layer(n=20, n_exp=6, k=6)
    res = o.moe_forward(inp, 6, "bf16", "f32")
    assert np.all(np.isinf(res["gap"]))
    assert res["ids"].tolist() == [list(range(6))] * 20
    dense, _ = _dense_form(o, inp, 6, "bf16")
    assert np.allclose(res["out64"], dense, rtol=1e-12, atol=1e-14)


def pin_worked_example(o):
    """The hand-worked instance in tests/golden/worked_example.json."""
    with open(os.path.join(GOLDEN, "worked_example.json")) as fh:
        g = json.load(fh)
    inp = dict(x=np.array(g["x"], np.float32), router_w=np.array(g["router_w"], np.float32),
               router_b=np.array(g["router_b"], np.float32))
    for key in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down"):
        inp[key] = _bf16_bits(np.array(g[key], np.float32))
    res = o.moe_forward(inp, 2, "bf16", "f32")
    assert res["ids"].tolist() == g["expected_ids"]
    env = {"sig": _sig}
    want_w = [eval(expr, env) for expr in g["expected_weights_closed_form"]]
    assert np.allclose(res["w"][0], want_w, rtol=1e-15, atol=0)
    want = [eval(expr, env) for expr in g["expected_out_closed_form"]]
    assert np.allclose(res["out64"][0], want, rtol=1e-14, atol=1e-15)


def pin_token_outputs_match_full(o):
    """Evaluating sampled tokens one by one agrees with the full layer."""
    cfg, inp = _small_layer(n=30, n_exp=16, k=6, w_dtype="fp8", x_dtype="bf16", seed=3)
    full = o.moe_forward(inp, 6, "fp8", "bf16")
    toks = [0, 7, 29]
    part = o.token_outputs(inp, toks, 6, "fp8")
    assert np.array_equal(part["ids"], full["ids"])
    assert np.allclose(part["out64"], full["out64"][toks], rtol=1e-12, atol=1e-14)
    # with 1 x 128 activation quantisation
    cfg, inp = _small_layer(n=20, n_exp=8, k=3, w_dtype="fp8", x_dtype="bf16", seed=5, d=256, f=128,
                            scale_block=128)
    full = o.moe_forward(inp, 3, "fp8", "bf16", act_quant=True)
    part = o.token_outputs(inp, toks[:2] + [19], 3, "fp8", act_quant=True)
    assert np.allclose(part["out64"], full["out64"][toks[:2] + [19]], rtol=1e-12, atol=1e-14)


def pin_renormalized_weights(o):
    """Renormalised gate: softmax over the selected unbiased logits.

    Weights sum to one, their ratios are exp of logit differences, the bias
    never scales them, and the hand-worked instance gives sigmoid(+-3).
    """
    rng = np.random.default_rng(9)
    h = rng.standard_normal((30, 16)).astype(np.float32)
    b = (rng.standard_normal(16) * 0.1).astype(np.float32)
    ids, _, _ = o.select_topk(h, b, 5)
    w = o.mixture_weights(h, ids, renormalize=True)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    hs = np.take_along_axis(h, ids.astype(np.int64), axis=1).astype(np.float64)
    assert np.allclose(w[:, 0] / w[:, 1], np.exp(hs[:, 0] - hs[:, 1]), rtol=1e-12)
    ids2, _, _ = o.select_topk(h, b + np.float32(0.5), 5)
    assert np.array_equal(o.mixture_weights(h, ids2, renormalize=True), w)
    # the worked example: selected logits 2 and -1
    with open(os.path.join(GOLDEN, "worked_example.json")) as fh:
        g = json.load(fh)
    inp = dict(x=np.array(g["x"], np.float32), router_w=np.array(g["router_w"], np.float32),
               router_b=np.array(g["router_b"], np.float32))
    for key in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down"):
        inp[key] = _bf16_bits(np.array(g[key], np.float32))
    res = o.moe_forward(inp, 2, "bf16", "f32", renormalize=True)
    assert np.allclose(res["w"][0], [_sig(3.0), _sig(-3.0)], rtol=1e-15, atol=0)
    s1, s2, sm1 = _sig(1.0), _sig(3.0), _sig(-1.0)
    want = [s1 + s2 * 2 * s1 - _sig(-3.0) * 2 * sm1, -s2 * s1 - _sig(-3.0) * 2 * sm1]
    assert np.allclose(res["out64"][0], want, rtol=1e-14, atol=1e-15)


def pin_rms_norm(o):
    """RMSNorm equals torch's rms_norm in float64; a constant row has a closed form."""
    rng = np.random.default_rng(10)
    v = rng.standard_normal((7, 48)) * 3.0
    g = rng.standard_normal(48).astype(np.float32)
    eps = 1e-6
    ref = torch.nn.functional.rms_norm(torch.from_numpy(v), (48,), torch.from_numpy(g.astype(np.float64)), eps)
    assert np.allclose(o.rms_norm(v, g, eps), ref.numpy(), rtol=1e-13, atol=1e-15)
    c = -2.5
    got = o.rms_norm(np.full((1, 16), c), np.ones(16, np.float32) * 3.0, 0.25)
    assert np.allclose(got, 3.0 * c / math.sqrt(c * c + 0.25), rtol=1e-15)


def pin_block_worked_example(o):
    """Sandwich-normalised block reduces to the hand-worked instance.

    Residual r = [1, 2] and pre-norm weights sqrt(2.5) make the normalised
    input exactly x = [1, 2] after rounding to bfloat16; with unit post-norm
    weights and eps = 0 the block output is r + y / rms(y), y the worked
    example's layer output.
    """
    with open(os.path.join(GOLDEN, "worked_example.json")) as fh:
        g = json.load(fh)
    inp = dict(router_w=np.array(g["router_w"], np.float32), router_b=np.array(g["router_b"], np.float32))
    for key in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down"):
        inp[key] = _bf16_bits(np.array(g[key], np.float32))
    resid = _bf16_bits(np.array([[1.0, 2.0]], np.float32))
    g_pre = np.full(2, math.sqrt(2.5), np.float32)
    res = o.block_forward(inp, resid, g_pre, np.ones(2, np.float32), 0.0, 2, "bf16", "bf16")
    assert res["x_norm"].tolist() == _bf16_bits(np.array([[1.0, 2.0]], np.float32)).tolist()
    env = {"sig": _sig}
    y = np.array([eval(expr, env) for expr in g["expected_out_closed_form"]])
    want = np.array([1.0, 2.0]) + y / math.sqrt(float(np.mean(y * y)))
    assert np.allclose(res["out64"][0], want, rtol=1e-14, atol=1e-15)


def pin_block_scale_invariance(o):
    """Scaling the residual by c > 0 leaves the MoE input unchanged (eps ~ 0)."""
    cfg, inp = _small_layer(n=12, n_exp=8, k=2, x_dtype="f32", seed=4)
    rng = np.random.default_rng(11)
    r = rng.standard_normal((12, cfg.d_model)).astype(np.float32)
    gp = (1 + 0.1 * rng.standard_normal(cfg.d_model)).astype(np.float32)
    gq = (1 + 0.1 * rng.standard_normal(cfg.d_model)).astype(np.float32)
    a = o.block_forward(inp, r, gp, gq, 1e-12, 2, "bf16", "f32")
    b = o.block_forward(inp, (r * 4.0).astype(np.float32), gp, gq, 1e-12, 2, "bf16", "f32")
    assert np.allclose(a["y64"], b["y64"], rtol=1e-6, atol=1e-9)
    assert np.allclose(b["out64"] - 4.0 * r, a["out64"] - r, rtol=1e-6, atol=1e-9)


def pin_page_arithmetic(o):
    """Expert parameter counts printed on the pages."""
    with open(os.path.join(GOLDEN, "page_arithmetic.json")) as fh:
        g = json.load(fh)
    c = o.expert_param_counts(g["d_model"], g["d_ff"], g["n_routed"], g["top_k"], g["n_shared"])
    assert c["per_expert"] == g["per_expert_exact"]
    assert round(c["per_token_block"] / 1e6, 1) == g["per_token_block_printed_millions"]
    assert round(c["per_block"] / 1e9, 2) == g["per_block_printed_billions"]


def pin_residual_add(o):
    """With a residual the old output is added before the one rounding."""
    cfg, inp = _small_layer(n=10, n_exp=8, k=2, x_dtype="bf16")
    res0 = o.moe_forward(inp, 2, "bf16", "bf16")
    resid = inp["x"]
    res1 = o.moe_forward(inp, 2, "bf16", "bf16", residual=resid)
    assert np.allclose(res1["out64"], res0["out64"] + o.decode_bf16(resid), rtol=1e-15, atol=1e-15)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
