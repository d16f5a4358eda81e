"""Plant mistakes in a copy of the oracle (on the CPU) and show a pin fails.

Each mutation is a plausible slip in one step of the layer: a wrong sign, a
dropped term, a transposed or swapped operand, the wrong logits feeding the
weights, an unstable dispatch.  The pins must catch every one of them.
"""
import os
import types

import pytest

from tests import oracle_pins as P

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "moe_oracle.py")

MUTATIONS = {
    "bias_sign": ("s = (h32 + b32[None, :]).astype(np.float32)",
                  "s = (h32 - b32[None, :]).astype(np.float32)"),
    "select_on_unbiased": ("s = (h32 + b32[None, :]).astype(np.float32)",
                           "s = (h32 + 0 * b32[None, :]).astype(np.float32)"),
    "weights_renormalised": ("        return z / z.sum(axis=1, keepdims=True)\n    return 1.0 / (1.0 + np.exp(-h))",
                             "        return z / z.sum(axis=1, keepdims=True)\n    w = 1.0 / (1.0 + np.exp(-h))\n"
                             "    return w / w.sum(axis=1, keepdims=True)"),
    "weights_sign": ("        return z / z.sum(axis=1, keepdims=True)\n    return 1.0 / (1.0 + np.exp(-h))",
                     "        return z / z.sum(axis=1, keepdims=True)\n    return 1.0 / (1.0 + np.exp(h))"),
    "tie_to_higher_id": ("order = np.argsort(-s.astype(np.float64), axis=1, kind=\"stable\")",
                         "order = n_exp - 1 - np.argsort(-s[:, ::-1].astype(np.float64), axis=1, kind=\"stable\")"),
    "slots_by_score": ("ids = np.sort(chosen, axis=1).astype(np.int32)",
                       "ids = chosen.astype(np.int32)"),
    "dispatch_unstable": ("    for t in range(n):\n        for j in range(k):\n            e = ids[t, j]",
                          "    for t in reversed(range(n)):\n        for j in range(k):\n            e = ids[t, j]"),
    "silu_on_up": ("hidden = a * _sigmoid(a) * u", "hidden = u * _sigmoid(u) * a"),
    "down_transposed": ("return hidden @ wd.T", "return hidden @ wd.T[::-1]"),
    "shared_dropped": ("out = ys.copy()", "out = np.zeros_like(ys)"),
    "combine_wrong_slot": ("out = out + w[:, j:j + 1] * y_rows[row_of_pair.reshape(n, k)[:, j]]",
                           "out = out + w[:, (j + 1) % k:(j + 1) % k + 1] * y_rows[row_of_pair.reshape(n, k)[:, j]]"),
    "e4m3_bias": ("np.exp2(e.astype(np.float64) - 7.0)", "np.exp2(e.astype(np.float64) - 8.0)"),
    "e4m3_no_subnormal": ("subnormal = (m / 8.0) * 2.0 ** (1 - 7)", "subnormal = (1.0 + m / 8.0) * 2.0 ** (0 - 7)"),
    "fp8_scale_pow2": ("return q * s[..., :, None]", "return q * np.exp2(np.round(np.log2(s)))[..., :, None]"),
    "logits_sign": ("return (x64 @ w64.T).astype(np.float32)", "return (-(x64 @ w64.T)).astype(np.float32)"),
    "logits_bf16": ("return (x64 @ w64.T).astype(np.float32)",
                    "return (x64 @ w64.T).astype(np.float32).astype(np.float16).astype(np.float32)"),
    "bf16_shift": ("<< np.uint32(16)", "<< np.uint32(15)"),
    "param_count": ("per_expert = 3 * d_model * d_ff", "per_expert = 2 * d_model * d_ff"),
    "residual_dropped": ("out64 = out64 + _x_to_f64(residual)", "out64 = out64"),
    "renorm_no_max_shift_sign": ("z = np.exp(h - h.max(axis=1, keepdims=True))",
                                 "z = np.exp(h.max(axis=1, keepdims=True) - h)"),
    "block_scale_transposed": ("return q * np.repeat(np.repeat(s, bo, axis=-2), bi, axis=-1)",
                               "return q * np.repeat(np.repeat(s, bi, axis=-1), bo, axis=-2)[..., ::-1, :]"),
    "aq_scale_240": ("amax / np.float32(E4M3_MAX)", "amax / np.float32(240.0)"),
    "aq_ties_up": ("pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))", "pick_hi = d_hi <= d_lo"),
    "aq_hidden_plain": ("        hidden = fake_quant(hidden)\n", "        hidden = hidden\n"),
    "aq_x_plain": ("xe = fake_quant(x64) if act_quant else x64", "xe = x64"),
    "aq_tokens_plain": ("        if act_quant:   # groups lie within one row, so a row quantises on its own\n            xt = fake_quant(xt)",
                        "        pass"),
    "rms_no_sqrt": ("return v64 / np.sqrt(np.mean(v64 * v64, axis=-1, keepdims=True) + eps) * g64",
                    "return v64 / (np.mean(v64 * v64, axis=-1, keepdims=True) + eps) * g64"),
    "block_no_post_norm": ("    z = rms_norm(res[\"out64\"], g_post, eps)", "    z = res[\"out64\"]"),
    "block_no_residual": ("    out64 = r64 + z", "    out64 = z"),
    "renorm_ignored": ("    w = mixture_weights(h32, ids, renormalize)\n    counts,",
                       "    w = mixture_weights(h32, ids)\n    counts,"),
}


def _mutant(name):
    with open(SRC_PATH) as fh:
        src = fh.read()
    old, new = MUTATIONS[name]
    assert src.count(old) >= 1, f"mutation {name} no longer applies"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new, 1), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_some_pin_catches(name):
    mod = _mutant(name)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(mod)
        except Exception:  # an assertion or a shape error both count
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutation {name}"
