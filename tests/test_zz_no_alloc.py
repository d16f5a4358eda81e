"""moe_forward_noalloc (the library's own per-GPU scratch) against moe_forward with a caller
workspace, through the C ABI (needs an MI355X)."""
import sys

import numpy as np
import pytest
import torch

from moe_inputs import generate, get_config
from tests import parity as PA
from tests import report

pytestmark = pytest.mark.gpu


_CASE = [""]


def _say(*a):
    """Print progress; a case line and its result line also go to the run's summary."""
    line = " ".join(str(v) for v in a)
    print(line, flush=True)
    sys.stdout.flush()
    if line.startswith("case"):
        _CASE[0] = line
    elif line.lstrip().startswith("->"):
        report.add(f"{_CASE[0]}  {line.strip()}")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fine_grained_sparse_amd import binding
    binding.lib()  # raises if the library is missing


def _both(cfg, host, act_quant=False):
    """The same call through both entry points; every output and intermediate, as numpy."""
    from fine_grained_sparse_amd import binding as B
    dev = PA.to_device(host)
    x = dev["x"]
    n = x.shape[0]
    layer = B.MoeLayer(cfg.top_k, dev, n, x.dtype)
    flags = B.MOE_FLAG_FP8_ACT_QUANT if act_quant else 0
    desc = layer.desc(n, flags)
    res = []
    for noalloc in (False, True):
        bufs = B.route_outputs(n, cfg.n_experts, cfg.top_k, x.device)
        out = torch.full_like(x, float("nan"))
        if noalloc:
            st = B.forward_noalloc_raw(desc, x, dev["router_w"], dev["router_b"], layer.weights, out,
                                       B.aux_struct(bufs))
        else:
            ws = torch.empty(B.workspace_size(desc), dtype=torch.uint8, device=x.device)
            st = B.forward_raw(desc, x, dev["router_w"], dev["router_b"], layer.weights, out, ws,
                               B.aux_struct(bufs))
        assert st == B.MOE_OK, B.status_string(st)
        torch.cuda.synchronize()
        r = {k: v.cpu().numpy() for k, v in bufs.items()}
        r["out_bits"] = out.view(torch.int16 if out.dtype == torch.bfloat16 else torch.int32).cpu().numpy()
        r["out"] = out.float().cpu().numpy().astype(np.float64)
        res.append(r)
    return res


@pytest.mark.parametrize("first,second", [
    # the GEMM path at its largest fitting batch, then a stream-path batch
    (dict(name="decode", n_tokens=256), dict(name="decode", n_tokens=7)),
    # E4M3 block weights with 1 x 128 activations, then a smaller batch of the same layer
    (dict(name="fp8block", n_tokens=150, aq=True), dict(name="fp8block", n_tokens=33, aq=True)),
])
def test_noalloc_matches_workspace_entry_point(first, second):
    """Two calls in a row, the second smaller: outputs and every intermediate equal the
    workspace entry point's bit for bit, and the output passes the oracle check."""
    for spec in (first, second):
        cfg = get_config(spec["name"], n_tokens=spec["n_tokens"])
        aq = spec.get("aq", False)
        _say(f"case noalloc {cfg.name} N={cfg.n_tokens} act_quant={aq}")
        host = generate(cfg, seed=31 + cfg.n_tokens)
        ref, got = _both(cfg, host, act_quant=aq)
        for key in ("out_bits", "logits", "topk_ids", "topk_w", "gap", "expert_offsets", "pair_of_row",
                    "row_of_pair"):
            assert np.array_equal(ref[key], got[key], equal_nan=True), key
        stats = PA.full_check(cfg, host, got, act_quant=aq)
        _say(f"  -> {stats}")


def test_noalloc_rejects_oversized():
    """A description whose workspace exceeds the scratch array is refused before any launch."""
    from fine_grained_sparse_amd import binding as B
    cfg = get_config("decode", n_tokens=320)
    dev = PA.to_device(generate(cfg, seed=3))
    layer = B.MoeLayer(cfg.top_k, dev, cfg.n_tokens, torch.bfloat16)
    desc = layer.desc(cfg.n_tokens)
    assert B.workspace_size(desc) > B.MOE_NOALLOC_SCRATCH_BYTES
    out = torch.full_like(dev["x"], float("nan"))
    st = B.forward_noalloc_raw(desc, dev["x"], dev["router_w"], dev["router_b"], layer.weights, out)
    torch.cuda.synchronize()
    assert st == B.MOE_ERR_WORKSPACE
    assert torch.isnan(out.float()).all()
