"""HIP library vs the CPU oracle, through the C ABI (needs an MI355X)."""
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


def _run_full(cfg, seed=0, residual=False, renormalize=False, act_quant=False):
    _say(f"case {cfg.name} N={cfg.n_tokens} d={cfg.d_model} E={cfg.n_experts} k={cfg.top_k} "
         f"f={cfg.d_ff} fs={cfg.d_ff_shared} x={cfg.x_dtype} w={cfg.w_dtype} blk={cfg.scale_block} seed={seed} "
         f"residual={residual} renorm={renormalize} act_quant={act_quant}")
    host = generate(cfg, seed=seed)
    dev = PA.to_device(host)
    res_t = res_np = None
    if residual:
        g = torch.Generator().manual_seed(seed + 99)
        r = torch.randn(host["x"].shape, generator=g).to(host["x"].dtype)
        res_t = r.cuda()
        res_np = r.view(torch.int16).numpy().view(np.uint16) if r.dtype == torch.bfloat16 else r.numpy()
    g = PA.run_gpu(cfg, dev, residual=res_t, renormalize=renormalize, act_quant=act_quant)
    stats = PA.full_check(cfg, host, g, residual=res_np, renormalize=renormalize, act_quant=act_quant)
    _say(f"  -> {stats}")
    return stats


@pytest.mark.parametrize("n", [128, 300])
def test_toy(n):
    """The toy layer on the stream path (128 tokens, two 64-row tiles for the shared expert) and
    on the grouped GEMMs (300 tokens)."""
    _run_full(get_config("toy", n_tokens=n))


@pytest.mark.parametrize("n", [1, 2, 5, 7, 32, 64, 65, 130, 192])
def test_decode_full_shape(n):
    """Full-size layer on the stream path (above 64 tokens: several 64-row tiles per group); up to
    4 tokens top-k and dispatch share one workgroup, from 5 to 64 the last top-k workgroup lays out
    the dispatch, above that the dispatch kernels run on their own."""
    _run_full(get_config("decode", n_tokens=n))


@pytest.mark.parametrize("cfg_name,over", [("decode", dict(n_tokens=32)), ("decode", dict(n_tokens=96, w_dtype="fp8")),
                                          ("toy", dict(n_tokens=300, x_dtype="bf16"))])
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_other_seeds(cfg_name, over, seed):
    """Fresh inputs for the stream path (bf16 and E4M3 weights) and the grouped GEMMs."""
    _run_full(get_config(cfg_name, **over), seed=seed)


@pytest.mark.parametrize("n", [16, 129])
def test_decode_fp8_weights(n):
    _run_full(get_config("decode", w_dtype="fp8", n_tokens=n))


_TOY_VARIANTS = [
    dict(top_k=1), dict(top_k=8), dict(n_experts=6, top_k=6), dict(n_experts=40),
    dict(d_model=192, d_ff=128, d_ff_shared=64), dict(x_dtype="bf16", w_dtype="fp8"),
    dict(n_tokens=1), dict(n_tokens=600), dict(n_tokens=257, n_experts=1024, top_k=8),
]


@pytest.mark.parametrize("over,n", [(v, None) for v in _TOY_VARIANTS] +
                         [(v, 300) for v in _TOY_VARIANTS if "n_tokens" not in v])
def test_toy_variants(over, n):
    """Odd shapes and dtypes at the toy's own batch (stream path up to 192 tokens) and at 300
    tokens (grouped GEMMs)."""
    _run_full(get_config("toy", **(dict(over, n_tokens=n) if n else over)))


@pytest.mark.parametrize("over", [
    dict(n_tokens=40, top_k=1), dict(n_tokens=40, top_k=8), dict(n_tokens=9, n_experts=6, top_k=6),
    dict(n_tokens=64, n_experts=1024, top_k=8), dict(n_tokens=33, x_dtype="bf16"), dict(n_tokens=5, x_dtype="bf16"),
])
def test_tail_dispatch_variants(over):
    """5 to 64 tokens on the stream path: the dispatch is laid out by the last top-k workgroup to
    finish (k = 1 and 8, every expert selected, 1024 experts, FP32 and bf16 x)."""
    _run_full(get_config("toy", **over))


def test_accumulate_into_residual():
    _run_full(get_config("toy", x_dtype="bf16", n_tokens=50), residual=True)
    _run_full(get_config("toy", n_tokens=20), residual=True)


@pytest.mark.parametrize("cfg_name,over", [
    ("toy", {}), ("toy", dict(x_dtype="bf16", n_tokens=300)), ("decode", dict(n_tokens=8)),
])
def test_renormalized_gate(cfg_name, over):
    """The softmax-over-selected gate variant (MOE_FLAG_RENORMALIZE)."""
    _run_full(get_config(cfg_name, **over), renormalize=True)


@pytest.mark.parametrize("over", [
    dict(n_tokens=16), dict(n_tokens=128), dict(n_tokens=600),
    dict(n_tokens=9, x_dtype="bf16", d_model=384, d_ff=256, d_ff_shared=128),
    dict(n_tokens=200, x_dtype="bf16", d_model=384, d_ff=256, d_ff_shared=128),
    dict(n_tokens=250, x_dtype="bf16", d_model=3072, d_ff=256, d_ff_shared=128),   # 24 K blocks: direct-to-LDS tile
    dict(n_tokens=250, x_dtype="bf16", d_model=3200, d_ff=256, d_ff_shared=128),   # 25 K blocks: register-staged tile
])
def test_fp8_block_scales_toy(over):
    """FP8 weights with one scale per 128 x 128 block (MOE_FLAG_FP8_BLOCK128): stream and GEMM
    paths, FP32 and bf16 activations, an odd count of 128-row output blocks, f != f_s, both GEMM
    tiles."""
    base = dict(w_dtype="fp8", scale_block=128, d_ff=128, d_ff_shared=128)
    base.update(over)
    _run_full(get_config("toy", **base))


@pytest.mark.parametrize("n", [4, 48])
def test_decode_fp8_block_scales(n):
    _run_full(get_config("fp8block", n_tokens=n))


@pytest.mark.parametrize("dtype,rows,cols", [("bf16", 1, 128), ("bf16", 37, 2560), ("f32", 300, 512),
                                             ("f32", 5, 384), ("bf16", 4096, 2560)])
def test_quantize_groups_bit_exact(dtype, rows, cols):
    """moe_quantize_groups: codes and scales bit-identical to the oracle's 1 x 128 quantiser."""
    from fine_grained_sparse_amd import binding as B
    from oracle import moe_oracle as O
    _say(f"case quantize {dtype} rows={rows} cols={cols}")
    g = torch.Generator().manual_seed(rows * 7 + cols)
    v = torch.randn(rows, cols, generator=g) * torch.exp2(torch.randint(-30, 30, (rows, 1), generator=g).float())
    v[0, :128] = 0.0                          # an all-zero group
    if rows > 2:
        v[1, 3] = -0.0                        # negative zero inside a non-zero group
        table = O.decode_e4m3fn(np.arange(0x7F, dtype=np.uint8))
        mids = (table[:-1] + table[1:]) / 2   # exact ties once the scale is 1
        v[2, :128] = 0.0
        v[2, 0] = 448.0
        v[2, 1:127] = torch.from_numpy(np.concatenate([mids[:63], -mids[63:126]]))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    v = v.to(tdt)
    q, sc = B.quantize_groups(v.cuda())
    torch.cuda.synchronize()
    rq, rs = O.quantize_groups(v.float().numpy())
    assert np.array_equal(sc.cpu().numpy(), rs), "scales differ"
    qg = q.cpu().numpy()
    bad = np.argwhere(qg != rq)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:5].tolist()}: {qg[tuple(bad[0])]} vs {rq[tuple(bad[0])]}"


@pytest.mark.parametrize("over", [
    dict(n_tokens=16), dict(n_tokens=128), dict(n_tokens=600), dict(n_tokens=16, scale_block=0),
    dict(n_tokens=200, scale_block=0), dict(n_tokens=9, d_model=384, d_ff=256, d_ff_shared=128),
    dict(n_tokens=200, d_model=384, d_ff=256, d_ff_shared=128),
    dict(n_tokens=250, d_model=3072, d_ff=256, d_ff_shared=128),   # 24 K blocks: the direct-to-LDS tile's limit
    dict(n_tokens=250, d_model=3200, d_ff=256, d_ff_shared=128),   # 25 K blocks: the register-staged tile
    # from 8192 tokens: the 256 x 256 FP8 x FP8 gate/up tile (8 waves of 128 x 64)
    dict(n_tokens=8192, n_experts=8, top_k=2, d_model=256, d_ff=256, d_ff_shared=128),
    dict(n_tokens=8192, n_experts=8, top_k=2, d_model=256, d_ff=256, d_ff_shared=128, scale_block=0),
    dict(n_tokens=8300, n_experts=24, top_k=3, d_model=640, d_ff=128, d_ff_shared=384),   # odd stage count
    dict(n_tokens=8200, n_experts=40, top_k=4, d_model=128, d_ff=256, d_ff_shared=128, scale_block=0),  # 1 stage
    dict(n_tokens=9000, n_experts=256, top_k=8, d_model=384, d_ff=128, d_ff_shared=256),  # ~280 rows per expert
])
def test_fp8_act_quant_toy(over):
    """1 x 128 activation quantisation with FP8 x FP8 matmuls (MOE_FLAG_FP8_ACT_QUANT): stream and
    GEMM paths, block and per-channel weight scales, odd block counts, f != f_s, the 128-row tiles
    (direct-to-LDS and register-staged) and the 256-row gate/up tile."""
    base = dict(x_dtype="bf16", w_dtype="fp8", scale_block=128, d_ff=128, d_ff_shared=128)
    base.update(over)
    _run_full(get_config("toy", **base), act_quant=True)


@pytest.mark.parametrize("name,n", [("fp8block", 32), ("fp8", 48), ("fp8block", 150)])
def test_decode_act_quant(name, n):
    _run_full(get_config(name, n_tokens=n), act_quant=True)


def test_block_act_quant():
    """Sandwich-norm block with 1 x 128 activation quantisation."""
    cfg = get_config("fp8block", n_tokens=150)
    _say(f"case block act_quant {cfg.name} N={cfg.n_tokens}")
    stats = PA.block_run_and_check(cfg, generate(cfg, seed=3), seed=3, act_quant=True)
    _say(f"  -> {stats}")


@pytest.mark.parametrize("cfg_name,over", [
    ("decode", dict(n_tokens=192)),                                    # largest batch on the stream path
    ("decode", dict(n_tokens=193)),                                    # smallest batch on the grouped GEMMs
    ("decode", dict(n_tokens=65)),                                     # two 64-row stream tiles for the shared expert
    ("toy", dict(n_tokens=40, n_experts=448, top_k=8)),                # small batch, 7 experts per lane in top-k
    ("toy", dict(n_tokens=8, d_model=4096, n_experts=64, d_ff=512, d_ff_shared=512, x_dtype="bf16")),  # widest stream rows
    ("toy", dict(n_tokens=16, d_model=4160, n_experts=48, d_ff=128, d_ff_shared=128, x_dtype="bf16")),  # d past the stream path
    ("toy", dict(n_tokens=16, d_ff=640, d_ff_shared=512)),             # f past the stream path: GEMM at tiny m
    ("toy", dict(n_tokens=100, d_model=2560, n_experts=1024, top_k=8, x_dtype="bf16")),  # most experts, largest k
    ("toy", dict(n_tokens=300, n_experts=202, top_k=7, x_dtype="bf16")),  # router GEMM: one ragged expert tile, E % 4 != 0
    ("toy", dict(n_tokens=24, d_model=640, x_dtype="bf16")),            # small-batch router: two waves per k-slice
    ("toy", dict(n_tokens=24, d_model=1280, x_dtype="bf16")),           # small-batch router: four waves per k-slice
    ("toy", dict(n_tokens=16640)),                                      # 65 dispatch blocks: separate scan launch
    ("toy", dict(n_tokens=20000, x_dtype="bf16", d_model=128, d_ff=64, d_ff_shared=64)),  # the same with wide tiles
])
def test_shape_limits(cfg_name, over):
    """Edges of the supported shapes and of the stream/GEMM path choice."""
    _run_full(get_config(cfg_name, **over))


@pytest.mark.parametrize("cfg_name,over,kw", [
    ("decode", dict(n_tokens=3), dict(renormalize=True)),
    ("decode", dict(n_tokens=4, w_dtype="fp8"), {}),
    ("fp8block", dict(n_tokens=2), dict(act_quant=True)),
    ("toy", dict(n_tokens=4, n_experts=1024, top_k=8), {}),           # 16 experts per lane, the largest k
    ("toy", dict(n_tokens=1, x_dtype="bf16"), dict(residual=True)),
])
def test_fused_route(cfg_name, over, kw):
    """Batches of at most four tokens run top-k and dispatch as one kernel."""
    _run_full(get_config(cfg_name, **over), **kw)


_WIDE = dict(x_dtype="bf16")


@pytest.mark.parametrize("cfg_name,over", [
    ("decode", dict(n_tokens=8200)),                                   # ragged last tiles, bf16 weights
    ("decode", dict(n_tokens=8192, w_dtype="fp8")),                    # E4M3 weights, per-channel scales
    # f not a multiple of 128 (a half-empty column block), K of 3 stages, about 3000 rows per expert
    ("toy", dict(_WIDE, n_tokens=8192, n_experts=16, d_model=192, d_ff=192, d_ff_shared=64)),
    ("toy", dict(_WIDE, n_tokens=8192, n_experts=16, d_model=192, d_ff=192, d_ff_shared=64, w_dtype="fp8")),
    # short K (d = 128: 2 stages), f = 64, the most experts, the largest k
    ("toy", dict(_WIDE, n_tokens=8300, n_experts=512, top_k=8, d_model=128, d_ff=64, d_ff_shared=128)),
    ("toy", dict(_WIDE, n_tokens=8192, n_experts=64, d_model=64, d_ff=64, d_ff_shared=64, w_dtype="fp8")),  # 1 stage
])
def test_wide_tile(cfg_name, over):
    """Large batches with bf16 activations run the 256-row gate/up tiles (bf16 or per-channel E4M3
    weights) while the down product walks a 128-row list of its own: odd widths, ragged and
    multi-tile experts, short K."""
    _run_full(get_config(cfg_name, **over))


@pytest.mark.parametrize("cfg_name,over", [
    ("toy", dict(n_tokens=300, d_model=256, d_ff=192, d_ff_shared=256)),             # one column block, f != f_s
    ("toy", dict(n_tokens=600, n_experts=64, top_k=8, d_model=512, d_ff=256, d_ff_shared=192)),
    ("toy", dict(n_tokens=600, n_experts=64, top_k=8, d_model=512, d_ff=256, d_ff_shared=192, w_dtype="fp8")),
    ("toy", dict(n_tokens=6000, n_experts=32, top_k=4, d_model=1024, d_ff=192, d_ff_shared=320)),  # ~4 items per CU
    ("toy", dict(n_tokens=3000, n_experts=32, top_k=4, d_model=768, d_ff=128, d_ff_shared=320, w_dtype="fp8")),
    ("toy", dict(n_tokens=300)),                                        # K of one stage: the ring runs items ahead
    ("toy", dict(n_tokens=300, w_dtype="fp8", x_dtype="bf16")),
    ("decode", dict(n_tokens=193)),                                    # ~13 items per CU, most of 1-8 rows
    ("decode", dict(n_tokens=250, w_dtype="fp8")),
    # from 8192 tokens with bf16 activations: 256 x 256 items (16 waves)
    ("toy", dict(_WIDE, n_tokens=8192, n_experts=8, top_k=2, d_model=256, d_ff=256, d_ff_shared=192)),
    ("toy", dict(_WIDE, n_tokens=8192, n_experts=8, top_k=2, d_model=256, d_ff=256, d_ff_shared=192, w_dtype="fp8")),
    ("toy", dict(_WIDE, n_tokens=8300, n_experts=24, top_k=3, d_model=512, d_ff=64, d_ff_shared=128)),   # K of 1-2 stages
    ("toy", dict(_WIDE, n_tokens=8300, n_experts=24, top_k=3, d_model=512, d_ff=64, d_ff_shared=128, w_dtype="fp8")),
    ("toy", dict(_WIDE, n_tokens=9000, n_experts=256, top_k=8, d_model=768, d_ff=128, d_ff_shared=256)),  # ~280 rows per expert
    # E4M3 weights with 128 x 128 block scales: every stage folded with its K block's scale
    ("toy", dict(n_tokens=300, w_dtype="fp8", scale_block=128, d_model=256, d_ff=128, d_ff_shared=256)),
    ("toy", dict(n_tokens=600, w_dtype="fp8", scale_block=128, x_dtype="bf16", n_experts=64, top_k=8,
                 d_model=768, d_ff=384, d_ff_shared=128)),
    ("toy", dict(n_tokens=5000, w_dtype="fp8", scale_block=128, x_dtype="bf16", n_experts=24, top_k=4,
                 d_model=512, d_ff=256, d_ff_shared=512)),
])
def test_persistent_down(cfg_name, over):
    """bf16 or per-channel E4M3 weights with d a multiple of 256 run the persistent down products,
    whose DMA rings cross item boundaries: 128 x 256 items below 8192 tokens, 256 x 256 items
    (with the wide gate/up tiles) from there; items of different K (shared expert), K shorter than
    the rings, one or several column blocks, few and many items per workgroup, nearly empty row
    tiles, per-channel scales staged per item."""
    _run_full(get_config(cfg_name, **over))


@pytest.mark.parametrize("over", [
    dict(n_tokens=300, d_model=256),                                                  # one stage: items run ahead
    dict(n_tokens=300, d_model=256, scale_block=0),
    dict(n_tokens=6000, n_experts=32, top_k=4, d_model=1024, d_ff=384, d_ff_shared=512),   # ~4 items per CU
    dict(n_tokens=3000, n_experts=32, top_k=4, d_model=768, d_ff=128, d_ff_shared=256, scale_block=0),
    dict(n_tokens=600, n_experts=64, top_k=8, d_model=512, d_ff=256, d_ff_shared=384),
])
def test_persistent_down_act_quant(over):
    """1 x 128 quantised H with E4M3 weights (block or per-channel scales), d a multiple of 256
    and K at most 4 blocks: the persistent FP8 x FP8 down product, its ring crossing items of
    different K, the activation and weight scales staged per item in LDS."""
    base = dict(x_dtype="bf16", w_dtype="fp8", scale_block=128, d_ff=128, d_ff_shared=128)
    base.update(over)
    _run_full(get_config("toy", **base), act_quant=True)


@pytest.mark.parametrize("over", [dict(n_tokens=250), dict(n_tokens=1000)])
def test_persistent_down_act_quant_full(over):
    """The full layer shape (d = 2560, f = 512, 384 experts) with the released checkpoint's
    format: about 13 mostly short items per CU at 250 tokens, about 20 at 1000."""
    _run_full(get_config("fp8block", **over), act_quant=True)


@pytest.mark.parametrize("n", [300, 40, 4096, 8192])
def test_router_full_fp32_weights(n):
    """FP32 router weights that are not bf16 values (mid and lo split terms nonzero) for a scattered
    subset of experts: expert blocks with all, some and none of their experts flagged (the router
    GEMM skips the zero-term slices only where a whole block has none), the N <= 64 router, and
    the top-k's two- and four-token waves (N = 4096, 8192; 4 and 2 K slices per split term)."""
    cfg = get_config("toy", n_tokens=n, x_dtype="bf16", n_experts=384, d_ff=64, d_ff_shared=64)
    host = generate(cfg, seed=8)
    rw = host["router_w"].clone()
    pert = torch.zeros(cfg.n_experts, dtype=torch.bool)
    pert[0:128] = True                                   # block 0: every expert
    pert[128:256:7] = True                               # block 1: some experts
    rw[pert] = rw[pert] * (1.0 + 3.0 * 2.0 ** -12)       # no longer bf16-representable
    assert not torch.equal(rw[pert].to(torch.bfloat16).float(), rw[pert])
    host = dict(host, router_w=rw)
    _say(f"case full-fp32 router N={n} E={cfg.n_experts}")
    g = PA.run_gpu(cfg, PA.to_device(host))
    stats = PA.full_check(cfg, host, g)
    _say(f"  -> {stats}")


@pytest.mark.parametrize("n", [16, 200])
def test_128_experts(n):
    """The 128-expert shape of the predecessor model, top-6, full hidden size."""
    _run_full(get_config("decode", n_experts=128, n_tokens=n))


@pytest.mark.parametrize("cfg_name,over,renorm", [
    ("toy", {}, False), ("toy", dict(x_dtype="bf16", n_tokens=300), False), ("decode", {}, False),
    ("decode", dict(n_tokens=100, w_dtype="fp8"), True), ("decode", dict(n_tokens=3), False),
])
def test_block_sandwich_norm(cfg_name, over, renorm):
    """moe_block_forward: pre-RMSNorm, the layer, post-RMSNorm + residual fused in the combine."""
    cfg = get_config(cfg_name, **over)
    _say(f"case block {cfg.name} N={cfg.n_tokens} x={cfg.x_dtype} w={cfg.w_dtype} renorm={renorm}")
    stats = PA.block_run_and_check(cfg, generate(cfg, seed=2), seed=2, renormalize=renorm)
    _say(f"  -> {stats}")


def test_deterministic():
    cfg = get_config("decode", n_tokens=32)
    dev = PA.to_device(generate(cfg, seed=5))
    a = PA.run_gpu(cfg, dev)
    b = PA.run_gpu(cfg, dev)
    for key in a:
        assert np.array_equal(a[key], b[key], equal_nan=True), key


@pytest.mark.parametrize("cfg_name,over,aq", [("decode", dict(n_tokens=32), False), ("toy", dict(n_tokens=300), False),
                                             ("fp8block", dict(n_tokens=200), True), ("decode", dict(n_tokens=2), False)])
def test_graph_replay_matches_eager(cfg_name, over, aq):
    """moe_forward captured in a HIP graph: every replay equals the eager result bit for bit,
    with eager work on the same buffers between replays."""
    from fine_grained_sparse_amd import binding as B
    cfg = get_config(cfg_name, **over)
    _say(f"case graph {cfg.name} N={cfg.n_tokens} act_quant={aq}")
    dev = PA.to_device(generate(cfg, seed=6))
    x = dev["x"]
    layer = B.MoeLayer(cfg.top_k, dev, x.shape[0], x.dtype)
    ref = torch.empty_like(x)
    layer.forward(x, out=ref, act_quant=aq)
    out = torch.empty_like(x)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward(x, out=out, act_quant=aq)   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(x, out=out, act_quant=aq)
    for rep in range(3):
        out.fill_(float("nan"))
        layer.forward(x[: max(1, x.shape[0] // 2)], act_quant=aq)   # eager work that reuses the workspace
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out.view(torch.int32),
                           ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref.view(torch.int32)), rep


def test_in_place_residual():
    """x == out with MOE_FLAG_ACCUMULATE: out = round(x + layer(x)), the in-place residual update."""
    from fine_grained_sparse_amd import binding as B
    from oracle import moe_oracle as O
    from moe_inputs import to_numpy
    cfg = get_config("decode", n_tokens=24)
    host = generate(cfg, seed=11)
    dev = PA.to_device(host)
    x = dev["x"].clone()
    layer = B.MoeLayer(cfg.top_k, dev, x.shape[0], x.dtype)
    layer.forward(x, out=x, accumulate=True)
    torch.cuda.synchronize()
    npi = to_numpy(host)
    ref = O.moe_forward(npi, cfg.top_k, cfg.w_dtype, cfg.x_dtype, residual=npi["x"])
    got = x.float().cpu().numpy().astype(np.float64)
    err = PA.rel_err(got, ref["out64"])
    _say(f"case in-place residual: max rel err {err.max():.3e}")
    assert err.max() <= PA.OUT_TOL[cfg.w_dtype]


def test_two_streams_concurrently():
    """Two layers with their own workspaces on two streams at once: both match their eager results."""
    from fine_grained_sparse_amd import binding as B
    cfgs = [get_config("decode", n_tokens=32), get_config("toy", n_tokens=300, x_dtype="bf16")]
    devs = [PA.to_device(generate(c, seed=20 + i)) for i, c in enumerate(cfgs)]
    layers = [B.MoeLayer(c.top_k, d, d["x"].shape[0], d["x"].dtype) for c, d in zip(cfgs, devs)]
    refs = []
    for lay, d in zip(layers, devs):
        r = torch.empty_like(d["x"])
        lay.forward(d["x"], out=r)
        refs.append(r)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.full_like(d["x"], float("nan")) for d in devs]
    for rep in range(5):
        for st, lay, d, o in zip(streams, layers, devs, outs):
            with torch.cuda.stream(st):
                lay.forward(d["x"], out=o)
    torch.cuda.synchronize()
    for o, r in zip(outs, refs):
        assert torch.equal(o.view(torch.int16), r.view(torch.int16))


def test_zero_tokens_is_noop():
    from fine_grained_sparse_amd import binding as B
    cfg = get_config("toy")
    dev = PA.to_device(generate(cfg, seed=0, n_tokens=4))
    layer = B.MoeLayer(cfg.top_k, dev, 4, torch.float32)
    x = dev["x"][:0]
    out = torch.empty_like(x)
    layer.forward(x, out=out)
    torch.cuda.synchronize()


@pytest.mark.parametrize("name,aq", [("prefill", False), ("fp8", False), ("fp8block", False), ("zipf", False),
                                     ("fp8block", True), ("zipf", True)])
def test_full_size(name, aq):
    """Full-size workloads, every token: routing, dispatch layout and every output row against the
    oracle.  These are the cases that run the grouped GEMMs over many row tiles per expert (Zipf:
    about 120 tiles for the hottest expert, ragged last tiles) and the full-grid XCD work order."""
    cfg = get_config(name)
    _say(f"case {name} N={cfg.n_tokens} w={cfg.w_dtype} bias={cfg.bias_kind} act_quant={aq} (every token)")
    host = generate(cfg, seed=0)
    g = PA.run_gpu(cfg, PA.to_device(host), act_quant=aq)
    _say("  gpu done; oracle on every token")
    stats = PA.full_check(cfg, host, g, act_quant=aq)
    counts = np.diff(g["expert_offsets"])
    stats["empty_experts"] = int((counts == 0).sum())
    stats["max_expert_rows"] = int(counts.max())
    _say(f"  -> {stats}")
    assert stats["tokens"] == cfg.n_tokens
    if name == "zipf":
        # skewed routing: some experts receive no token, one receives most
        assert stats["empty_experts"] > 0 and stats["max_expert_rows"] > cfg.n_tokens // 2


# Exact ties.  Expert ids of a tie group share one router row and one bias, so
# their biased scores are bit-equal on both sides; the other experts are pushed
# above (forced) or below the group so that the tie sits exactly at the k-th /
# (k+1)-th place of every token (gap 0).  The lower id must win every time: no
# near-tie exemption applies.
_TIES = {
    # four forced experts, three tied ones: the two lowest ids of the three are selected
    "triple": dict(forced=[0, 100, 250, 300], tied=[7, 200, 383], tied_bias=[32.0, 32.0, 32.0], rest=None),
    # five forced experts, a tied pair whose biases differ only in the sign of zero
    "neg_zero_low": dict(forced=[3, 4, 5, 6, 7], tied=[50, 51], tied_bias=[-0.0, 0.0], rest=-64.0),
    "neg_zero_high": dict(forced=[3, 4, 5, 6, 7], tied=[50, 51], tied_bias=[0.0, -0.0], rest=-64.0),
    # the tied pair's router rows are zero: both scores are exactly zero
    "zero_score": dict(forced=[10, 20, 30, 40, 380], tied=[60, 61], tied_bias=[0.0, -0.0], rest=-64.0, zero=True),
}


@pytest.mark.parametrize("n", [32, 300])
@pytest.mark.parametrize("kind", list(_TIES))
def test_exact_score_ties(kind, n):
    """Bit-equal biased scores at the selection boundary go to the lower expert id (N <= 64 router
    and top-k, and the router GEMM with multi-token top-k waves above 64 tokens)."""
    spec = _TIES[kind]
    cfg = get_config("decode", n_tokens=n)
    host = generate(cfg, seed=13)
    rw, rb = host["router_w"].clone(), host["router_b"].clone()
    tied, forced = spec["tied"], spec["forced"]
    if spec["rest"] is not None:
        rb[:] = spec["rest"]
    rb[forced] = 64.0
    row = torch.zeros_like(rw[0]) if spec.get("zero") else rw[tied[0]].clone()
    for e, b in zip(tied, spec["tied_bias"]):
        rw[e] = row
        rb[e] = b
    host = dict(host, router_w=rw, router_b=rb)
    _say(f"case ties {kind} N={n} forced={forced} tied={tied} bias={spec['tied_bias']}")
    g = PA.run_gpu(cfg, PA.to_device(host))
    # the premise: the tied logits are bit-identical on the GPU for every token
    lg = g["logits"][:, tied]
    assert np.all(lg.view(np.uint32) == lg[:, :1].view(np.uint32)), "tied experts' GPU logits differ"
    k = cfg.top_k
    n_pick = k - len(forced)
    want = np.array(sorted(forced + tied[:n_pick]), dtype=np.int32)
    # exemption off: every token selects the forced ids and the lowest tied ids
    bad = np.nonzero(np.any(g["topk_ids"] != want[None, :], axis=1))[0]
    assert bad.size == 0, f"{bad.size} tokens break the tie rule, first {bad[:5]}: {g['topk_ids'][bad[:3]]}"
    assert np.all(g["gap"] == 0.0), "gap of an exact tie must be 0"
    stats = PA.full_check(cfg, host, g)
    assert stats["differing_ids"] == 0
    _say(f"  -> {stats}")
