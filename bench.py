#!/usr/bin/env python3
"""Throughput of the fine-grained MoE layer on one MI355X.

A step is one moe_forward call (router, top-k, dispatch, routed and shared
experts, combine) over one batch of synthetic tokens, with every input already
resident in HBM.  The default workload is the decode batch of the full layer:
N=32 tokens, d=2560, 384 routed experts top-6 + 1 shared, SwiGLU width 512,
bf16 activations and weights.  Successive steps cycle through `--layers`
independent layer instances (each with its own router, bias, experts and
token batch), as consecutive MoE layers of a model would, so that no step
finds its expert weights in the 256 MB last-level cache.

Prints one JSON line.  Besides throughput (eager launches) it reports the
roofline of the dominant kernel, timed live with HIP events that the library
records on the stream that runs the kernels (on every fifth timed step: each
event record drains the queue and would otherwise slow the steps it
measures), the distribution of single-step times, the rate of the same steps
replayed from a captured HIP graph, and the CPU oracle timed on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}
METRIC = "MoE-layer tokens/s + % HBM roofline (decode N<=64), % MFMA peak (prefill)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode", choices=["decode", "prefill", "fp8", "fp8block", "zipf", "toy"])
    ap.add_argument("--tokens", type=int, default=None, help="override the batch size")
    ap.add_argument("--layers", type=int, default=4, help="independent layer instances cycled by the steps")
    ap.add_argument("--event-stride", type=int, default=5,
                    help="the timed loop records the expert kernels' HIP events on every n-th step (n coprime "
                         "with --layers samples every layer instance); each event record drains the queue, "
                         "so events on every step cost the step about 14 us at decode size")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the extra timing of the same steps replayed from a captured HIP graph")
    ap.add_argument("--act-quant", action="store_true",
                    help="FP8 x FP8 expert matmuls on 1 x 128 quantised activations (FP8 weights only)")
    ap.add_argument("--variant", default="plain", choices=["plain", "renorm", "block"],
                    help="plain moe_forward; renormalised gate; or moe_block_forward (sandwich RMSNorms, "
                         "residual updated in place)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain device copy of known size (counter calibration)")
    return ap.parse_args()


class Hip:
    """hipEvent calls on the HIP runtime torch already loaded."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        ev = ctypes.c_void_p()
        st = self.lib.hipEventCreate(ctypes.byref(ev))
        if st != 0:
            raise RuntimeError(f"hipEventCreate failed: {st}")
        return ev.value

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        st = self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {st}")
        return float(ms.value)

    def destroy(self, ev):
        self.lib.hipEventDestroy(ev)


def copy_probe():
    import torch
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "launches": 3}), flush=True)


# source files that define each expert kernel (with the device helpers it uses)
KERNEL_SOURCES = {"gate_up_stream": ("stream.hip", "moe_common.h"), "down_stream": ("stream.hip", "moe_common.h"),
                  "gate_up_gemm": ("gemm.hip", "moe_common.h"), "down_gemm": ("gemm.hip", "moe_common.h")}


def kernel_sources_hash(kernel: str) -> str:
    """Hash of the sources of `kernel`: stored traffic counts are used only while it matches."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fine_grained_sparse_amd", "csrc")
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(name.encode() + fh.read())
    return h.hexdigest()[:16]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_probe:
        copy_probe()
        return

    from fine_grained_sparse_amd import binding as B
    from moe_inputs import generate, get_config

    cfg = get_config(args.workload)
    if args.tokens is not None:
        cfg = cfg.replace(n_tokens=args.tokens)
    N, d, E, k, f, fs = cfg.n_tokens, cfg.d_model, cfg.n_experts, cfg.top_k, cfg.d_ff, cfg.d_ff_shared
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = max(1, args.layers)
    print(f"[bench] workload={cfg.name} N={N} layers={L}: drawing inputs on the GPU", file=sys.stderr, flush=True)
    layers = []
    for li in range(L):
        inp = generate(cfg, seed=1000 + li, device="cuda", cache=False)
        layers.append(inp)
    torch.cuda.synchronize()

    x_torch_dtype = torch.float32 if cfg.x_dtype == "f32" else torch.bfloat16
    mods = [B.MoeLayer(k, inp, N, x_torch_dtype) for inp in layers]
    ws = mods[0].workspace
    for m in mods[1:]:
        m.workspace = ws  # one workspace, calls are stream-ordered
    outs = [torch.empty_like(inp["x"]) for inp in layers]
    flags = (B.MOE_FLAG_RENORMALIZE if args.variant == "renorm" else 0) | \
        (B.MOE_FLAG_FP8_ACT_QUANT if args.act_quant else 0)
    descs = [m.desc(N, flags) for m in mods]
    need = max(B.workspace_size(dsc) for dsc in descs)
    if need > ws.numel():
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    if args.variant == "block":
        need = max(int(B.lib().moe_block_workspace_size(ctypes.byref(dsc))) for dsc in descs)
        if need > ws.numel():
            ws = torch.empty(need, dtype=torch.uint8, device=dev)
        gen = torch.Generator(device="cuda").manual_seed(77)
        norms = [((1.0 + 0.1 * torch.randn(d, generator=gen, device="cuda")).to(torch.bfloat16).float(),
                  (1.0 + 0.1 * torch.randn(d, generator=gen, device="cuda")).to(torch.bfloat16).float())
                 for _ in range(L)]
    stream = torch.cuda.current_stream(dev).cuda_stream

    # routing of each instance (outside the timed region): touched experts
    touched = []
    for li, m in enumerate(mods):
        bufs = B.route_outputs(N, E, k, dev)
        st = B.forward_raw(descs[li], layers[li]["x"], layers[li]["router_w"], layers[li]["router_b"], m.weights,
                           outs[li], ws, B.aux_struct(bufs), stream)
        if st != B.MOE_OK:
            raise B.MoeError(st, "moe_forward")
        torch.cuda.synchronize()
        counts = np.diff(bufs["expert_offsets"].cpu().numpy())
        touched.append(int((counts > 0).sum()))

    hip = Hip()
    STAGE_GU, STAGE_DN = 3, 4
    n_ev = 2 * B.MOE_NUM_STAGES
    ev_arrays = []
    ev_handles = []
    stride = max(1, args.event_stride)
    sampled = list(range(0, args.steps, stride))   # timed steps that carry the kernel events
    for i in sampled:
        arr = (ctypes.c_void_p * n_ev)()
        hs = {}
        for s in (STAGE_GU, STAGE_DN):
            for j in (2 * s, 2 * s + 1):
                hs[j] = hip.event()
                arr[j] = hs[j]
        ev_arrays.append(arr)
        ev_handles.append(hs)
    aux_timed = {i: B.MoeAux(None, None, None, None, None, None, None, ctypes.cast(a, ctypes.c_void_p))
                 for i, a in zip(sampled, ev_arrays)}

    def step(i, aux=None, strm=None):
        li = i % L
        m = mods[li]
        strm = stream if strm is None else strm
        if args.variant == "block":
            # the layer instance's token batch is its residual stream, updated in place
            st = B.lib().moe_block_forward(ctypes.byref(descs[li]), layers[li]["x"].data_ptr(),
                                           norms[li][0].data_ptr(), norms[li][1].data_ptr(), 1e-6,
                                           layers[li]["router_w"].data_ptr(), layers[li]["router_b"].data_ptr(),
                                           ctypes.byref(m.weights), ws.data_ptr(), ws.numel(),
                                           ctypes.byref(aux) if aux is not None else None, strm)
            if st != B.MOE_OK:
                raise B.MoeError(st, "moe_block_forward")
            return
        st = B.lib().moe_forward(ctypes.byref(descs[li]), layers[li]["x"].data_ptr(),
                                 layers[li]["router_w"].data_ptr(), layers[li]["router_b"].data_ptr(),
                                 ctypes.byref(m.weights), outs[li].data_ptr(), ws.data_ptr(), ws.numel(),
                                 ctypes.byref(aux) if aux is not None else None, strm)
        if st != B.MOE_OK:
            raise B.MoeError(st, "moe_forward")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps); timing {args.steps} steps", file=sys.stderr, flush=True)

    cur = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, aux_timed.get(i))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    value = N * args.steps / elapsed

    # distribution of single steps: a second pass with an event pair around every step
    # (kept out of the timed loop above, where the extra events would cost time)
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        step_ev[i][0].record(cur)
        step(i)
        step_ev[i][1].record(cur)
    torch.cuda.synchronize()
    step_us = np.array([a.elapsed_time(b) * 1e3 for a, b in step_ev])
    step_stats = {"p10": round(float(np.percentile(step_us, 10)), 2), "median": round(float(np.median(step_us)), 2),
                  "p90": round(float(np.percentile(step_us, 90)), 2), "pass": "separate, one event pair per step"}

    # the same steps replayed from a HIP graph (one graph holds one step of every
    # layer instance); reported beside `value`, which stays the eager-launch rate
    graph = None
    if not args.no_graph:
        try:
            graph = graph_replay(torch, dev, cur, step, L, N, args.steps)
        except Exception as exc:   # a capture failure is reported, not fatal to the measurement
            graph = {"error": f"{type(exc).__name__}: {exc}"}

    # per-launch durations of the expert kernels from the library's events
    gu_ms = [hip.elapsed_ms(hs[2 * STAGE_GU], hs[2 * STAGE_GU + 1]) for hs in ev_handles]
    dn_ms = [hip.elapsed_ms(hs[2 * STAGE_DN], hs[2 * STAGE_DN + 1]) for hs in ev_handles]
    for hs in ev_handles:
        for e in hs.values():
            hip.destroy(e)

    sw = 1 if cfg.w_dtype == "fp8" else 2
    sx = 4 if cfg.x_dtype == "f32" else 2
    def sc_row(n_in):   # FP32 scale bytes per weight row of n_in inputs
        if cfg.w_dtype != "fp8":
            return 0
        return 4 * n_in / (128 * 128) if cfg.scale_block else 4   # per 128x128 block, or per output channel
    stream_path = N <= 192 and d <= 4096 and f <= 512 and fs <= 512   # the library's own rule
    kind = "stream" if stream_path else "gemm"

    # algorithmic bytes and flops per launch of the two expert kernels, for U
    # touched routed experts (+ the shared expert)
    def gu_bytes(U):   # touched experts' gate+up rows (+ shared), x read once
        return (U * 2 * f * (d * sw + sc_row(d)) + 2 * fs * (d * sw + sc_row(d)) + N * d * sx)

    def dn_bytes(U):   # touched experts' down rows (+ shared)
        return (U * d * (f * sw + sc_row(f)) + d * (fs * sw + sc_row(fs)))

    gu_flops = 2.0 * (N * k * 2 * f + N * 2 * fs) * d
    dn_flops = 2.0 * (N * k * f + N * fs) * d
    # the expert matmuls run bf16 (FP8 weights decoded), or FP8 x FP8 with quantised activations
    mfma_dtype = "fp8" if args.act_quant else "bf16"
    mfma_peak = MFMA_PEAK_TFLOPS[mfma_dtype]

    def roof(name, bytes_sum, flops_sum, secs, n):
        t_hbm = bytes_sum / (HBM_PEAK_GBS * 1e9)
        t_mfma = flops_sum / (mfma_peak * 1e12)
        hbm_frac = bytes_sum / secs / 1e9 / HBM_PEAK_GBS
        mfma_frac = flops_sum / secs / 1e12 / mfma_peak
        if t_hbm >= t_mfma:
            r = {"bound": "hbm", "achieved": round(bytes_sum / secs / 1e9, 1), "peak": HBM_PEAK_GBS,
                 "unit": "GB/s", "frac": round(hbm_frac, 4)}
        else:
            r = {"bound": "mfma", "achieved": round(flops_sum / secs / 1e12, 1), "peak": mfma_peak,
                 "unit": "TFLOP/s", "frac": round(mfma_frac, 4)}
        r.update({"kernel": name, "avg_launch_us": round(secs / n * 1e6, 2),
                  "algorithmic_bytes_per_launch": int(bytes_sum / n), "flops_per_launch": int(flops_sum / n),
                  "hbm_frac": round(hbm_frac, 4), f"mfma_frac_{mfma_dtype}": round(mfma_frac, 4)})
        return r

    gu_b = sum(gu_bytes(touched[i % L]) for i in sampled)
    dn_b = sum(dn_bytes(touched[i % L]) for i in sampled)
    gu_t, dn_t = sum(gu_ms) * 1e-3, sum(dn_ms) * 1e-3
    r_gu = roof(f"gate_up_{kind}", gu_b, gu_flops * len(sampled), gu_t, len(gu_ms))
    r_dn = roof(f"down_{kind}", dn_b, dn_flops * len(sampled), dn_t, len(dn_ms))
    dom = r_gu if gu_t >= dn_t else r_dn

    layer_bytes = [N * d * sx + E * d * 4 + E * 4 + touched[li] * 3 * (d * f * sw)
                   + touched[li] * (2 * f * sc_row(d) + d * sc_row(f))
                   + 3 * d * fs * sw + 2 * fs * sc_row(d) + d * sc_row(fs) + N * d * sx for li in range(L)]
    layer_b = sum(layer_bytes[i % L] for i in range(args.steps))
    layer_flops = (2.0 * N * d * E + gu_flops + dn_flops) * args.steps

    traffic = None
    tpath = os.path.join(ROOT, "profiles", f"traffic_{cfg.name}{'_aq' if args.act_quant else ''}.json")
    if os.path.exists(tpath):
        with open(tpath) as fh:
            tr = json.load(fh)
        if tr.get("kernel") == dom["kernel"] and tr.get("kernel_sources_hash") == kernel_sources_hash(dom["kernel"]):
            traffic = tr.get("bytes_per_launch")

    roofline = {k2: dom[k2] for k2 in ("bound", "achieved", "peak", "unit", "frac")}
    roofline["traffic"] = traffic
    roofline.update({k2: v for k2, v in dom.items() if k2 not in roofline})
    roofline["other_expert_kernel"] = r_dn if dom is r_gu else r_gu
    roofline["timing"] = (f"HIP events around the expert kernels on every {stride}-th timed step "
                          f"({len(sampled)} of {args.steps})")
    roofline["whole_step"] = {"hbm_frac": round(layer_b / elapsed / 1e9 / HBM_PEAK_GBS, 4),
                              f"mfma_frac_{mfma_dtype}": round(layer_flops / elapsed / 1e12 / mfma_peak, 4),
                              "algorithmic_bytes": int(layer_b / args.steps),
                              "flops": int(layer_flops / args.steps)}

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": ("bf16" if cfg.w_dtype == "bf16" else "fp8" if args.act_quant else "fp8-weights/bf16"),
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: N={N} d={d} E={E} top_k={k} f={f} f_shared={fs} "
                               f"x={cfg.x_dtype} w={cfg.w_dtype}"
                               + (f" scales={cfg.scale_block}x{cfg.scale_block}" if cfg.scale_block else "")
                               + f" bias={cfg.bias_kind}",
                   "n_tokens": N, "layers_cycled": L, "touched_experts": touched, "expert_path": kind,
                   "variant": args.variant, "act_quant": bool(args.act_quant)},
        "roofline": roofline,
        "step_us": step_stats,
    }
    if graph is not None:
        result["graph_replay"] = graph

    if not args.no_cpu_baseline and args.variant == "plain" and not args.act_quant:
        result["cpu_baseline"], result["parity_step0"] = cpu_baseline(cfg, layers[0], outs, mods, descs, ws, stream,
                                                                       args.cpu_seconds)
    print(json.dumps(result), flush=True)


def graph_replay(torch, dev, cur, step, L, N, steps):
    """Capture one step of every layer instance in a HIP graph and time its replays."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(dev)
    side.wait_stream(cur)
    with torch.cuda.stream(side):
        for i in range(L):   # warm the capture stream
            step(i, None, side.cuda_stream)
    cur.wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        cs = torch.cuda.current_stream(dev).cuda_stream
        for i in range(L):
            step(i, None, cs)
    reps = max(1, steps // L)
    g.replay()
    torch.cuda.synchronize()
    tg = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    gms = (time.perf_counter() - tg) * 1e3 / (reps * L)
    return {"ms_per_step": round(gms, 5), "tokens_per_s": round(N / gms * 1e3, 1), "replays": reps,
            "steps_per_replay": L}


def cpu_baseline(cfg, inp0, outs, mods, descs, ws, stream, target_s):
    """Time the CPU oracle on layer instance 0 (same inputs as the GPU steps)."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    import oracle.moe_oracle as O
    from fine_grained_sparse_amd import binding as B
    from moe_inputs import to_numpy

    # recompute step 0's output for the parity line
    st = B.forward_raw(descs[0], inp0["x"], inp0["router_w"], inp0["router_b"], mods[0].weights, outs[0], ws,
                       None, stream)
    if st != B.MOE_OK:
        raise B.MoeError(st, "moe_forward")
    torch.cuda.synchronize()
    gpu_out = outs[0].float().cpu().numpy().astype(np.float64)
    npi = to_numpy(inp0)
    N = cfg.n_tokens
    if N > 256:
        # big batches: time the oracle on a token subset of the same batch
        sub = max(1, int(N * min(1.0, 256 / N)))
        toks = np.arange(sub)
        t0 = time.perf_counter()
        part = O.token_outputs(npi, toks, cfg.top_k, cfg.w_dtype)
        dt = time.perf_counter() - t0
        ref, done, sample = part["out64"], sub, f"oracle token_outputs on the first {sub} of {N} tokens, layer 0"
        err = np.abs(gpu_out[toks] - ref).max(axis=1) / np.abs(ref).max(axis=1)
    else:
        t0 = time.perf_counter()
        reps = 0
        while True:
            res = O.moe_forward(npi, cfg.top_k, cfg.w_dtype, cfg.x_dtype)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= target_s or reps >= 50:
                break
        done = reps * N
        sample = f"oracle moe_forward on layer 0's batch of {N} tokens, repeated {reps}x"
        ref = res["out64"]
        err = np.abs(gpu_out - ref).max(axis=1) / np.abs(ref).max(axis=1)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    cpu = {"value": round(done / dt, 3), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
           "sample": sample, "seconds": round(dt, 2), "host_cpus": os.cpu_count()}
    return cpu, {"max_rel_err": float(err.max()), "tokens": int(len(err))}


if __name__ == "__main__":
    main()
