#!/usr/bin/env python3
"""Benchmark of the MoE layer forward on one MI355X (gfx950).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--variant bf16|mxfp8|train]

A step is one full layer forward (route, counts/splits, permute, grouped
SiLU-gated expert FFN, weighted combine into the residual) over one batch of
synthetic inputs already resident in device memory, through the C ABI of
libmoe. W untimed steps, then K timed steps bracketed by device
synchronisation. Prints one JSON line with the throughput (tokens/s), the
roofline of the dominant kernel (the grouped gate_up GEMM with its SiLU-gate
epilogue, timed with HIP events on its own stream) and the CPU oracle timed on
a bounded sample of the same workload.

--variant mxfp8 runs the layer with its expert FFN in MXFP8 (activations
quantized after the permute, weights packed once at set-up) and reports the
MXFP8 gate_up GEMM against the FP8 matrix peak.

--variant train times a training step of the layer: the forward (keeping the
gate and up pre-activations), then the backward from a seeded output
gradient (input, router, expert and shared expert weight gradients). The
roofline is that of the step's largest kernel, the grouped weight-gradient
GEMM of gate_up_proj (HBM-bound: its fp32 gradient is most of its bytes).

Only one GPU is used: --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

DEFAULT_WORKLOAD = "worked_example_geometry"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 matrix peak
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 matrix peak (MXFP8 block-scaled included)
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
COUNTERS = {
    "bf16": os.path.join(ROOT, "profiles", "gate_up_gemm_{w}_counters.txt"),
    "mxfp8": os.path.join(ROOT, "profiles", "gate_up_gemm_mxfp8_{w}_counters.txt"),
    "train": os.path.join(ROOT, "profiles", "weight_grad_gemm_{w}_counters.txt"),
}
GEMM_SRC = {
    "bf16": os.path.join(ROOT, "mixture_experts_layer_fp32_amd", "csrc", "ffn_bf16.hip"),
    "mxfp8": os.path.join(ROOT, "mixture_experts_layer_fp32_amd", "csrc", "ffn_mxfp8.hip"),
    "train": os.path.join(ROOT, "mixture_experts_layer_fp32_amd", "csrc", "ffn_bwd.hip"),
}


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # A step of the default workload is ~0.2 ms of GPU work: 50 untimed steps
    # bring the clocks to their steady state (5 leave them ramping, ~15 %
    # slower) and 200 timed steps take well under a second.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--variant", choices=("bf16", "mxfp8", "train"), default="bf16",
                    help="expert FFN arithmetic: the workload's dtype, or MXFP8; or a "
                         "training step (forward + backward)")
    ap.add_argument("--kernel-launches", type=int, default=None,
                    help="launches of the dominant kernel timed on its own (default: --steps)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target duration of the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    return ap.parse_args(argv)


def source_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic(workload: str, variant: str = "bf16"):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None when it is absent or was taken on other kernel source."""
    path = COUNTERS[variant].format(w=workload)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        m = re.match(r"^\s*([a-z0-9_]+)\s*:\s*(\S+)", line)
        if m:
            kv[m.group(1)] = m.group(2)
    if kv.get("kernel_source_sha256_16") != source_hash(GEMM_SRC[variant]):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def events_avg_ms(fn, n: int, stream) -> float:
    """Average duration of fn() launched n times back to back on `stream`:
    HIP events recorded on that stream before the first launch and after the
    last (an event between launches would add its own cache write-back to
    every launch it follows)."""
    import torch
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        for _ in range(n):
            fn()
        ev1.record(stream)
    stream.synchronize()
    return ev0.elapsed_time(ev1) / n


def _oracle_layer_mxfp8(om, mo, x, wr, packed, k, ep_size, bias):
    """The oracle's layer forward with the MXFP8 expert FFN: its router,
    permute, counts and combine around the MXFP8 oracle FFN (weights packed
    beforehand, as the GPU layer packs them once at set-up)."""
    r = om.router(x, wr, k, bias)
    E = wr.shape[0]
    p = om.permute(x, r["topk_idx"], 0, E)
    c = om.counts_offsets_splits(r["topk_idx"], 0, E, E, ep_size)
    y = mo.expert_ffn_mxfp8_packed(p["x_perm"], c["offsets"], *packed)["y"]
    return om.combine(y, p["pos"], r["topk_w"], residual=x)


def cpu_baseline(w, inp, target_s: float, variant: str = "bf16"):
    """The CPU oracle (unchanged) on a bounded sample of the same workload."""
    from threadpoolctl import threadpool_info
    from oracle import moe_backward_oracle as ob
    from oracle import moe_oracle as om
    from oracle import mxfp8_oracle as mo

    f = lambda t: None if t is None else t.float().numpy()  # noqa: E731
    x_all = f(inp["x"])
    wr, bias = f(inp["w_router"]), f(inp["logit_bias"])
    wgu, wd = f(inp["w_gate_up"]), f(inp["w_down"])
    sgu, sd = f(inp["shared_gate_up"]), f(inp["shared_down"])
    if w.rank_share:
        x = x_all[w.ep_rank * w.T:(w.ep_rank + 1) * w.T]
        eb, ee = w.ep_rank * w.E_loc, (w.ep_rank + 1) * w.E_loc
    else:
        x, eb, ee = x_all, 0, w.E
    if variant == "mxfp8":
        packed = mo.pack_weights(wgu) + mo.pack_weights(wd)
    if variant == "train":
        import torch
        dout_all = torch.randn(w.T, w.D, generator=torch.Generator().manual_seed(1)).to(
            torch.bfloat16).float().numpy()
    # sample: consecutive chunks of tokens, until the target time is spent
    chunk = min(w.T, 1024)
    done = 0
    t0 = time.perf_counter()
    while True:
        s = (done // chunk) % max(1, w.T // chunk)
        xs = x[s * chunk:(s + 1) * chunk]
        if variant == "mxfp8":
            _oracle_layer_mxfp8(om, mo, xs, wr, packed, w.k, w.ep_size, bias)
        elif variant == "train":
            ob.layer_backward(xs, wr, wgu, wd, w.k, dout_all[s * chunk:(s + 1) * chunk],
                              logit_bias=bias, shared_gate_up=sgu, shared_down=sd)
        else:
            om.layer_forward(xs, wr, wgu, wd, w.k, ep_size=w.ep_size, e_begin=eb, e_end=ee,
                             logit_bias=bias, shared_gate_up=sgu, shared_down=sd)
        done += len(xs)
        el = time.perf_counter() - t0
        if el >= target_s or done >= 64 * w.T:
            break
    threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    return {"value": done / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} tokens ({chunk}-token chunks of the same workload, seed 0) "
                      f"through the full float64 oracle layer "
                      f"{'forward and backward' if variant == 'train' else 'forward'}"
                      f"{' (MXFP8 expert FFN, weights packed once beforehand)' if variant == 'mxfp8' else ''}"
                      f" in {el:.1f} s"}


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the layer forward "
              "here is one expert-parallel rank's share; nothing is sharded across GPUs.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import mixture_experts_layer_fp32_amd as moe
    import workloads as wl

    moe.load_library()  # raises if libmoe.so is missing: no fallback path exists
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    w = wl.WORKLOADS[args.workload]
    mx = args.variant == "mxfp8"
    train = args.variant == "train"
    if mx and (w.rank_share or w.dtype != "bf16" or w.I_shared > 0):
        raise SystemExit(f"--variant mxfp8 takes a bf16 workload without rank share or shared "
                         f"expert ({w.name} is not one)")
    if train and w.rank_share:
        raise SystemExit(f"--variant train takes a workload without rank share "
                         f"({w.name} is not one)")
    dev = torch.device("cuda:0")
    inp = wl.make_inputs(w, seed=0)
    g = {k: (None if v is None else v.to(dev)) for k, v in inp.items()}
    stream = torch.cuda.current_stream(dev)

    if w.rank_share:
        run = moe.EPRankShareForward(w.T, w.D, w.E, w.k, w.I, w.ep_size, w.ep_rank, g["x"],
                                     g["w_router"], g["w_gate_up"], g["w_down"],
                                     logit_bias=g["logit_bias"],
                                     shared_gate_up=g["shared_gate_up"],
                                     shared_down=g["shared_down"], I_shared=w.I_shared,
                                     dtype=w.dtype)
        run.setup()
        logits = torch.empty(w.T, w.E, device=dev) if w.return_logits else None
        step = lambda: run(logits=logits)  # noqa: E731
    else:
        d = moe.make_desc(T=w.T, D=w.D, E=w.E, top_k=w.k, I=w.I, ep_size=w.ep_size,
                          dtype=w.dtype, I_shared=w.I_shared)
        if train:
            lay = moe.LayerTrain(d, g["w_router"], g["w_gate_up"], g["w_down"],
                                 logit_bias=g["logit_bias"], shared_gate_up=g["shared_gate_up"],
                                 shared_down=g["shared_down"])
            dout = torch.randn(w.T, w.D, generator=torch.Generator().manual_seed(1)).to(
                w.torch_dtype).to(dev)
        elif mx:
            lay = moe.LayerForwardMXFP8(d, g["w_router"], g["w_gate_up"], g["w_down"],
                                        logit_bias=g["logit_bias"],
                                        want_logits=w.return_logits)
        else:
            lay = moe.LayerForward(d, g["w_router"], g["w_gate_up"], g["w_down"],
                                   logit_bias=g["logit_bias"],
                                   shared_gate_up=g["shared_gate_up"],
                                   shared_down=g["shared_down"], want_logits=w.return_logits)
        if train:
            def step():
                lay.forward(g["x"])
                lay.backward(dout)
        else:
            step = lambda: lay(g["x"])  # noqa: E731

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_s = t1 - t0
    ms_per_step = wall_s / args.steps * 1e3
    gpu_ms_per_step = ev0.elapsed_time(ev1) / args.steps
    tokens_per_s = w.T * args.steps / wall_s
    print(f"[bench] {w.name}: {args.steps} steps, {ms_per_step:.4f} ms/step (wall), "
          f"{gpu_ms_per_step:.4f} ms/step (events), {tokens_per_s:,.0f} tokens/s",
          file=sys.stderr, flush=True)

    if train:
        return finish_train(args, w, lay, g, d, dev, stream, tokens_per_s, ms_per_step,
                            gpu_ms_per_step, inp)

    # ---- the dominant kernel on the same rows: grouped gate_up GEMM + SiLU gate ----
    if w.rank_share:
        n_exp, x_perm, offsets = w.E_loc, run.x_recv, run.recv_offsets
        d_ffn = run.d_src
        cap = run.recv_cap
        w_gu, w_dn = g["w_gate_up"], g["w_down"]
    else:
        n_exp, d_ffn, cap = w.E, d, w.T * w.k
        offsets = lay.offsets
        x_perm = torch.empty(cap, w.D, dtype=w.torch_dtype, device=dev)
        pws = moe.workspace(moe.moe_permute_workspace_size(d, 0, w.E))
        tmp = [torch.empty_like(t) for t in (lay.counts, lay.offsets, lay.split)]
        moe.moe_permute(d, g["x"], lay.topk_idx, 0, w.E, cap, tmp[0], offsets, tmp[2],
                        torch.empty_like(lay.perm_src), torch.empty_like(lay.pos), x_perm, pws)
        w_gu, w_dn = g["w_gate_up"], g["w_down"]
    torch.cuda.synchronize()
    M = int(offsets[-1].item())
    h_dtype = torch.float16 if w.dtype == "bf16" else torch.float32
    h = torch.empty(cap, w.I, dtype=h_dtype, device=dev)
    y = torch.empty(cap, w.D, dtype=torch.float32, device=dev)
    L = args.kernel_launches or args.steps
    if mx:
        u8 = torch.uint8
        h = torch.empty(cap, w.I, dtype=torch.bfloat16, device=dev)
        xq = torch.empty(cap, w.D, dtype=u8, device=dev)
        xs = torch.empty(cap, w.D // 32, dtype=u8, device=dev)
        hq = torch.empty(cap, w.I, dtype=u8, device=dev)
        hs = torch.empty(cap, w.I // 32, dtype=u8, device=dev)
        moe.moe_mxfp8_quantize_rows(x_perm, xq, xs)
        gu = lambda: moe.moe_expert_gate_up_mxfp8(d_ffn, n_exp, w.I, cap, xq, xs,  # noqa: E731
                                                  offsets, lay.guq, lay.gus, h)
        gu()
        moe.moe_mxfp8_quantize_rows(h, hq, hs)
        dn = lambda: moe.moe_expert_down_mxfp8(d_ffn, n_exp, w.I, cap, hq, hs,  # noqa: E731
                                               offsets, lay.dq, lay.ds, y)
    else:
        gu = lambda: moe.moe_expert_gate_up(d_ffn, n_exp, w.I, cap, x_perm, offsets,  # noqa
                                            w_gu, h)
        dn = lambda: moe.moe_expert_down(d_ffn, n_exp, w.I, cap, h, offsets, w_dn, y)  # noqa
    gu()
    dn()
    gate_up_ms = events_avg_ms(gu, L, stream)
    down_ms = events_avg_ms(dn, L, stream)
    gu_flops = 2.0 * M * w.D * 2 * w.I
    dn_flops = 2.0 * M * w.I * w.D
    peak = PEAK_FP8_TFLOPS if mx else (PEAK_BF16_TFLOPS if w.dtype == "bf16"
                                        else PEAK_FP32_TFLOPS)
    achieved = gu_flops / (gate_up_ms * 1e-3) / 1e12
    expert_tflops = (gu_flops + dn_flops) / ((gate_up_ms + down_ms) * 1e-3) / 1e12
    traffic = read_traffic(w.name, args.variant) if w.dtype == "bf16" else None
    print(f"[bench] gate_up GEMM {gate_up_ms * 1e3:.1f} us ({achieved:.1f} TFLOP/s), "
          f"down GEMM {down_ms * 1e3:.1f} us, expert FFN {expert_tflops:.1f} TFLOP/s over "
          f"M={M} rows", file=sys.stderr, flush=True)

    # ---- permute and combine on their own: algorithmic HBM bytes / time ----
    mem = None
    if not w.rank_share:
        s_act = 2 if w.dtype == "bf16" else 4
        cnt = torch.empty_like(lay.counts)
        off = torch.empty_like(lay.offsets)
        spl = torch.empty_like(lay.split)
        psrc = torch.empty_like(lay.perm_src)
        ppos = torch.empty_like(lay.pos)
        pws = moe.workspace(moe.moe_permute_workspace_size(d, 0, w.E))
        out = torch.empty(w.T, w.D, dtype=w.torch_dtype, device=dev)
        perm = lambda: moe.moe_permute(d, g["x"], lay.topk_idx, 0, w.E, cap, cnt, off,  # noqa
                                       spl, psrc, ppos, x_perm, pws)
        comb = lambda: moe.moe_unpermute_combine(d, y, ppos, lay.topk_w, g["x"], None,  # noqa
                                                 0, w.T, out)
        lg = torch.empty(w.T, w.E, device=dev) if w.return_logits else None
        ridx = torch.empty_like(lay.topk_idx)
        rw = torch.empty_like(lay.topk_w)
        route = lambda: moe.moe_route(d, g["x"], g["w_router"], g["logit_bias"], lg,  # noqa
                                      None, ridx, rw)
        route()
        perm()
        comb()
        route_ms = events_avg_ms(route, L, stream)
        perm_ms = events_avg_ms(perm, L, stream)
        comb_ms = events_avg_ms(comb, L, stream)
        # router: tokens, gate weight (fp32), chosen ids and weights (+ logits)
        route_bytes = (w.T * w.D * s_act + w.E * w.D * 4 + w.T * w.k * 8
                       + (w.T * w.E * 4 if w.return_logits else 0))
        # permute: routing ids read, token rows read once, expert rows written,
        # perm_src and pos written; combine: expert outputs (fp32), positions
        # and weights, the residual read, the output written
        perm_bytes = w.T * w.k * 4 + w.T * w.D * s_act + M * w.D * s_act + 2 * M * 4
        comb_bytes = M * w.D * 4 + w.T * w.k * 8 + 2 * w.T * w.D * s_act
        mem = {"route_us": route_ms * 1e3,
               "route_gbs": route_bytes / (route_ms * 1e-3) / 1e9,
               "permute_us": perm_ms * 1e3,
               "permute_gbs": perm_bytes / (perm_ms * 1e-3) / 1e9,
               "combine_us": comb_ms * 1e3,
               "combine_gbs": comb_bytes / (comb_ms * 1e-3) / 1e9,
               "peak_gbs": PEAK_HBM_GBS}
        print(f"[bench] route {route_ms * 1e3:.1f} us ({mem['route_gbs']:.0f} GB/s), "
              f"permute {perm_ms * 1e3:.1f} us ({mem['permute_gbs']:.0f} GB/s), combine "
              f"{comb_ms * 1e3:.1f} us ({mem['combine_gbs']:.0f} GB/s)", file=sys.stderr,
              flush=True)

    if args.calibrate_copy_mib > 0:
        nbytes = args.calibrate_copy_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] calibration copy of {nbytes} bytes done", file=sys.stderr, flush=True)

    line = {
        "metric": "MoE layer tokens/sec at 1 GPU; grouped-GEMM MFMA util %; "
                  "permute/combine HBM GB/s",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8" if mx else ("bf16" if w.dtype == "bf16" else "f32"),
        "data": "synthetic (seeded N(0,1) tokens, N(0,0.02) weights)",
        "config": {"workload": w.name + ("+mxfp8_ffn" if mx else ""), "T": w.T, "D": w.D, "E": w.E, "top_k": w.k, "I": w.I,
                   "ep_size": w.ep_size, "rank_share": w.rank_share, "I_shared": w.I_shared,
                   "parallelism": "one GPU (one EP rank's share)"},
        "gpu_ms_per_step": gpu_ms_per_step,
        "expert_tflops": expert_tflops,
        "mfma_util": expert_tflops / peak if w.dtype == "bf16" else None,
        "expert_ffn": ("MXFP8: E4M3 elements, E8M0 scale per 32 along K, fp32 accumulation"
                       if mx else None),
        "kernels_us": {"gate_up_gemm": gate_up_ms * 1e3, "down_gemm": down_ms * 1e3},
        "permute_combine_hbm": mem,
        "roofline": {
            "kernel": ("ffn_gemm_mxfp8<kGateUp> (grouped MXFP8 gate_up GEMM + SiLU gate)" if mx
                       else "ffn_gemm_bf16<kGateUp> (grouped gate_up GEMM + SiLU gate)"),
            "bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
            "frac": achieved / peak, "traffic": traffic,
        },
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds, args.variant)
    print(json.dumps(line), flush=True)


def finish_train(args, w, lay, g, d, dev, stream, tokens_per_s, ms_per_step, gpu_ms_per_step,
                 inp):
    """Kernel timing and the JSON line of --variant train: the grouped
    weight-gradient GEMM of gate_up_proj (dW_gate_up = x_perm^T [dG | dU], the
    step's largest kernel), launched on its own on the routed rows of the
    step, timed with events on the launch stream."""
    import torch

    import mixture_experts_layer_fp32_amd as moe

    M = w.T * w.k
    s_act = 2 if w.dtype == "bf16" else 4
    gen = torch.Generator().manual_seed(2)
    # any dG | dU: values do not change the timing
    dgu = torch.randn(M, 2 * w.I, generator=gen).to(w.torch_dtype).to(dev)
    dwgu = torch.empty(w.E, w.D, 2 * w.I, device=dev)
    wgr = lambda: moe.moe_expert_weight_grad(d, w.E, M, lay.x_perm, w.D, dgu,  # noqa: E731
                                             2 * w.I, lay.offsets, dwgu)
    wgr()
    L = args.kernel_launches or args.steps
    wgr_ms = events_avg_ms(wgr, L, stream)
    flops = 2.0 * M * w.D * 2 * w.I
    tflops = flops / (wgr_ms * 1e-3) / 1e12
    # reads x_perm and dG | dU, writes dW_gate_up in fp32: those bytes at the
    # HBM peak take longer than the FLOPs at the bf16 matrix peak (HBM-bound)
    wgr_bytes = M * w.D * s_act + M * 2 * w.I * s_act + w.E * w.D * 2 * w.I * 4
    wgr_gbs = wgr_bytes / (wgr_ms * 1e-3) / 1e9
    print(f"[bench] weight-gradient GEMM (gate_up_proj) {wgr_ms * 1e3:.1f} us "
          f"({tflops:.1f} TFLOP/s, {wgr_gbs:.0f} GB/s)", file=sys.stderr, flush=True)
    if args.calibrate_copy_mib > 0:
        nbytes = args.calibrate_copy_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] calibration copy of {nbytes} bytes done", file=sys.stderr, flush=True)
    line = {
        "metric": "MoE layer tokens/sec at 1 GPU; grouped-GEMM MFMA util %; "
                  "permute/combine HBM GB/s",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) tokens and output gradient, N(0,0.02) weights)",
        "config": {"workload": w.name + "+backward", "T": w.T, "D": w.D, "E": w.E,
                   "top_k": w.k, "I": w.I, "ep_size": w.ep_size, "I_shared": w.I_shared,
                   "step": "forward + backward (input, router and expert weight gradients)",
                   "gate_up_preactivations": ("saved by the forward (fp32)"
                                              if lay.gu is not None else "recomputed"),
                   "parallelism": "one GPU (one EP rank's share)"},
        "gpu_ms_per_step": gpu_ms_per_step,
        "kernels_us": {"weight_grad_gemm": wgr_ms * 1e3},
        "roofline": {
            "kernel": "gemm_tn_bf16 (grouped weight gradient of gate_up_proj)",
            "bound": "hbm", "achieved": wgr_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": wgr_gbs / PEAK_HBM_GBS,
            "traffic": read_traffic(w.name, "train") if w.dtype == "bf16" else None,
            "tflops": tflops, "tflops_frac": tflops / PEAK_BF16_TFLOPS,
        },
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds, "train")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
