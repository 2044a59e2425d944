#!/usr/bin/env python3
"""Benchmark of the MoE layer forward on one MI355X (gfx950).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--variant bf16|mxfp8|train] [--overlap-shared]

A step is one full layer forward (route, counts/splits, permute, grouped
SiLU-gated expert FFN, weighted combine into the residual) over one batch of
synthetic inputs already resident in device memory, through the C ABI of
libmoe. The default workload is the Mixtral-style layer (T = 8192 tokens,
D = 4096, 8 experts, top-2, I = 14336), the largest that fits one GPU.

Order of the run:
  1. each kernel of the path launched on its own on the step's inputs
     (router, permute, grouped gate_up GEMM, grouped down GEMM, combine; the
     shared expert where the workload has one): before every launch a 1 GiB
     read evicts the 256 MB last-level cache, and a pair of HIP events on the
     launch stream brackets the launch alone, so each duration is the
     kernel's own from HBM-resident inputs;
  2. W untimed steps, then K timed steps bracketed by device
     synchronisation; value = tokens per second over the K steps;
  3. the CPU oracle on a bounded sample of the same workload.
The JSON line carries the roofline of the dominant kernel (the grouped
gate_up GEMM with its SiLU-gate epilogue) against the bf16 matrix peak, the
router, permute and combine against the HBM peak (algorithmic bytes: each
expert row counted once at the activation width), the near-tie counts of
the routing (from the GPU's own fp32 logits) and the per-logical-rank split
sizes.

--variant mxfp8 runs the layer with its expert FFN in MXFP8 (activations
quantized after the permute, weights packed once at set-up) and reports the
MXFP8 gate_up GEMM against the FP8 matrix peak.

--variant train times a training step of the layer: the forward (keeping the
gate and up pre-activations), then the backward from a seeded output
gradient (input, router, expert and shared expert weight gradients). The
roofline is that of the step's largest kernel, the grouped weight-gradient
GEMM of gate_up_proj: HBM-bound where its bytes (mostly the fp32 gradient)
take longer at the HBM peak than its FLOPs at the bf16 matrix peak (small
expert batches), matrix-bound otherwise.

Only one GPU is used: --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

DEFAULT_WORKLOAD = "mixtral_style"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 matrix peak
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 matrix peak (MXFP8 block-scaled included)
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
FLUSH_BYTES = 1 << 30       # read before every standalone launch (> the 256 MB MALL)
NEAR_TIE = 1e-6             # k-th vs (k+1)-th fp32 logit gap reported as a near tie
COUNTERS = {
    "bf16": os.path.join(ROOT, "profiles", "layer_forward_{w}_counters.txt"),
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
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--variant", choices=("bf16", "mxfp8", "train"), default="bf16",
                    help="expert FFN arithmetic: the workload's dtype, or MXFP8; or a "
                         "training step (forward + backward)")
    ap.add_argument("--overlap-shared", action="store_true",
                    help="rank-share workload: run the shared expert on a second stream")
    ap.add_argument("--weights", choices=("packed", "stacked"), default="packed",
                    help="expert weight layout of the bf16 layer: packed once at set-up "
                         "(moe_pack_expert_weights; the pack is timed and reported) or the "
                         "stacked tensors as given")
    ap.add_argument("--kernel-launches", type=int, default=20,
                    help="flushed launches of each kernel timed on its own")
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


class Flushed:
    """Standalone kernel timing: before every launch a 1 GiB read on the
    launch stream evicts the 256 MB last-level cache (a read leaves its lines
    clean, so the timed kernel does not pay for writing back the flush's own
    data); a pair of HIP events on that stream brackets the launch alone."""

    def __init__(self, stream, device):
        import torch
        self.torch = torch
        self.stream = stream
        self.buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=device)
        self.sink = torch.empty((), dtype=torch.float32, device=device)

    def time(self, fn, n: int) -> dict:
        torch = self.torch
        pairs = []
        with torch.cuda.stream(self.stream):
            for _ in range(n):
                torch.sum(self.buf, dim=0, out=self.sink)
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(self.stream)
                fn()
                b.record(self.stream)
                pairs.append((a, b))
        self.stream.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in pairs)
        return {"mean_us": 1e3 * sum(ms) / len(ms), "median_us": 1e3 * statistics.median(ms),
                "p10_us": 1e3 * ms[len(ms) // 10], "p90_us": 1e3 * ms[(9 * len(ms)) // 10]}


def hbm_entry(t: dict, nbytes: float) -> dict:
    gbs = nbytes / (t["mean_us"] * 1e-6) / 1e9
    return {"us": t["mean_us"], "median_us": t["median_us"], "algorithmic_bytes": nbytes,
            "gbs": gbs, "frac": gbs / PEAK_HBM_GBS}


def near_ties(logits, k: int) -> int:
    """Tokens whose k-th and (k+1)-th fp32 logits (the GPU's) differ by less
    than 1e-6: their choice is the one reported apart from exact parity."""
    import torch
    if k >= logits.shape[1]:
        return 0
    top = torch.topk(logits, k + 1, dim=1).values
    return int(((top[:, k - 1] - top[:, k]) < NEAR_TIE).sum().item())


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


def standalone(args, w, g, lay, run, d, dev, stream, mx):
    """Each kernel of the path on its own (flushed, event-timed), on the same
    inputs and routing as the step. Returns (kernel timings, GEMM inputs,
    routing report)."""
    import torch

    import mixture_experts_layer_fp32_amd as moe

    fl = Flushed(stream, dev)
    L = args.kernel_launches
    s_act = 2 if w.dtype == "bf16" else 4
    t = {}
    rep = {}
    if w.rank_share:
        # the rank's own routing, its send permute over all experts, the
        # receive permute of every logical rank's pairs for the local experts
        E, k = w.E, w.k
        lg = torch.empty(w.T, E, device=dev)
        route = lambda: moe.moe_route(run.d_own, run.x_own, g["w_router"], g["logit_bias"],  # noqa
                                      lg, None, run.idx_own, run.w_own, ws=run.route_ws)
        psend = lambda: moe.moe_permute(run.d_own, run.x_own, run.idx_own, 0, E,  # noqa: E731
                                        run.send_cap, run.send_counts, run.send_offsets,
                                        run.send_split, run.send_perm_src, run.send_pos,
                                        run.x_send, run.send_ws)
        precv = lambda: moe.moe_permute(run.d_src, run.x_src, run.idx_src, run.e_begin,  # noqa
                                        run.e_end, run.recv_cap, run.recv_counts,
                                        run.recv_offsets, run.recv_split, run.recv_perm_src,
                                        run.recv_pos, run.x_recv, run.recv_ws)
        route()
        psend()
        precv()
        torch.cuda.synchronize()
        rep["near_ties"] = near_ties(lg, k)
        rep["split"] = [int(v) for v in run.send_split.cpu().tolist()]
        t["route"] = fl.time(route, L)
        t["permute_send"] = fl.time(psend, L)
        t["permute_recv"] = fl.time(precv, L)
        n_exp, x_perm, offsets, cap, d_ffn = (w.E_loc, run.x_recv, run.recv_offsets,
                                              run.recv_cap, run.d_src)
        w_gu, w_dn = run.w["w_gate_up"], run.w["w_down"]
        M = int(offsets[-1].item())
        # receive: every source pair's ids; token rows read once per token that
        # has a local pair; local rows written; perm_src and pos
        idx_all = run.idx_src
        has_local = ((idx_all >= run.e_begin) & (idx_all < run.e_end)).any(1)
        n_tok_local = int(has_local.sum().item())
        send_bytes = w.T * k * 4 + w.T * w.D * s_act + w.T * k * w.D * s_act + 2 * w.T * k * 4
        recv_bytes = (w.T_src * k * 4 + n_tok_local * w.D * s_act + M * w.D * s_act
                      + M * 4 + w.T_src * k * 4)
        route_bytes = w.T * w.D * s_act + w.E * w.D * 4 + w.T * k * 8
        shared = lambda: moe.moe_expert_ffn(run.d_own, 1, w.I_shared, w.T, run.x_own, None,  # noqa
                                            run.w["shared_gate_up"], run.w["shared_down"],
                                            run.shared_out, run.shared_ws)
    else:
        E, k = w.E, w.k
        lg = torch.empty(w.T, E, device=dev)
        ridx = torch.empty(w.T, k, dtype=torch.int32, device=dev)
        rw = torch.empty(w.T, k, device=dev)
        rws = moe.workspace(moe.moe_route_workspace_size(d), dev)
        route = lambda: moe.moe_route(d, g["x"], g["w_router"], g["logit_bias"], lg,  # noqa
                                      None, ridx, rw, ws=rws)
        cap = w.T * k
        cnt = torch.empty(E, dtype=torch.int32, device=dev)
        offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
        spl = torch.empty(w.ep_size, dtype=torch.int32, device=dev)
        psrc = torch.empty(cap, dtype=torch.int32, device=dev)
        ppos = torch.empty(w.T, k, dtype=torch.int32, device=dev)
        x_perm = torch.empty(cap, w.D, dtype=w.torch_dtype, device=dev)
        pws = moe.workspace(moe.moe_permute_workspace_size(d, 0, E))
        perm = lambda: moe.moe_permute(d, g["x"], ridx, 0, E, cap, cnt, offsets, spl,  # noqa
                                       psrc, ppos, x_perm, pws)
        route()
        perm()
        torch.cuda.synchronize()
        rep["near_ties"] = near_ties(lg, k)
        rep["split"] = [int(v) for v in spl.cpu().tolist()]
        t["route"] = fl.time(route, L)
        t["permute"] = fl.time(perm, L)
        n_exp, d_ffn = E, lay.d
        w_gu, w_dn = (lay.w["w_gate_up"], lay.w["w_down"]) if not mx else (None, None)
        M = int(offsets[-1].item())
        route_bytes = (w.T * w.D * s_act + w.E * w.D * 4 + w.T * k * 8
                       + (w.T * w.E * 4 if w.return_logits else 0))
        # routing ids, each token row read once, expert rows written, perm_src, pos
        perm_bytes = w.T * k * 4 + w.T * w.D * s_act + M * w.D * s_act + 2 * M * 4
    h_dtype = torch.float16 if w.dtype == "bf16" else torch.float32
    h = torch.empty(cap, w.I, dtype=h_dtype, device=dev)
    # expert outputs in the dtype the layer keeps them in (fp16 or fp32)
    y_dtype = torch.float16 if d_ffn.expert_out_dtype == moe.MOE_F16 else torch.float32
    y = torch.empty(cap, w.D, dtype=y_dtype, device=dev)
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
        # both GEMMs with their part buffers, as the layer runs them (the last
        # partial round of tiles split along K)
        gws = moe.workspace(moe.moe_gate_up_workspace_size(d_ffn, w.I, cap), dev)
        gu = lambda: moe.moe_expert_gate_up(d_ffn, n_exp, w.I, cap, x_perm, offsets,  # noqa
                                            w_gu, h, ws=gws)
        dws = moe.workspace(moe.moe_down_workspace_size(d_ffn, cap), dev)
        dn = lambda: moe.moe_expert_down(d_ffn, n_exp, w.I, cap, h, offsets, w_dn, y,  # noqa
                                         ws=dws)
    gu()
    dn()
    t["gate_up_gemm"] = fl.time(gu, L)
    t["down_gemm"] = fl.time(dn, L)
    # combine on the GEMM's outputs: each token's k expert rows (counted at
    # the activation width), weights and positions, residual, output
    if w.rank_share:
        shared()
        t["shared_ffn"] = fl.time(shared, L)
        out = torch.empty(w.T_src, w.D, dtype=w.torch_dtype, device=dev)
        comb = lambda: moe.moe_unpermute_combine(run.d_src, y, run.recv_pos, run.w_src,  # noqa
                                                 run.x_own, run.shared_out, run.r * w.T, w.T,
                                                 out)
        comb_bytes = (M * w.D * s_act + w.T_src * k * 8 + w.T_src * w.D * s_act
                      + w.T * w.D * s_act + w.T * w.D * s_act)
    else:
        out = torch.empty(w.T, w.D, dtype=w.torch_dtype, device=dev)
        comb = lambda: moe.moe_unpermute_combine(lay.d, y, ppos, rw, g["x"], None, 0,  # noqa
                                                 w.T, out)
        comb_bytes = M * w.D * s_act + w.T * k * 8 + 2 * w.T * w.D * s_act
    comb()
    t["combine"] = fl.time(comb, L)
    hbm = {"route": hbm_entry(t["route"], route_bytes),
           "combine": hbm_entry(t["combine"], comb_bytes)}
    if w.rank_share:
        hbm["permute_send"] = hbm_entry(t["permute_send"], send_bytes)
        hbm["permute_recv"] = hbm_entry(t["permute_recv"], recv_bytes)
    else:
        hbm["permute"] = hbm_entry(t["permute"], perm_bytes)
    return t, hbm, rep, M


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
    print(f"[bench] {w.name}: inputs resident", file=sys.stderr, flush=True)

    run = lay = d = None
    packed = args.weights == "packed" and w.dtype == "bf16" and not mx and not train
    pack_ms = None
    if packed:
        # the one-time pack of the expert weights (routed and shared), timed
        # on its own with events (the step then reads the packed copies)
        dp = moe.make_desc(T=w.T, D=w.D, E=w.E, top_k=w.k, I=w.I, ep_size=w.ep_size,
                           dtype=w.dtype, I_shared=w.I_shared)
        for _ in range(2):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            pk = moe.pack_expert_weights(dp, g["w_gate_up"], g["w_down"])
            if w.I_shared > 0:
                pk += moe.pack_expert_weights(dp, g["shared_gate_up"], g["shared_down"])
            e1.record(stream)
            torch.cuda.synchronize()
            pack_ms = e0.elapsed_time(e1)
            del pk
        print(f"[bench] expert weights packed in {pack_ms:.2f} ms (one-time set-up)",
              file=sys.stderr, flush=True)
    if w.rank_share:
        run = moe.EPRankShareForward(w.T, w.D, w.E, w.k, w.I, w.ep_size, w.ep_rank, g["x"],
                                     g["w_router"], g["w_gate_up"], g["w_down"],
                                     logit_bias=g["logit_bias"],
                                     shared_gate_up=g["shared_gate_up"],
                                     shared_down=g["shared_down"], I_shared=w.I_shared,
                                     dtype=w.dtype, overlap_shared=args.overlap_shared,
                                     packed=packed)
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
                                   shared_down=g["shared_down"], want_logits=w.return_logits,
                                   packed=packed)
        if train:
            def step():
                lay.forward(g["x"])
                lay.backward(dout)
        else:
            step = lambda: lay(g["x"])  # noqa: E731

    if train:
        kt = None
    else:
        kt, hbm, rep, M = standalone(args, w, g, lay, run, d, dev, stream, mx)
        print(f"[bench] standalone kernels (flushed, us): "
              + ", ".join(f"{k} {v['mean_us']:.1f}" for k, v in kt.items()),
              file=sys.stderr, flush=True)

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

    gu_us, dn_us = kt["gate_up_gemm"]["mean_us"], kt["down_gemm"]["mean_us"]
    gu_flops = 2.0 * M * w.D * 2 * w.I
    dn_flops = 2.0 * M * w.I * w.D
    peak = PEAK_FP8_TFLOPS if mx else (PEAK_BF16_TFLOPS if w.dtype == "bf16"
                                        else PEAK_FP32_TFLOPS)
    achieved = gu_flops / (gu_us * 1e-6) / 1e12
    expert_tflops = (gu_flops + dn_flops) / ((gu_us + dn_us) * 1e-6) / 1e12
    traffic = read_traffic(w.name, args.variant) if w.dtype == "bf16" else None
    print(f"[bench] gate_up GEMM {gu_us:.1f} us ({achieved:.1f} TFLOP/s), down GEMM "
          f"{dn_us:.1f} us ({dn_flops / (dn_us * 1e-6) / 1e12:.1f} TFLOP/s), expert FFN "
          f"{expert_tflops:.1f} TFLOP/s over M={M} rows", file=sys.stderr, flush=True)
    print("[bench] HBM: " + ", ".join(f"{k} {v['us']:.1f} us {v['gbs']:.0f} GB/s "
                                      f"({100 * v['frac']:.0f}%)" for k, v in hbm.items()),
          file=sys.stderr, flush=True)

    if args.calibrate_copy_mib > 0:
        nbytes = args.calibrate_copy_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] calibration copy of {nbytes} bytes done", file=sys.stderr, flush=True)

    cfg = {"workload": w.name + ("+mxfp8_ffn" if mx else ""), "T": w.T, "D": w.D, "E": w.E,
           "top_k": w.k, "I": w.I, "ep_size": w.ep_size, "rank_share": w.rank_share,
           "I_shared": w.I_shared, "parallelism": "one GPU (one EP rank's share)"}
    if w.rank_share:
        cfg["T_source"] = w.T_src
        cfg["shared_expert_stream"] = "second stream" if args.overlap_shared else "same stream"
    if w.dtype == "bf16" and not mx:
        cfg["expert_weights"] = ("packed once at set-up (moe_pack_expert_weights)" if packed
                                 else "stacked tensors as given")
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
        "config": cfg,
        "gpu_ms_per_step": gpu_ms_per_step,
        "expert_rows": M,
        "expert_tflops": expert_tflops,
        "mfma_util": expert_tflops / peak,
        "expert_ffn": ("MXFP8: E4M3 elements, E8M0 scale per 32 along K, fp32 accumulation"
                       if mx else None),
        "kernels_us": {k: v["mean_us"] for k, v in kt.items()},
        "weight_pack_ms": pack_ms,
        "kernel_timing": "each kernel launched alone, 1 GiB read (cache flush) before every "
                         f"launch, HIP events around the launch, mean of {args.kernel_launches}",
        "hbm": hbm,
        "routing": {"near_ties": rep["near_ties"], "near_tie_gap": NEAR_TIE,
                    "split_per_logical_rank": rep["split"]},
        "roofline": {
            "kernel": ("ffn_gemm_mxfp8<kGateUp> (grouped MXFP8 gate_up GEMM + SiLU gate)" if mx
                       else "ffn_gemm_bf16<kGateUp, packed=%s> (grouped gate_up GEMM + SiLU gate)"
                       % ("true" if packed else "false")),
            "bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
            "frac": achieved / peak, "traffic": traffic,
            "flop_per_launch": gu_flops, "avg_launch_us": gu_us,
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
    step (flushed, event-timed)."""
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
    t = Flushed(stream, dev).time(wgr, args.kernel_launches)
    wgr_ms = t["mean_us"] * 1e-3
    flops = 2.0 * M * w.D * 2 * w.I
    tflops = flops / (wgr_ms * 1e-3) / 1e12
    # reads x_perm and dG | dU, writes dW_gate_up in fp32. The bound is the
    # roof that takes longer: the bytes at the HBM peak (worked-example
    # geometry: 352 MB, 44 us, against 27 us of FLOPs) or the FLOPs at the
    # bf16 matrix peak (Mixtral-style: 1.54 ms, against 0.60 ms of bytes).
    wgr_bytes = M * w.D * s_act + M * 2 * w.I * s_act + w.E * w.D * 2 * w.I * 4
    wgr_gbs = wgr_bytes / (wgr_ms * 1e-3) / 1e9
    hbm_bound = wgr_bytes / (PEAK_HBM_GBS * 1e9) >= flops / (PEAK_BF16_TFLOPS * 1e12)
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
            **({"bound": "hbm", "achieved": wgr_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": wgr_gbs / PEAK_HBM_GBS} if hbm_bound else
               {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": tflops / PEAK_BF16_TFLOPS}),
            "traffic": read_traffic(w.name, "train") if w.dtype == "bf16" else None,
            "gbs": wgr_gbs, "tflops": tflops, "tflops_frac": tflops / PEAK_BF16_TFLOPS,
        },
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds, "train")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
