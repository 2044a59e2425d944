"""GPU parity of every C entry point against the CPU oracle (needs MI355X).

Every workload, small and full size (in the launch configuration the
benchmark uses), is compared element by element: routing, counts, offsets,
split sizes and the permutation bit-exactly (near-tie tokens aside, counted
and reported), routing weights within 1e-5, every layer output within
1e-2 + 2e-2 |ref|. Each test prints its near-tie counts (and the split sizes
over the logical ranks) on a "[parity]" line.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_fp32_amd as moe
from oracle import moe_oracle as om
import workloads as wl
from parity import (assert_out_close, check_logits, check_routing, np32, npi, print_report,
                    to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_and_library():
    # Fail, not skip: these tests exist to run on the GPU with the HIP library.
    assert torch.cuda.is_available(), "no GPU visible"
    moe.load_library()
    yield
    torch.cuda.synchronize()


def _desc(w: wl.Workload, T=None):
    return moe.make_desc(T=w.T if T is None else T, D=w.D, E=w.E, top_k=w.k, I=w.I,
                         ep_size=w.ep_size, ep_rank=w.ep_rank, dtype=w.dtype,
                         I_shared=w.I_shared)


def _oracle_router(inp, w):
    return om.router(np32(inp["x"][:w.T] if w.rank_share else inp["x"]), np32(inp["w_router"]),
                     w.k, np32(inp["logit_bias"]))


SMALL = {
    "tiny_fp32": wl.WORKLOADS["tiny_fp32"],
    "worked_example_geometry": wl.WORKLOADS["worked_example_geometry"],
    "ragged_bf16": wl.Workload("ragged_bf16", T=333, D=192, E=12, k=3, I=320, ep_size=3),
    "ragged_f32": wl.Workload("ragged_f32", T=77, D=64, E=5, k=2, I=128, dtype="f32"),
    "k_equals_E": wl.Workload("k_equals_E", T=130, D=128, E=4, k=4, I=192),
    "one_expert": wl.Workload("one_expert", T=65, D=64, E=1, k=1, I=64),
    "zipf_small": wl.Workload("zipf_small", T=600, D=128, E=32, k=4, I=128, zipf_s=3.0,
                              return_logits=True),
}


def _run_layer(w, inp_d, packed=False):
    d = _desc(w)
    lay = moe.LayerForward(d, inp_d["w_router"], inp_d["w_gate_up"], inp_d["w_down"],
                           logit_bias=inp_d["logit_bias"], shared_gate_up=inp_d["shared_gate_up"],
                           shared_down=inp_d["shared_down"], want_logits=True, packed=packed)
    lay(inp_d["x"])
    torch.cuda.synchronize()
    return lay


@pytest.mark.parametrize("name", sorted(SMALL))
def test_layer_forward_full_compare(name):
    """Every output of moe_layer_forward, element by element."""
    w = SMALL[name]
    inp = wl.make_inputs(w, seed=0)
    lay = _run_layer(w, to_dev(inp))
    x = np32(inp["x"])
    ref_r = om.router(x, np32(inp["w_router"]), w.k, np32(inp["logit_bias"]))
    check_logits(np32(lay.logits), ref_r["logits"])
    routing, rep = check_routing(npi(lay.topk_idx), np32(lay.topk_w), ref_r)
    print_report(name, rep, npi(lay.split))
    ref = om.layer_forward(x, np32(inp["w_router"]), np32(inp["w_gate_up"]), np32(inp["w_down"]),
                           w.k, ep_size=w.ep_size, logit_bias=np32(inp["logit_bias"]),
                           routing=routing)
    assert np.array_equal(npi(lay.counts), ref["counts"])
    assert np.array_equal(npi(lay.offsets), ref["offsets"])
    assert np.array_equal(npi(lay.split), ref["split"])
    M = int(ref["offsets"][-1])
    assert M == w.T * w.k
    assert np.array_equal(npi(lay.perm_src)[:M], ref["perm_src"])
    assert np.array_equal(npi(lay.pos), ref["pos"])
    assert_out_close(np32(lay.out), ref["out"], f"{name} layer output")


@pytest.mark.parametrize("name", sorted(SMALL))
def test_stepwise_entry_points(name):
    """moe_route -> moe_permute -> moe_expert_ffn -> moe_unpermute_combine,
    each fed the same inputs as the oracle's step."""
    w = SMALL[name]
    inp = wl.make_inputs(w, seed=1)
    dv = to_dev(inp)
    d = _desc(w)
    T, D, E, k = w.T, w.D, w.E, w.k
    dev = "cuda"
    dt = w.torch_dtype
    logits = torch.empty(T, E, device=dev)
    probs = torch.empty(T, E, device=dev)
    idx = torch.empty(T, k, dtype=torch.int32, device=dev)
    wts = torch.empty(T, k, device=dev)
    moe.moe_route(d, dv["x"], dv["w_router"], dv["logit_bias"], logits, probs, idx, wts)
    torch.cuda.synchronize()
    x = np32(inp["x"])
    ref_r = om.router(x, np32(inp["w_router"]), k, np32(inp["logit_bias"]))
    check_logits(np32(logits), ref_r["logits"])
    assert float(np.abs(np32(probs) - ref_r["probs"]).max()) <= 1e-5
    routing, _ = check_routing(npi(idx), np32(wts), ref_r)

    # permute over a sub-range of experts, fed the GPU's own routing
    gidx = npi(idx)
    for (eb, ee) in [(0, E), (E // 3, max(E // 3 + 1, 2 * E // 3))]:
        n = ee - eb
        cap = T * min(k, n)
        counts = torch.empty(n, dtype=torch.int32, device=dev)
        offsets = torch.empty(n + 1, dtype=torch.int32, device=dev)
        split = torch.empty(w.ep_size, dtype=torch.int32, device=dev)
        perm_src = torch.full((cap,), -7, dtype=torch.int32, device=dev)
        pos = torch.empty(T, k, dtype=torch.int32, device=dev)
        x_perm = torch.empty(cap, D, dtype=dt, device=dev)
        ws = moe.workspace(moe.moe_permute_workspace_size(d, eb, ee))
        moe.moe_permute(d, dv["x"], idx, eb, ee, cap, counts, offsets, split, perm_src, pos,
                        x_perm, ws)
        torch.cuda.synchronize()
        c = om.counts_offsets_splits(gidx, eb, ee, E, w.ep_size)
        p = om.permute(x, gidx, eb, ee)
        M = int(c["offsets"][-1])
        assert np.array_equal(npi(counts), c["counts"])
        assert np.array_equal(npi(offsets), c["offsets"])
        assert np.array_equal(npi(split), c["split"])
        assert np.array_equal(npi(perm_src)[:M], p["perm_src"])
        assert np.all(npi(perm_src)[M:] == -7)  # rows past the end are untouched
        assert np.array_equal(npi(pos), p["pos"])
        assert torch.equal(x_perm[:M].cpu(), inp["x"][torch.from_numpy(p["perm_src"])])

    # expert FFN on the full-range permutation, fed the oracle's x_perm
    c = om.counts_offsets_splits(routing[0], 0, E, E, w.ep_size)
    p = om.permute(x, routing[0], 0, E)
    M = int(c["offsets"][-1])
    xp = inp["x"][torch.from_numpy(p["perm_src"])].to(dev)
    off_d = torch.from_numpy(c["offsets"].astype(np.int32)).to(dev)
    y = torch.empty(M, D, dtype=torch.float32, device=dev)
    ws = moe.workspace(moe.moe_ffn_workspace_size(d, w.I, M))
    moe.moe_expert_ffn(d, E, w.I, M, xp, off_d, dv["w_gate_up"], dv["w_down"], y, ws)
    torch.cuda.synchronize()
    y_ref = om.expert_ffn(np32(xp), c["offsets"], np32(inp["w_gate_up"]), np32(inp["w_down"]))
    scale = float(np.sqrt(np.mean(y_ref ** 2))) if M else 1.0
    # the expert output on its own, at a tolerance relative to its scale
    assert_out_close(np32(y), y_ref, f"{name} expert FFN", rtol=2e-2, atol=1e-2 * scale)

    # combine, fed the oracle's y_perm rounded to fp32
    y_in = torch.from_numpy(y_ref.astype(np.float32))
    out = torch.empty(T, D, dtype=dt, device=dev)
    pos_d = torch.from_numpy(p["pos"].astype(np.int32)).to(dev)
    w_d = torch.from_numpy(routing[1].astype(np.float32)).to(dev)
    moe.moe_unpermute_combine(d, y_in.to(dev), pos_d, w_d, dv["x"], None, 0, T, out)
    torch.cuda.synchronize()
    ref_out = om.combine(np32(y_in), p["pos"], np32(w_d), residual=x)
    assert_out_close(np32(out), ref_out, f"{name} combine", rtol=1e-2, atol=1e-3)


@pytest.mark.gpu
@pytest.mark.parametrize("copy_rows", [True, False])
def test_permute_large_token_blocks(copy_rows):
    """Many tokens x experts: the block-count table outgrows one scan's LDS at
    256-token blocks, so blocks of 512 tokens are used and a workgroup's share
    of a block spans two 256-token chunks (with and without the row copy)."""
    T, D, E, k = 194 * 256, 64, 64, 2
    rng = np.random.default_rng(7)
    first = rng.integers(0, E, size=T)
    second = (first + rng.integers(1, E, size=T)) % E  # distinct from the first
    gidx = np.stack([first, second], axis=1).astype(np.int32)
    g = torch.Generator().manual_seed(7)
    x = torch.randn(T, D, generator=g).to(torch.bfloat16)
    w = wl.scaled(wl.WORKLOADS["worked_example_geometry"], T=T, D=D, E=E, k=k, ep_size=4)
    d = _desc(w)
    dev = "cuda"
    idx = torch.from_numpy(gidx).to(dev)
    xd = x.to(dev)
    for (eb, ee) in [(0, E), (10, 40)]:
        n = ee - eb
        cap = T * k
        counts = torch.empty(n, dtype=torch.int32, device=dev)
        offsets = torch.empty(n + 1, dtype=torch.int32, device=dev)
        split = torch.empty(w.ep_size, dtype=torch.int32, device=dev)
        perm_src = torch.full((cap,), -7, dtype=torch.int32, device=dev)
        pos = torch.empty(T, k, dtype=torch.int32, device=dev)
        x_perm = torch.empty(cap, D, dtype=torch.bfloat16, device=dev) if copy_rows else None
        ws = moe.workspace(moe.moe_permute_workspace_size(d, eb, ee))
        moe.moe_permute(d, xd, idx, eb, ee, cap, counts, offsets, split, perm_src, pos,
                        x_perm, ws)
        torch.cuda.synchronize()
        c = om.counts_offsets_splits(gidx, eb, ee, E, w.ep_size)
        p = om.permute(None, gidx, eb, ee)
        M = int(c["offsets"][-1])
        assert np.array_equal(npi(counts), c["counts"])
        assert np.array_equal(npi(offsets), c["offsets"])
        assert np.array_equal(npi(split), c["split"])
        assert np.array_equal(npi(perm_src)[:M], p["perm_src"])
        assert np.all(npi(perm_src)[M:] == -7)
        assert np.array_equal(npi(pos), p["pos"])
        if copy_rows:
            assert torch.equal(x_perm[:M].cpu(), x[torch.from_numpy(p["perm_src"])])


def test_determinism_and_stream():
    """Two runs on a side stream give bit-identical results."""
    w = SMALL["zipf_small"]
    inp = to_dev(wl.make_inputs(w, seed=2))
    s = torch.cuda.Stream()
    outs = []
    for _ in range(2):
        with torch.cuda.stream(s):
            lay = moe.LayerForward(_desc(w), inp["w_router"], inp["w_gate_up"], inp["w_down"],
                                   logit_bias=inp["logit_bias"], want_logits=True)
            lay(inp["x"], stream=s)
        s.synchronize()
        outs.append([t.clone() for t in (lay.out, lay.logits, lay.topk_idx, lay.topk_w,
                                         lay.perm_src, lay.pos)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_empty_and_zero_row_experts():
    """T = 0 is a no-op; experts that receive no tokens leave empty segments."""
    w = wl.Workload("empty", T=0, D=64, E=4, k=2, I=64)
    d = _desc(w)
    z = torch.zeros(0, 64, dtype=torch.bfloat16, device="cuda")
    moe.moe_route(d, z, torch.zeros(4, 64, device="cuda"), None, None, None,
                  torch.zeros(0, 2, dtype=torch.int32, device="cuda"),
                  torch.zeros(0, 2, device="cuda"))
    # a bias that sends every token to experts 3 and 1 only
    w2 = wl.Workload("zero_rows", T=300, D=64, E=6, k=2, I=64)
    inp = wl.make_inputs(w2, seed=4)
    inp["logit_bias"] = torch.tensor([0, 50, 0, 100, 0, 0], dtype=torch.float32)
    lay = _run_layer(w2, to_dev(inp))
    assert npi(lay.counts).tolist() == [0, 300, 0, 300, 0, 0]
    assert npi(lay.topk_idx).tolist() == [[3, 1]] * 300
    ref = om.layer_forward(np32(inp["x"]), np32(inp["w_router"]), np32(inp["w_gate_up"]),
                           np32(inp["w_down"]), 2, logit_bias=np32(inp["logit_bias"]))
    assert_out_close(np32(lay.out), ref["out"], "zero-row experts")


# More shapes: the router's wide-expert and two-token-block variants, the
# largest expert count and top-k the library takes, a shared expert inside
# moe_layer_forward, plain softmax weights, and a small rank share.
EXTRA = {
    "wide_experts": wl.Workload("wide_experts", T=600, D=64, E=256, k=8, I=64),
    "max_experts_topk": wl.Workload("max_experts_topk", T=70, D=64, E=1024, k=16, I=64),
    "router_two_blocks": wl.Workload("router_two_blocks", T=8192, D=64, E=128, k=2, I=64),
    "shared_expert": wl.Workload("shared_expert", T=200, D=128, E=8, k=2, I=128,
                                 I_shared=192),
}


@pytest.mark.parametrize("name", sorted(EXTRA))
def test_layer_forward_more_shapes(name):
    w = EXTRA[name]
    inp = wl.make_inputs(w, seed=5)
    lay = _run_layer(w, to_dev(inp))
    x = np32(inp["x"])
    ref_r = om.router(x, np32(inp["w_router"]), w.k, np32(inp["logit_bias"]))
    check_logits(np32(lay.logits), ref_r["logits"])
    routing, rep = check_routing(npi(lay.topk_idx), np32(lay.topk_w), ref_r)
    print_report(name, rep)
    ref = om.layer_forward(x, np32(inp["w_router"]), np32(inp["w_gate_up"]), np32(inp["w_down"]),
                           w.k, ep_size=w.ep_size, logit_bias=np32(inp["logit_bias"]),
                           shared_gate_up=np32(inp["shared_gate_up"]),
                           shared_down=np32(inp["shared_down"]), routing=routing)
    assert np.array_equal(npi(lay.counts), ref["counts"])
    assert np.array_equal(npi(lay.offsets), ref["offsets"])
    assert np.array_equal(npi(lay.perm_src), ref["perm_src"])
    assert np.array_equal(npi(lay.pos), ref["pos"])
    assert_out_close(np32(lay.out), ref["out"], f"{name} layer output")


def test_route_plain_softmax_weights():
    """norm_topk = 0: the routing weights are the full softmax values."""
    w = wl.Workload("plain", T=300, D=128, E=16, k=3, I=64)
    inp = wl.make_inputs(w, seed=6)
    dv = to_dev(inp)
    d = moe.make_desc(T=w.T, D=w.D, E=w.E, top_k=w.k, I=w.I, norm_topk=False)
    idx = torch.empty(w.T, w.k, dtype=torch.int32, device="cuda")
    wts = torch.empty(w.T, w.k, device="cuda")
    probs = torch.empty(w.T, w.E, device="cuda")
    moe.moe_route(d, dv["x"], dv["w_router"], None, None, probs, idx, wts)
    torch.cuda.synchronize()
    ref = om.router(np32(inp["x"]), np32(inp["w_router"]), w.k, norm_topk=False)
    assert float(np.abs(np32(probs) - ref["probs"]).max()) <= 1e-5
    routing, _ = check_routing(npi(idx), np32(wts), ref, norm_topk=False)
    assert float(np.abs(np32(wts) - ref["topk_w"]).max()) <= 1e-5
    assert np.all(np32(wts).sum(1) < 1.0)


@pytest.mark.parametrize("overlap,packed", [(True, False), (False, False), (False, True)])
def test_ep_rank_share_small(overlap, packed):
    """A small rank share (rank 1 of 4) with a shared expert, every output
    compared; with and without the shared expert on its own stream."""
    w = wl.Workload("share_small", T=96, D=128, E=16, k=4, I=128, ep_size=4,
                    rank_share=True, ep_rank=1, I_shared=64)
    inp = wl.make_inputs(w, seed=8)
    dv = to_dev(inp)
    run = moe.EPRankShareForward(w.T, w.D, w.E, w.k, w.I, w.ep_size, w.ep_rank, dv["x"],
                                 dv["w_router"], dv["w_gate_up"], dv["w_down"],
                                 shared_gate_up=dv["shared_gate_up"],
                                 shared_down=dv["shared_down"], I_shared=w.I_shared,
                                 overlap_shared=overlap, packed=packed)
    run.setup()
    run()
    torch.cuda.synchronize()
    x = np32(inp["x"])
    ref_r = om.router(x, np32(inp["w_router"]), w.k)
    routing, _ = check_routing(npi(run.idx_src), np32(run.w_src), ref_r)
    eb, ee = run.e_begin, run.e_end
    own = slice(w.ep_rank * w.T, (w.ep_rank + 1) * w.T)
    # receiver-side partials of every source token ...
    ref = om.layer_forward(x, np32(inp["w_router"]), np32(inp["w_gate_up"]),
                           np32(inp["w_down"]), w.k, ep_size=w.ep_size, e_begin=eb, e_end=ee,
                           routing=routing, residual=False)
    expect = ref["out"].astype(np.float64)
    # ... plus residual and shared expert on the own tokens
    expect[own] += x[own] + om.swiglu_ffn(x[own], np32(inp["shared_gate_up"]),
                                          np32(inp["shared_down"]))
    assert np.array_equal(npi(run.recv_counts), ref["counts"])
    assert np.array_equal(npi(run.recv_pos), ref["pos"])
    assert_out_close(np32(run.out_src), expect, "small rank share")


# ---------------------------------------------------------------------------
# Wide (256 x 256) tiles in both grouped GEMMs, every element of H and Y.
# ---------------------------------------------------------------------------
def test_wide_tiles_full_compare():
    """E = 8, 10000 ragged expert rows, D = I = 1536: both grouped GEMMs take
    256-row x 256-column tiles (asserted through the tile-shape query). Each
    expert's ~1250 rows make five 250-row blocks, so every tile ends in a
    partly filled 32-row slice and rows past it are zero-filled. H (fp16) and
    Y (fp32) are compared with the oracle in full, including each expert's
    last row block."""
    w = wl.Workload("wide_tiles", T=5000, D=1536, E=8, k=2, I=1536)
    d = _desc(w)
    M = w.T * w.k
    for gemm in (0, 1):
        rows, cols = moe.moe_ffn_tile_shape(d, w.E, w.I, M, True, gemm)
        assert (rows, cols) == (256, 256), (gemm, rows, cols)
    inp = wl.make_inputs(w, seed=11)
    x = np32(inp["x"])
    ref_r = om.router(x, np32(inp["w_router"]), w.k)
    routing = (ref_r["topk_idx"].astype(np.int64), ref_r["topk_w"])
    c = om.counts_offsets_splits(routing[0], 0, w.E, w.E, 1)
    p = om.permute(x, routing[0], 0, w.E)
    assert int(c["offsets"][-1]) == M
    xp = inp["x"][torch.from_numpy(p["perm_src"])].cuda()
    off = torch.from_numpy(c["offsets"].astype(np.int32)).cuda()
    h = torch.empty(M, w.I, dtype=torch.float16, device="cuda")
    y = torch.empty(M, w.D, dtype=torch.float32, device="cuda")
    dv = to_dev(inp)
    moe.moe_expert_gate_up(d, w.E, w.I, M, xp, off, dv["w_gate_up"], h)
    moe.moe_expert_down(d, w.E, w.I, M, h, off, dv["w_down"], y)
    torch.cuda.synchronize()
    wgu, wd = np32(inp["w_gate_up"]), np32(inp["w_down"])
    xpp = np32(xp).astype(np.float64)
    h_ref = np.zeros((M, w.I))
    for e in range(w.E):
        a, b = int(c["offsets"][e]), int(c["offsets"][e + 1])
        g = xpp[a:b] @ wgu[e][:, :w.I].astype(np.float64)
        u = xpp[a:b] @ wgu[e][:, w.I:].astype(np.float64)
        h_ref[a:b] = g / (1.0 + np.exp(-g)) * u
    # H: fp32 accumulation then one fp16 rounding (2^-11 relative)
    assert_out_close(np32(h), h_ref, "wide-tile H", rtol=2e-3, atol=1e-3)
    y_ref = om.expert_ffn(np32(xp), c["offsets"], wgu, wd)
    scale = float(np.sqrt(np.mean(y_ref ** 2)))
    assert_out_close(np32(y), y_ref, "wide-tile Y", rtol=2e-2, atol=1e-2 * scale)


def test_ptrs_ffn_against_oracle():
    """ModuleList-style experts (one buffer per expert, found through a device
    array of pointers; page "Expert Parallel (EP)", Requirements) against the
    oracle's expert FFN, on ragged segments with an empty expert."""
    w = wl.Workload("ptrs", T=700, D=256, E=6, k=2, I=320)
    inp = wl.make_inputs(w, seed=12)
    x = np32(inp["x"])
    g = np.random.default_rng(12)
    first = g.integers(0, w.E - 1, size=w.T)       # expert 5 gets no rows
    second = (first + g.integers(1, w.E - 1, size=w.T)) % (w.E - 1)
    idx = np.stack([first, second], 1)
    assert (idx[:, 0] != idx[:, 1]).all()
    c = om.counts_offsets_splits(idx, 0, w.E, w.E, 1)
    assert c["counts"][w.E - 1] == 0
    p = om.permute(x, idx, 0, w.E)
    M = int(c["offsets"][-1])
    d = _desc(w)
    xp = inp["x"][torch.from_numpy(p["perm_src"])].cuda()
    off = torch.from_numpy(c["offsets"].astype(np.int32)).cuda()
    gu_list = [inp["w_gate_up"][e].clone().cuda() for e in range(w.E)]
    dn_list = [inp["w_down"][e].clone().cuda() for e in range(w.E)]
    y = torch.empty(M, w.D, dtype=torch.float32, device="cuda")
    ws = moe.workspace(moe.moe_ffn_workspace_size(d, w.I, M))
    moe.moe_expert_ffn_ptrs(d, w.E, w.I, M, xp, off, gu_list, dn_list, y, ws)
    torch.cuda.synchronize()
    y_ref = om.expert_ffn(np32(xp), c["offsets"], np32(inp["w_gate_up"]), np32(inp["w_down"]))
    scale = float(np.sqrt(np.mean(y_ref ** 2)))
    assert_out_close(np32(y), y_ref, "pointer-array FFN", rtol=2e-2, atol=1e-2 * scale)


def test_h_saturates_at_fp16_max():
    """bf16 layers keep H in fp16: a gated activation beyond 65504 saturates
    to +-65504 (documented in moe.h) instead of becoming infinite. With
    x = 300/64 (exact in bf16) in every element and all-ones gate_up_proj,
    every gate and up pre-activation is exactly 300, so
    H = SiLU(300) * 300 = 90000 > 65504 saturates; with down_proj entries of
    +-2^-10, Y = +-64 * 65504 * 2^-10 exactly, finite."""
    D, I, M = 64, 64, 40
    d = moe.make_desc(T=M, D=D, E=1, top_k=1, I=I)
    x = torch.full((M, D), 300.0 / D, dtype=torch.float32).to(torch.bfloat16)
    assert float(x[0, 0]) * D == 300.0
    gu = torch.ones(1, D, 2 * I, dtype=torch.bfloat16)
    dn = torch.full((1, I, D), 2.0 ** -10, dtype=torch.bfloat16)
    dn[0, :, 1] = -(2.0 ** -10)
    h = torch.empty(M, I, dtype=torch.float16, device="cuda")
    y = torch.empty(M, D, dtype=torch.float32, device="cuda")
    off = torch.tensor([0, M], dtype=torch.int32, device="cuda")
    moe.moe_expert_gate_up(d, 1, I, M, x.cuda(), off, gu.cuda(), h)
    moe.moe_expert_down(d, 1, I, M, h, off, dn.cuda(), y)
    torch.cuda.synchronize()
    assert 300.0 / (1.0 + np.exp(-300.0)) * 300.0 > 65504.0
    assert torch.all(h == 65504.0), "H must saturate at the fp16 maximum"
    yy = y.cpu().numpy()
    assert np.isfinite(yy).all()
    assert np.all(yy[:, 0] == 65504.0 * I * 2.0 ** -10)
    assert np.all(yy[:, 1] == -65504.0 * I * 2.0 ** -10)


# ---------------------------------------------------------------------------
# Full-size workloads: every output element against the oracle.
# ---------------------------------------------------------------------------
@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["mixtral_style", "skewed_fine_grained",
                                  "worked_example_geometry"])
def test_full_size_layer(name):
    """The benchmark's workloads at full size, through moe_layer_forward:
    routing and permutation bit-exact, then every element of the layer output
    against the oracle's layer on the same routing (near-tie tokens take the
    GPU's valid choice)."""
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w, seed=0)
    dv = to_dev(inp)
    lay = _run_layer(w, dv)
    # the benchmark's layout: expert weights packed once; the same MFMAs on the
    # same values in the same order, except that with packed weights the gated
    # GEMM's last partial round of tiles runs split along K (fp32 sums of G
    # and U in another order): nearly every output element is identical, the
    # rest differ by a rounding step of H or of an fp16 expert row (up to
    # 2^-7 at |y| < 16, whatever the output's own size after the residual
    # cancels) and of the bf16 output
    lay_p = _run_layer(w, dv, packed=True)
    a, b = lay.out.float().cpu().numpy(), lay_p.out.float().cpu().numpy()
    same = float(np.mean(lay.out.view(torch.int16).cpu().numpy() ==
                         lay_p.out.view(torch.int16).cpu().numpy()))
    assert same >= 0.99, same
    assert_out_close(b, a, f"{name} packed vs stacked layer", rtol=8e-3, atol=1e-2)
    del dv, lay_p
    x = np32(inp["x"])
    ref_r = om.router(x, np32(inp["w_router"]), w.k, np32(inp["logit_bias"]))
    check_logits(np32(lay.logits), ref_r["logits"])
    routing, rep = check_routing(npi(lay.topk_idx), np32(lay.topk_w), ref_r)
    print_report(name, rep, npi(lay.split))
    ref = om.layer_forward(x, np32(inp["w_router"]), np32(inp["w_gate_up"]),
                           np32(inp["w_down"]), w.k, ep_size=w.ep_size,
                           logit_bias=np32(inp["logit_bias"]), routing=routing)
    assert ref["counts"].sum() == w.T * w.k
    assert np.array_equal(npi(lay.counts), ref["counts"])
    assert np.array_equal(npi(lay.offsets), ref["offsets"])
    assert np.array_equal(npi(lay.split), ref["split"])
    assert np.array_equal(npi(lay.perm_src), ref["perm_src"])
    assert np.array_equal(npi(lay.pos), ref["pos"])
    if w.zipf_s > 0:
        assert (ref["counts"] == 0).any(), "the Zipf bias should leave some experts empty"
    out = np32(lay.out)
    del lay
    err = assert_out_close(out, ref["out"], f"{name} layer output (every element)")
    print(f"[parity] {name}: {out.size} output elements, max abs err {err:.3e}", flush=True)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("overlap,packed", [(False, True)])
def test_ep_rank_share_full_size(overlap, packed):
    """DeepSeek-V3-style rank share (rank 0 of 8 logical EP ranks): send-side
    and receive-side routing and permutation bit-exact; every row of the
    receiver-side output (32768 source tokens: the weighted sum over this
    rank's experts, plus residual and shared expert on the own 4096) against
    the oracle."""
    w = wl.WORKLOADS["deepseek_v3_rank_share"]
    inp = wl.make_inputs(w, seed=0)
    dv = to_dev(inp)
    run = moe.EPRankShareForward(w.T, w.D, w.E, w.k, w.I, w.ep_size, w.ep_rank, dv["x"],
                                 dv["w_router"], dv["w_gate_up"], dv["w_down"],
                                 shared_gate_up=dv["shared_gate_up"],
                                 shared_down=dv["shared_down"], I_shared=w.I_shared,
                                 overlap_shared=overlap, packed=packed)
    run.setup()
    logits = torch.empty(w.T, w.E, device="cuda")
    run(logits=logits)
    torch.cuda.synchronize()
    x = np32(inp["x"])
    ref_r = om.router(x, np32(inp["w_router"]), w.k)  # every source token
    own = slice(w.ep_rank * w.T, (w.ep_rank + 1) * w.T)
    check_logits(np32(logits), ref_r["logits"][own])
    routing, rep = check_routing(npi(run.idx_src), np32(run.w_src), ref_r)
    # send side (own tokens, all experts, split sizes over the 8 ranks)
    idx_own = routing[0][own]
    cs = om.counts_offsets_splits(idx_own, 0, w.E, w.E, w.ep_size)
    ps = om.permute(None, idx_own, 0, w.E)
    print_report("deepseek_v3_rank_share", rep, cs["split"])
    assert np.array_equal(npi(run.send_counts), cs["counts"])
    assert np.array_equal(npi(run.send_split), cs["split"])
    assert np.array_equal(npi(run.send_perm_src)[:w.T * w.k], ps["perm_src"])
    assert np.array_equal(npi(run.send_pos), ps["pos"])
    # receive side (every source pair whose expert is one of the 32 local ones)
    eb, ee = run.e_begin, run.e_end
    ref = om.layer_forward(x, np32(inp["w_router"]), np32(inp["w_gate_up"]),
                           np32(inp["w_down"]), w.k, ep_size=w.ep_size, e_begin=eb, e_end=ee,
                           routing=routing, residual=False)
    M = int(ref["offsets"][-1])
    assert np.array_equal(npi(run.recv_counts), ref["counts"])
    assert np.array_equal(npi(run.recv_offsets), ref["offsets"])
    assert np.array_equal(npi(run.recv_perm_src)[:M], ref["perm_src"])
    assert np.array_equal(npi(run.recv_pos), ref["pos"])
    expect = ref["out"]
    del ref
    expect[own] += x[own] + om.swiglu_ffn(x[own], np32(inp["shared_gate_up"]),
                                          np32(inp["shared_down"]))
    out = np32(run.out_src)
    err = assert_out_close(out, expect, "rank-share receiver-side output (every row)")
    print(f"[parity] deepseek_v3_rank_share: {out.size} output elements "
          f"({out.shape[0]} source tokens), M={M}, max abs err {err:.3e}", flush=True)
