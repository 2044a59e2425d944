"""Packed expert weights (moe_pack_expert_weights, weight_layout = packed):
the layout against its definition, and the grouped GEMMs on packed weights
against the same GEMMs on the stacked tensors (bit for bit) and against the
oracle (needs MI355X)."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_fp32_amd as moe
from oracle import moe_oracle as om
import workloads as wl
from parity import assert_out_close, check_routing, np32, npi, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_and_library():
    assert torch.cuda.is_available(), "no GPU visible"
    moe.load_library()
    yield
    torch.cuda.synchronize()


def _expected_packed(w: torch.Tensor) -> torch.Tensor:
    """The packed order as the header defines it, by index arithmetic on the
    host: packed[e][cb][ks][l][j] = w[e][16 ks + 8 (l / 32) + j][32 cb + l % 32]."""
    n, K, N = w.shape
    v = w.reshape(n, K // 16, 2, 8, N // 32, 32)      # e, ks, l // 32, j, cb, l % 32
    v = v.permute(0, 4, 1, 2, 5, 3)                  # e, cb, ks, l // 32, l % 32, j
    return v.reshape(n, N // 32, K // 16, 64, 8).contiguous()


@pytest.mark.parametrize("n,D,I", [(3, 128, 192), (1, 256, 64)])
def test_pack_layout(n, D, I):
    g = torch.Generator().manual_seed(3)
    gu = torch.randn(n, D, 2 * I, generator=g).to(torch.bfloat16)
    dn = (torch.randn(n, I, D, generator=g) * 0.02).to(torch.bfloat16)
    dn[0, 0, :4] = torch.tensor([1e-6, -3e-7, 7e4, 0.0]).to(torch.bfloat16)  # subnormal, overflow
    d = moe.make_desc(T=1, D=D, E=n, top_k=1, I=I)
    pgu, pdn = moe.pack_expert_weights(d, gu.cuda(), dn.cuda())
    torch.cuda.synchronize()
    assert torch.equal(pgu.cpu().reshape(-1).view(torch.int16),
                       _expected_packed(gu).reshape(-1).view(torch.int16))
    # down_proj: bf16 -> fp16 with round-to-nearest-even (torch's conversion)
    exp_dn = _expected_packed(dn.float().to(torch.float16))
    assert torch.equal(pdn.cpu().reshape(-1).view(torch.int16),
                       exp_dn.reshape(-1).view(torch.int16))


def _ragged(T, E, k, seed):
    g = np.random.default_rng(seed)
    idx = np.stack([g.permutation(E)[:k] for _ in range(T)])
    return idx


@pytest.mark.parametrize("T,D,E,k,I", [
    (5000, 1536, 8, 2, 1536),   # 256 x 256 tiles in both GEMMs
    (700, 256, 6, 2, 320),      # 320-row persistent tiles, last column block partial
    (333, 192, 12, 3, 320),     # D and I not multiples of the tile widths
])
def test_packed_ffn_bit_identical_to_stacked(T, D, E, k, I):
    """Same MFMA operands in the same order: H and Y of the packed layout
    equal the stacked layout's bit for bit (also the dense shared-expert
    form, offsets = NULL)."""
    w = wl.Workload("packed", T=T, D=D, E=E, k=k, I=I)
    inp = wl.make_inputs(w, seed=21)
    idx = _ragged(T, E, k, 21)
    c = om.counts_offsets_splits(idx, 0, E, E, 1)
    p = om.permute(None, idx, 0, E)
    M = int(c["offsets"][-1])
    xp = inp["x"][torch.from_numpy(p["perm_src"])].cuda()
    off = torch.from_numpy(c["offsets"].astype(np.int32)).cuda()
    d = moe.make_desc(T=T, D=D, E=E, top_k=k, I=I)
    dp = moe.make_desc(T=T, D=D, E=E, top_k=k, I=I, packed=True)
    gu, dn = inp["w_gate_up"].cuda(), inp["w_down"].cuda()
    pgu, pdn = moe.pack_expert_weights(d, gu, dn)
    for offsets, n, rows in ((off, E, M), (None, 1, M)):
        wgu, wdn = (gu, dn) if offsets is not None else (gu[0], dn[0])
        qgu, qdn = (pgu, pdn) if offsets is not None else (pgu[0], pdn[0])
        h1 = torch.empty(rows, I, dtype=torch.float16, device="cuda")
        h2 = torch.empty_like(h1)
        y1 = torch.empty(rows, D, dtype=torch.float32, device="cuda")
        y2 = torch.empty_like(y1)
        moe.moe_expert_gate_up(d, n, I, rows, xp, offsets, wgu, h1)
        moe.moe_expert_down(d, n, I, rows, h1, offsets, wdn, y1)
        moe.moe_expert_gate_up(dp, n, I, rows, xp, offsets, qgu, h2)
        moe.moe_expert_down(dp, n, I, rows, h2, offsets, qdn, y2)
        torch.cuda.synchronize()
        assert torch.equal(h1.view(torch.int16), h2.view(torch.int16))
        assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))
    # and the fused two-GEMM call on packed weights
    y3 = torch.empty(M, D, dtype=torch.float32, device="cuda")
    ws = moe.workspace(moe.moe_ffn_workspace_size(dp, I, M))
    moe.moe_expert_ffn(dp, E, I, M, xp, off, pgu, pdn, y3, ws)
    torch.cuda.synchronize()
    y_ref = om.expert_ffn(np32(xp), c["offsets"], np32(inp["w_gate_up"]), np32(inp["w_down"]))
    scale = float(np.sqrt(np.mean(y_ref ** 2)))
    assert_out_close(np32(y3), y_ref, "packed expert FFN", rtol=2e-2, atol=1e-2 * scale)


@pytest.mark.parametrize("name", ["worked_example_geometry", "zipf_shared"])
def test_packed_layer_forward(name):
    """moe_layer_forward with packed routed and shared weights against the
    oracle (and bit-identical to the stacked layer)."""
    w = (wl.WORKLOADS[name] if name in wl.WORKLOADS else
         wl.Workload(name, T=900, D=256, E=32, k=4, I=192, I_shared=128, zipf_s=2.0,
                     return_logits=True))
    inp = wl.make_inputs(w, seed=0)
    dv = to_dev(inp)
    d = moe.make_desc(T=w.T, D=w.D, E=w.E, top_k=w.k, I=w.I, ep_size=w.ep_size,
                      I_shared=w.I_shared)
    outs = []
    for packed in (False, True):
        lay = moe.LayerForward(d, dv["w_router"], dv["w_gate_up"], dv["w_down"],
                               logit_bias=dv["logit_bias"], shared_gate_up=dv["shared_gate_up"],
                               shared_down=dv["shared_down"], want_logits=True, packed=packed)
        lay(dv["x"])
        torch.cuda.synchronize()
        outs.append(lay)
    assert torch.equal(outs[0].out.view(torch.int16), outs[1].out.view(torch.int16))
    lay = outs[1]
    x = np32(inp["x"])
    ref_r = om.router(x, np32(inp["w_router"]), w.k, np32(inp["logit_bias"]))
    routing, _ = check_routing(npi(lay.topk_idx), np32(lay.topk_w), ref_r)
    ref = om.layer_forward(x, np32(inp["w_router"]), np32(inp["w_gate_up"]), np32(inp["w_down"]),
                           w.k, ep_size=w.ep_size, logit_bias=np32(inp["logit_bias"]),
                           shared_gate_up=np32(inp["shared_gate_up"]),
                           shared_down=np32(inp["shared_down"]), routing=routing)
    assert np.array_equal(npi(lay.perm_src), ref["perm_src"])
    assert_out_close(np32(lay.out), ref["out"], f"{name} packed layer output")


def test_packed_ptrs_ffn():
    """ModuleList-style experts with packed per-expert buffers."""
    w = wl.Workload("ptrs_packed", T=500, D=256, E=5, k=2, I=192)
    inp = wl.make_inputs(w, seed=9)
    idx = _ragged(w.T, w.E, w.k, 9)
    c = om.counts_offsets_splits(idx, 0, w.E, w.E, 1)
    p = om.permute(None, idx, 0, w.E)
    M = int(c["offsets"][-1])
    xp = inp["x"][torch.from_numpy(p["perm_src"])].cuda()
    off = torch.from_numpy(c["offsets"].astype(np.int32)).cuda()
    dp = moe.make_desc(T=w.T, D=w.D, E=w.E, top_k=w.k, I=w.I, packed=True)
    gus, dns = [], []
    for e in range(w.E):
        a, b = moe.pack_expert_weights(dp, inp["w_gate_up"][e].cuda(), inp["w_down"][e].cuda())
        gus.append(a)
        dns.append(b)
    y = torch.empty(M, w.D, dtype=torch.float32, device="cuda")
    ws = moe.workspace(moe.moe_ffn_workspace_size(dp, w.I, M))
    moe.moe_expert_ffn_ptrs(dp, w.E, w.I, M, xp, off, gus, dns, y, ws)
    torch.cuda.synchronize()
    y_ref = om.expert_ffn(np32(xp), c["offsets"], np32(inp["w_gate_up"]), np32(inp["w_down"]))
    scale = float(np.sqrt(np.mean(y_ref ** 2)))
    assert_out_close(np32(y), y_ref, "packed pointer-array FFN", rtol=2e-2, atol=1e-2 * scale)
