"""Expert outputs in fp16 (expert_out_dtype = MOE_F16): the down GEMM's fp16
output is its fp32 output rounded to nearest even (bit for bit, same
accumulators), and the combine over fp16 expert outputs matches the oracle
(needs MI355X)."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_fp32_amd as moe
from oracle import moe_oracle as om
import workloads as wl
from parity import assert_out_close, np32, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_and_library():
    assert torch.cuda.is_available(), "no GPU visible"
    moe.load_library()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("T,D,E,k,I,packed", [
    (5000, 1536, 8, 2, 1536, False),   # 256 x 256 tiles
    (5000, 1536, 8, 2, 1536, True),
    (700, 256, 6, 2, 320, False),      # 320-row persistent tiles
    (700, 256, 6, 2, 320, True),
])
def test_down_fp16_is_rounded_fp32(T, D, E, k, I, packed):
    w = wl.Workload("yh", T=T, D=D, E=E, k=k, I=I)
    inp = wl.make_inputs(w, seed=31)
    g = np.random.default_rng(31)
    idx = np.stack([g.permutation(E)[:k] for _ in range(T)])
    c = om.counts_offsets_splits(idx, 0, E, E, 1)
    p = om.permute(None, idx, 0, E)
    M = int(c["offsets"][-1])
    xp = inp["x"][torch.from_numpy(p["perm_src"])].cuda()
    off = torch.from_numpy(c["offsets"].astype(np.int32)).cuda()
    d32 = moe.make_desc(T=T, D=D, E=E, top_k=k, I=I, packed=packed)
    d16 = moe.make_desc(T=T, D=D, E=E, top_k=k, I=I, packed=packed, y_fp16=True)
    gu, dn = inp["w_gate_up"].cuda(), inp["w_down"].cuda()
    if packed:
        gu, dn = moe.pack_expert_weights(d32, gu, dn)
    h = torch.empty(M, I, dtype=torch.float16, device="cuda")
    y32 = torch.empty(M, D, dtype=torch.float32, device="cuda")
    y16 = torch.empty(M, D, dtype=torch.float16, device="cuda")
    moe.moe_expert_gate_up(d32, E, I, M, xp, off, gu, h)
    moe.moe_expert_down(d32, E, I, M, h, off, dn, y32)
    moe.moe_expert_down(d16, E, I, M, h, off, dn, y16)
    torch.cuda.synchronize()
    assert torch.isfinite(y32).all()
    assert torch.equal(y16.view(torch.int16), y32.to(torch.float16).view(torch.int16))


def test_combine_fp16_outputs_against_oracle():
    """The combine of fp16 expert outputs (and an fp16 shared expert output)
    against the oracle's combine of the same values."""
    w = wl.Workload("comb16", T=500, D=256, E=12, k=3, I=64, I_shared=64)
    inp = wl.make_inputs(w, seed=32)
    dv = to_dev(inp)
    g = np.random.default_rng(32)
    idx = np.stack([g.permutation(w.E)[:w.k] for _ in range(w.T)])
    p = om.permute(None, idx, 0, w.E)
    M = w.T * w.k
    y = (torch.randn(M, w.D, generator=torch.Generator().manual_seed(33)) * 3).to(torch.float16)
    sh = torch.randn(w.T, w.D, generator=torch.Generator().manual_seed(34)).to(torch.float16)
    wts = torch.rand(w.T, w.k, generator=torch.Generator().manual_seed(35))
    d = moe.make_desc(T=w.T, D=w.D, E=w.E, top_k=w.k, I=w.I, I_shared=w.I_shared, y_fp16=True)
    out = torch.empty(w.T, w.D, dtype=torch.bfloat16, device="cuda")
    pos = torch.from_numpy(p["pos"].astype(np.int32)).cuda()
    moe.moe_unpermute_combine(d, y.cuda(), pos, wts.cuda(), dv["x"], sh.cuda(), 0, w.T, out)
    torch.cuda.synchronize()
    ref = om.combine(np32(y), p["pos"], wts.numpy(), residual=np32(inp["x"]), shared=np32(sh))
    # one rounding of the fp32 sum to bf16 (2^-9 relative) plus fp32 summation
    assert_out_close(np32(out), ref, "combine of fp16 expert outputs", rtol=4e-3, atol=5e-5)


def test_layer_forward_fp32_and_fp16_outputs():
    """The fused layer with fp32 and with fp16 expert outputs: both within
    the output tolerance of the oracle, and close to each other."""
    w = wl.Workload("yh_layer", T=800, D=256, E=16, k=4, I=256, I_shared=128)
    inp = wl.make_inputs(w, seed=36)
    dv = to_dev(inp)
    d = moe.make_desc(T=w.T, D=w.D, E=w.E, top_k=w.k, I=w.I, I_shared=w.I_shared)
    outs = {}
    for yh in (False, True):
        lay = moe.LayerForward(d, dv["w_router"], dv["w_gate_up"], dv["w_down"],
                               shared_gate_up=dv["shared_gate_up"],
                               shared_down=dv["shared_down"], y_fp16=yh)
        lay(dv["x"])
        torch.cuda.synchronize()
        outs[yh] = np32(lay.out)
    ref = om.layer_forward(np32(inp["x"]), np32(inp["w_router"]), np32(inp["w_gate_up"]),
                           np32(inp["w_down"]), w.k, shared_gate_up=np32(inp["shared_gate_up"]),
                           shared_down=np32(inp["shared_down"]))
    for yh, o in outs.items():
        assert_out_close(o, ref["out"], f"layer output (fp16 expert outputs: {yh})")
    assert float(np.abs(outs[True] - outs[False]).max()) < 0.05
