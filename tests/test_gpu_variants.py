"""GPU parity of the interface variants (include/moe_variants.h) against the
oracle. Needs an MI355X.

moe_route_typed: the logits in bf16 / fp16 are the correctly rounded dot
products (exact products, fp64 sum, one rounding), so they are compared bit
for bit with the oracle's rounding of the float64 dot product, and the top-k
choice (ties to the lower id on both sides) bit for bit as well; routing
weights and probabilities within 1e-5."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_fp32_amd as moe
from oracle import moe_oracle as om
import workloads as wl
from parity import PROB_ATOL, np32, npi

pytestmark = pytest.mark.gpu

TDT = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


@pytest.fixture(scope="module", autouse=True)
def _gpu_and_library():
    assert torch.cuda.is_available(), "no GPU visible"
    moe.load_library()
    yield
    torch.cuda.synchronize()


CASES = {
    "ragged": wl.Workload("ragged_router", T=333, D=192, E=12, k=3, I=64),
    "zipf_bias": wl.Workload("zipf_router", T=600, D=128, E=32, k=4, I=64, zipf_s=3.0),
    "wide_E": wl.Workload("wide_router", T=700, D=256, E=128, k=8, I=64, zipf_s=1.5),
    "fp32_acts": wl.Workload("f32_router", T=77, D=64, E=5, k=2, I=64, dtype="f32"),
    "worked_example_geometry": wl.WORKLOADS["worked_example_geometry"],
}


@pytest.mark.parametrize("fmt", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_route_typed(name, fmt):
    w = CASES[name]
    inp = wl.make_inputs(w, seed=6)
    wr = inp["w_router"].to(TDT[fmt])  # the gate weight held in the router dtype
    d = moe.make_desc(T=w.T, D=w.D, E=w.E, top_k=w.k, I=w.I, dtype=w.dtype)
    dev = "cuda"
    logits = torch.empty(w.T, w.E, dtype=TDT[fmt], device=dev)
    probs = torch.empty(w.T, w.E, device=dev)
    idx = torch.empty(w.T, w.k, dtype=torch.int32, device=dev)
    tw = torch.empty(w.T, w.k, device=dev)
    bias = inp["logit_bias"]
    moe.moe_route_typed(d, fmt, inp["x"].to(dev), wr.to(dev),
                        None if bias is None else bias.to(dev), logits, probs, idx, tw)
    torch.cuda.synchronize()
    ref = om.router(np32(inp["x"]), wr.double().numpy(), w.k, np32(bias), router_dtype=fmt)
    got_l = logits.double().cpu().numpy()
    if fmt == "fp32":
        # moe_route's fp32 logits: the fp32 rounding of the fp64 sum
        assert np.all(np.abs(got_l - ref["logits"]) <= 1e-5 + 1e-5 * np.abs(ref["logits"]))
    else:
        assert np.array_equal(got_l, ref["logits"].astype(np.float64)), (
            f"{int((got_l != ref['logits']).sum())} logits differ")
    if fmt != "fp32":
        assert np.array_equal(npi(idx), ref["topk_idx"].astype(np.int64))
        assert float(np.abs(np32(tw) - ref["topk_w"]).max()) <= PROB_ATOL
    assert float(np.abs(np32(probs) - ref["probs"]).max()) <= PROB_ATOL


@pytest.mark.parametrize("counts,D,I", [([300, 0, 17, 330], 192, 320), ([512] * 16, 1024, 2048)])
def test_expert_ffn_ptrs_matches_stacked(counts, D, I):
    """One weight buffer per expert gives the stacked tensors' result bit for
    bit (the same kernels, the weight base read from the pointer array)."""
    n = len(counts)
    M = sum(counts)
    g = torch.Generator().manual_seed(len(counts))
    dev = "cuda"
    x = torch.randn(M, D, generator=g).to(torch.bfloat16).to(dev)
    wgu = (torch.randn(n, D, 2 * I, generator=g) * 0.02).to(torch.bfloat16)
    wd = (torch.randn(n, I, D, generator=g) * 0.02).to(torch.bfloat16)
    off = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32, device=dev)
    d = moe.make_desc(T=M, D=D, E=n, top_k=1, I=I)
    ws = moe.workspace(moe.moe_ffn_workspace_size(d, I, M))
    y_ref = torch.empty(M, D, device=dev)
    moe.moe_expert_ffn(d, n, I, M, x, off, wgu.to(dev), wd.to(dev), y_ref, ws)
    gu_list = [wgu[j].clone().to(dev) for j in range(n)]  # separate allocations
    dn_list = [wd[j].clone().to(dev) for j in range(n)]
    y = torch.full((M, D), 5.0, device=dev)
    moe.moe_expert_ffn_ptrs(d, n, I, M, x, off, gu_list, dn_list, y, ws)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)

