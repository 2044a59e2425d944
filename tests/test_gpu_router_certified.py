"""The bf16 router's certified top-k against the oracle (needs MI355X).

For bf16 activations moe_route takes its logits from the bf16 matrix cores
and keeps a token's choice only when a computed error bound proves it; other
tokens get the exact logits of their candidate experts. These cases build
gate weights whose expert pairs differ in one element by a small delta, so
that many tokens have adjacent logits closer than that bound (gaps from
1e-8 to 1e-3), and pairs with identical rows (exact ties, broken towards the
lower expert id). Every token's choice must equal the oracle's bit for bit,
except tokens with an adjacent gap among their top k + 1 logits strictly
between 0 and 1e-6, where the fp64 summation order may decide the fp32
rounding. The cases cover both tile shapes of the router GEMM (E <= 32 and
larger E, with E not a multiple of the tile), hidden-dimension slices summed
across workgroups, and a masked expert (bias -inf). (At most 16 experts the
fp64 router computes every logit exactly; its tests are the parity tests.)
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_fp32_amd as moe
from oracle import moe_oracle as om
from parity import PROB_ATOL, check_logits, np32, npi

pytestmark = pytest.mark.gpu

CASES = {
    "e24_k2": (24, 2, 1024, 3000),
    "e32_k2_sliced": (32, 2, 4096, 200),
    "e32_k4": (32, 4, 2048, 2000),
    "e64_k8": (64, 8, 1024, 2000),
    "e256_k8_d7168": (256, 8, 7168, 600),
}


def _close_pairs_inputs(E, D, T, seed, mask_expert=None):
    g = np.random.default_rng(seed)
    x = torch.from_numpy(g.standard_normal((T, D)).astype(np.float32)).to(torch.bfloat16)
    w = (0.02 * g.standard_normal((E, D))).astype(np.float32)
    for j in range(E // 2):
        a, b = 2 * j, 2 * j + 1
        w[b] = w[a]
        if j % 3 != 0:  # every third pair stays an exact tie
            dcol = int(g.integers(0, D))
            delta = float(10.0 ** g.uniform(-6, -3)) * (1 if j % 2 else -1)
            w[b, dcol] = np.float32(w[a, dcol] + delta)
    bias = None
    if mask_expert is not None:
        bias = np.zeros(E, np.float32)
        bias[mask_expert] = -np.inf
    return x, torch.from_numpy(w), (None if bias is None else torch.from_numpy(bias))


def _excused(ref_logits, k):
    """Tokens with an adjacent gap in (0, 1e-6) among their top k + 1 logits."""
    s = -np.sort(-ref_logits.astype(np.float64), axis=1)[:, :k + 1]
    gaps = s[:, :-1] - s[:, 1:]
    return np.any((gaps > 0) & (gaps < om.NEAR_TIE), axis=1)


@pytest.mark.parametrize("name", sorted(CASES))
def test_certified_choice_matches_oracle(name):
    E, k, D, T = CASES[name]
    x, w, bias = _close_pairs_inputs(E, D, T, seed=7, mask_expert=E - 3)
    d = moe.make_desc(T=T, D=D, E=E, top_k=k, I=64, ep_size=1, dtype="bf16")
    dev = "cuda"
    logits = torch.empty(T, E, device=dev)
    probs = torch.empty(T, E, device=dev)
    idx = torch.empty(T, k, dtype=torch.int32, device=dev)
    wts = torch.empty(T, k, device=dev)
    ws = moe.workspace(moe.moe_route_workspace_size(d), dev)
    moe.moe_route(d, x.to(dev), w.to(dev), bias.to(dev), logits, probs, idx, wts, ws=ws)
    torch.cuda.synchronize()
    ref = om.router(np32(x), np32(w), k, np32(bias))
    got = npi(idx)
    exc = _excused(ref["logits"], k)
    diff = np.any(got != ref["topk_idx"], axis=1)
    print(f"[router] {name}: tokens={T} excused={int(exc.sum())} "
          f"differing={int(diff.sum())}", flush=True)
    bad = diff & ~exc
    assert not bad.any(), (
        f"{int(bad.sum())} tokens choose differently; first {np.nonzero(bad)[0][:4].tolist()}: "
        f"gpu {got[bad][:2].tolist()} ref {ref['topk_idx'][bad][:2].tolist()}")
    assert not np.any(got == E - 3), "the masked expert was chosen"
    check_logits(np32(logits)[:, :E - 3], ref["logits"][:, :E - 3])
    assert np.all(np32(logits)[:, E - 3] == -np.inf)
    same = ~diff
    p_err = np.abs(np32(probs) - ref["probs"]).max()
    assert p_err <= PROB_ATOL, p_err
    w_err = np.abs(np32(wts)[same] - ref["topk_w"][same]).max()
    assert w_err <= PROB_ATOL, w_err


def test_identical_rows_tie_to_lower_id():
    """All experts share one gate row: every logit of a token is the same
    value, so every token goes down the exact path and takes experts
    0 .. k-1 in order."""
    E, k, D, T = 40, 4, 512, 500
    g = np.random.default_rng(3)
    x = torch.from_numpy(g.standard_normal((T, D)).astype(np.float32)).to(torch.bfloat16)
    row = (0.02 * g.standard_normal(D)).astype(np.float32)
    w = torch.from_numpy(np.tile(row, (E, 1)))
    d = moe.make_desc(T=T, D=D, E=E, top_k=k, I=64, ep_size=1, dtype="bf16")
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    wts = torch.empty(T, k, device="cuda")
    moe.moe_route(d, x.cuda(), w.cuda(), None, None, None, idx, wts)
    torch.cuda.synchronize()
    assert npi(idx).tolist() == [list(range(k))] * T
    assert np.all(np.abs(np32(wts) - 1.0 / k) <= PROB_ATOL)


# (E, k, D, T, bias): expert counts off the 32 / 64 tiles and the select
# kernel's lane groupings (16 lanes up to 256 experts, 32 up to 512, 64
# beyond), k from 1 to 16, hidden sizes of one step up to many slices,
# token counts off the 16- and 64-token tiles.
SWEEP = [
    (17, 1, 64, 37, False), (17, 16, 128, 100, True), (31, 3, 576, 257, False),
    (48, 6, 2048, 130, True), (100, 8, 512, 1000, True), (129, 2, 1024, 77, False),
    (257, 8, 256, 300, True), (300, 16, 64, 65, False), (513, 4, 128, 50, True),
    (1000, 16, 192, 33, True),
]


@pytest.mark.parametrize("case", SWEEP, ids=[f"E{c[0]}_k{c[1]}_D{c[2]}_T{c[3]}" for c in SWEEP])
def test_certified_router_shape_sweep(case):
    """Random draws at shapes that exercise every tile tail and lane grouping
    of the certified router; a Zipf-like bias (when set) skews the logits."""
    E, k, D, T, with_bias = case
    g = np.random.default_rng(E * 7919 + D)
    x = torch.from_numpy(g.standard_normal((T, D)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy((0.02 * g.standard_normal((E, D))).astype(np.float32))
    bias = (torch.from_numpy((1.5 * np.log(1.0 / (1 + g.permutation(E)))).astype(np.float32))
            if with_bias else None)
    d = moe.make_desc(T=T, D=D, E=E, top_k=k, I=64, ep_size=1, dtype="bf16")
    dev = "cuda"
    logits = torch.empty(T, E, device=dev)
    idx = torch.empty(T, k, dtype=torch.int32, device=dev)
    wts = torch.empty(T, k, device=dev)
    moe.moe_route(d, x.to(dev), w.to(dev), None if bias is None else bias.to(dev), logits, None,
                  idx, wts)
    torch.cuda.synchronize()
    ref = om.router(np32(x), np32(w), k, None if bias is None else np32(bias))
    got = npi(idx)
    diff = np.any(got != ref["topk_idx"], axis=1)
    bad = diff & ~_excused(ref["logits"], k)
    assert not bad.any(), f"{int(bad.sum())} tokens choose differently"
    check_logits(np32(logits), ref["logits"])
    same = ~diff
    assert np.abs(np32(wts)[same] - ref["topk_w"][same]).max() <= PROB_ATOL
