"""Pins of the CPU oracle to facts outside itself (no GPU needed).

Each test checks the oracle against something the pages or the mathematics
fix: the worked example's printed values, closed forms, invariants, library
routines that compute a special case, and a brute-force per-token loop.
The last test plants mistakes into copies of the oracle and checks that the
pins catch every one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import moe_oracle as om
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _np(t):
    return t.float().numpy() if t is not None else None


def _small(T=37, D=24, E=8, k=2, I=20, seed=3, bias=None, dtype=torch.float32):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(T, D, generator=g).to(dtype).float().numpy()
    wr = (torch.randn(E, D, generator=g) * 0.3).numpy()
    wgu = (torch.randn(E, D, 2 * I, generator=g) * 0.2).to(dtype).float().numpy()
    wd = (torch.randn(E, I, D, generator=g) * 0.2).to(dtype).float().numpy()
    return x, wr, wgu, wd


def _torch_swiglu(x, wgu, wd):
    """Textbook SwiGLU FFN with torch CPU ops in float64."""
    xt = torch.from_numpy(np.asarray(x, np.float64))
    w = torch.from_numpy(np.asarray(wgu, np.float64))
    inter = w.shape[1] // 2
    h = torch.nn.functional.silu(xt @ w[:, :inter]) * (xt @ w[:, inter:])
    return (h @ torch.from_numpy(np.asarray(wd, np.float64))).numpy()


# ---------------------------------------------------------------------------
# Pin 1: the worked example (Steps 1-5), from tests/golden/worked_example.json
# ---------------------------------------------------------------------------
def _worked_example_case(o=om):
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    E, R, k = g["num_experts"], g["devices"], g["top_k"]
    D, I = 16, 12
    a = 0.25
    chosen = g["chosen_experts"]
    wts = g["routing_weights"]
    # Logits a + ln(weight) for the chosen experts, a + ln(0.4) - 1 elsewhere:
    # softmax over the two chosen logits is then exactly (0.6, 0.4), while the
    # un-renormalised softmax over all 16 would be about (0.196, 0.131).
    logit = np.full(E, a + math.log(0.4) - 1.0)
    for e, wv in zip(chosen, wts):
        logit[e] = a + math.log(wv)
    x = np.zeros((1, D), np.float32)
    x[0, 0] = 1.0
    x[0, 1:] = np.linspace(-0.5, 0.5, D - 1)  # a non-trivial FFN input
    wr = np.zeros((E, D), np.float32)
    wr[:, 0] = logit.astype(np.float32)
    gen = torch.Generator().manual_seed(11)
    wgu = (torch.randn(E, D, 2 * I, generator=gen) * 0.3).numpy()
    wd = (torch.randn(E, I, D, generator=gen) * 0.3).numpy()
    return g, x, wr, wgu, wd, E, R, k


def pin_worked_example(o=om):
    g, x, wr, wgu, wd, E, R, k = _worked_example_case(o)
    r = o.router(x, wr, k)
    assert r["topk_idx"][0].tolist() == g["chosen_experts"]
    np.testing.assert_allclose(r["topk_w"][0], g["routing_weights"], atol=1e-6)
    for e_str, dev in g["expert_owner"].items():
        owner, local = o.expert_rank(int(e_str), E, R)
        assert int(owner) == dev
        assert int(local) == g["expert_local_index"][e_str]
    dev0 = [e for e in range(E) if int(o.expert_rank(e, E, R)[0]) == 0]
    dev2 = [e for e in range(E) if int(o.expert_rank(e, E, R)[0]) == 2]
    assert dev0 == g["device_0_experts"] and dev2 == g["device_2_experts"]
    c = o.counts_offsets_splits(r["topk_idx"], 0, E, E, R)
    assert c["split"].tolist() == [1, 0, 1, 0]
    res = o.layer_forward(x, wr, wgu, wd, k, ep_size=R)
    e2, e11 = g["chosen_experts"]
    expect = (x.astype(np.float64)
              + 0.6 * _torch_swiglu(x, wgu[e2], wd[e2])
              + 0.4 * _torch_swiglu(x, wgu[e11], wd[e11]))
    np.testing.assert_allclose(res["out"], expect, rtol=1e-6, atol=1e-9)


def test_worked_example():
    pin_worked_example()


# ---------------------------------------------------------------------------
# Pin 2: router against exact sums and torch's softmax / topk
# ---------------------------------------------------------------------------
def pin_router_library(o=om):
    x, wr, _, _ = _small(T=64, D=40, E=16, k=4)
    r = o.router(x, wr, 4)
    # logits: the fp32 rounding of the exact dot product (math.fsum is exact)
    for t in (0, 7, 33, 63):
        for e in (0, 5, 15):
            exact = math.fsum(float(a) * float(b) for a, b in zip(x[t], wr[e]))
            assert r["logits"][t, e] == np.float32(exact)
    lt = torch.from_numpy(r["logits"].astype(np.float64))
    p_ref = torch.softmax(lt, dim=1).numpy()
    np.testing.assert_allclose(r["probs"], p_ref, rtol=1e-12, atol=1e-15)
    vals, idx = torch.topk(torch.from_numpy(r["logits"]), 4, dim=1)
    clear = (r["boundary_gap"] > o.NEAR_TIE) & (r["slot_gap"] > o.NEAR_TIE)
    assert clear.sum() > 50
    assert np.array_equal(r["topk_idx"][clear], idx.numpy()[clear])
    sel = torch.gather(torch.softmax(lt, 1), 1, idx.long()).numpy()
    w_ref = sel / sel.sum(1, keepdims=True)
    np.testing.assert_allclose(r["topk_w"][clear], w_ref[clear], rtol=1e-12)
    # renormalised weights sum to 1; plain weights are the probs
    np.testing.assert_allclose(r["topk_w"].sum(1), 1.0, rtol=1e-12)
    r2 = o.router(x, wr, 4, norm_topk=False)
    np.testing.assert_allclose(r2["topk_w"][clear], sel[clear], rtol=1e-12)


def test_router_library():
    pin_router_library()


def pin_router_ties(o=om):
    x = np.ones((1, 4), np.float32)
    wr = np.zeros((6, 4), np.float32)
    wr[[1, 3, 4], :] = 0.5  # three equal logits of 2.0
    r = o.router(x, wr, 2)
    assert r["topk_idx"][0].tolist() == [1, 3]
    assert r["boundary_gap"][0] == 0.0 and r["slot_gap"][0] == 0.0


def test_router_ties_go_to_lower_id():
    pin_router_ties()


def test_router_bias_is_added_in_fp32():
    x, wr, _, _ = _small(T=16, D=8, E=8, k=2)
    bias = np.linspace(-1, 1, 8).astype(np.float32)
    r0 = om.router(x, wr, 2)
    r1 = om.router(x, wr, 2, logit_bias=bias)
    assert np.array_equal(r1["logits"], (r0["logits"] + bias).astype(np.float32))


# ---------------------------------------------------------------------------
# Pin 3: counts / offsets / splits invariants and a closed form
# ---------------------------------------------------------------------------
def pin_counts(o=om):
    x, wr, _, _ = _small(T=200, D=16, E=16, k=3)
    r = o.router(x, wr, 3)
    c = o.counts_offsets_splits(r["topk_idx"], 0, 16, 16, 4)
    assert c["counts"].sum() == 200 * 3
    assert c["offsets"][0] == 0 and c["offsets"][-1] == 600
    assert np.all(np.diff(c["offsets"]) == c["counts"])
    assert c["split"].sum() == 600
    assert c["split"].tolist() == [int(c["counts"][4 * q:4 * q + 4].sum()) for q in range(4)]
    # each token's k experts are distinct
    assert all(len(set(row)) == 3 for row in r["topk_idx"].tolist())
    # closed form: a bias far above the logit spread makes the top-k ranked
    # experts win every token
    bias = np.zeros(16, np.float32)
    bias[[5, 9, 12]] = [300.0, 200.0, 100.0]
    rb = o.router(x, wr, 3, logit_bias=bias)
    assert np.all(rb["topk_idx"] == np.array([5, 9, 12]))
    cb = o.counts_offsets_splits(rb["topk_idx"], 0, 16, 16, 4)
    expect = np.zeros(16, np.int64)
    expect[[5, 9, 12]] = 200
    assert np.array_equal(cb["counts"], expect)
    # an expert range: only the in-range experts are counted
    cr = o.counts_offsets_splits(r["topk_idx"], 4, 8, 16, 4)
    assert np.array_equal(cr["counts"], c["counts"][4:8])
    assert cr["split"].tolist() == [0, int(c["counts"][4:8].sum()), 0, 0]


def test_counts():
    pin_counts()


# ---------------------------------------------------------------------------
# Pin 4: permute properties, and a library sort gives the same permutation
# ---------------------------------------------------------------------------
def pin_permute(o=om):
    x, wr, _, _ = _small(T=150, D=12, E=8, k=3)
    r = o.router(x, wr, 3)
    idx = r["topk_idx"]
    for (eb, ee) in [(0, 8), (2, 6)]:
        p = o.permute(x, idx, eb, ee)
        c = o.counts_offsets_splits(idx, eb, ee, 8, 1)
        M = int(c["offsets"][-1])
        assert p["x_perm"].shape == (M, 12) and p["perm_src"].shape == (M,)
        for t in range(150):
            for j in range(3):
                q = p["pos"][t, j]
                if eb <= idx[t, j] < ee:
                    assert q >= 0 and p["perm_src"][q] == t
                    assert np.array_equal(p["x_perm"][q], x[t])
                    assert c["offsets"][idx[t, j] - eb] <= q < c["offsets"][idx[t, j] - eb + 1]
                else:
                    assert q == -1
        # every row is used once
        used = np.sort(p["pos"][p["pos"] >= 0])
        assert np.array_equal(used, np.arange(M))
        # library cross-check: a stable sort of the in-range pairs by expert
        flat = idx.reshape(-1)
        keep = np.nonzero((flat >= eb) & (flat < ee))[0]
        order = keep[np.argsort(flat[keep], kind="stable")]
        assert np.array_equal(p["perm_src"], order // 3)


def test_permute():
    pin_permute()


def pin_combine_identity(o=om):
    """permute then unpermute with weights summing to 1 gives back x."""
    x, wr, _, _ = _small(T=90, D=10, E=8, k=4)
    r = o.router(x, wr, 4)
    p = o.permute(x, r["topk_idx"], 0, 8)
    out = o.combine(p["x_perm"], p["pos"], r["topk_w"])
    np.testing.assert_allclose(out, x, rtol=1e-12, atol=1e-12)
    out2 = o.combine(p["x_perm"], p["pos"], r["topk_w"], residual=x)
    np.testing.assert_allclose(out2, 2 * x.astype(np.float64), rtol=1e-12, atol=1e-12)


def test_combine_identity():
    pin_combine_identity()


# ---------------------------------------------------------------------------
# Pin 5: the FFN reduces to a textbook SwiGLU layer when E = 1, k = 1
# ---------------------------------------------------------------------------
def pin_single_expert(o=om):
    x, wr, wgu, wd = _small(T=33, D=16, E=1, k=1, I=24)
    res = o.layer_forward(x, wr, wgu, wd, 1)
    assert np.all(res["topk_idx"] == 0) and np.allclose(res["topk_w"], 1.0)
    expect = x.astype(np.float64) + _torch_swiglu(x, wgu[0], wd[0])
    np.testing.assert_allclose(res["out"], expect, rtol=1e-12, atol=1e-12)
    # shared expert: added unweighted
    sgu = wgu[0] * 0.5
    sd = wd[0] * 2.0
    res2 = o.layer_forward(x, wr, wgu, wd, 1, shared_gate_up=sgu, shared_down=sd)
    np.testing.assert_allclose(res2["out"], expect + _torch_swiglu(x, sgu, sd),
                               rtol=1e-12, atol=1e-12)


def test_single_expert():
    pin_single_expert()


# ---------------------------------------------------------------------------
# Pin 6: brute force per token equals the permuted path
# ---------------------------------------------------------------------------
def pin_brute_force(o=om, T=40, D=16, E=8, k=3, I=12, ep=2, shared=True):
    x, wr, wgu, wd = _small(T=T, D=D, E=E, k=k, I=I, seed=5)
    sgu = sd = None
    if shared:
        sgu, sd = wgu[1] * 0.7, wd[2] * 1.3
    res = o.layer_forward(x, wr, wgu, wd, k, ep_size=ep,
                          shared_gate_up=sgu, shared_down=sd)
    bf = o.brute_force_layer(x, res["topk_idx"], res["topk_w"], wgu, wd, sgu, sd)
    np.testing.assert_allclose(res["out"], bf, rtol=1e-12, atol=1e-12)


def test_brute_force_small():
    pin_brute_force()
    pin_brute_force(T=17, D=8, E=4, k=4, I=8, ep=4, shared=False)  # k == E
    pin_brute_force(T=9, D=8, E=16, k=1, I=8, ep=1, shared=False)


def test_brute_force_tiny_fp32_workload():
    w = wl.WORKLOADS["tiny_fp32"]
    inp = wl.make_inputs(w)
    x = _np(inp["x"])
    res = om.layer_forward(x, _np(inp["w_router"]), _np(inp["w_gate_up"]),
                           _np(inp["w_down"]), w.k)
    sub = slice(0, 64)  # brute force on a quarter of the tokens keeps it quick
    bf = om.brute_force_layer(x[sub], res["topk_idx"][sub], res["topk_w"][sub],
                              _np(inp["w_gate_up"]), _np(inp["w_down"]))
    np.testing.assert_allclose(res["out"][sub], bf, rtol=1e-12, atol=1e-12)
    assert res["counts"].sum() == w.T * w.k


def test_expert_range_partials_add_up():
    """Summing the receiver-side partials of every rank gives the full layer."""
    x, wr, wgu, wd = _small(T=30, D=12, E=8, k=3, I=10, seed=9)
    full = om.layer_forward(x, wr, wgu, wd, 3, residual=False)
    total = np.zeros_like(full["out"])
    for q in range(4):
        part = om.layer_forward(x, wr, wgu[2 * q:2 * q + 2], wd[2 * q:2 * q + 2], 3,
                                ep_size=4, e_begin=2 * q, e_end=2 * q + 2,
                                residual=False)
        total += part["out"]
    np.testing.assert_allclose(total, full["out"], rtol=1e-12, atol=1e-12)


def test_ffn_rows_matches_layer():
    x, wr, wgu, wd = _small(T=25, D=12, E=8, k=2, I=10, seed=4)
    res = om.layer_forward(x, wr, wgu, wd, 2, residual=False)
    rows = om.ffn_rows(x[3:9], res["topk_idx"][3:9], res["topk_w"][3:9], wgu, wd)
    np.testing.assert_allclose(rows, res["out"][3:9], rtol=1e-12, atol=1e-12)


def test_workloads_are_seeded():
    w = wl.scaled(wl.WORKLOADS["skewed_fine_grained"], T=64, D=64, I=64)
    a = wl.make_inputs(w, seed=0)
    b = wl.make_inputs(w, seed=0)
    c = wl.make_inputs(w, seed=1)
    for key in a:
        if a[key] is not None:
            assert torch.equal(a[key], b[key])
    assert not torch.equal(a["x"], c["x"])
    assert a["x"].dtype == torch.bfloat16 and a["w_router"].dtype == torch.float32
    assert a["w_gate_up"].shape == (128, 64, 128) and a["w_down"].shape == (128, 64, 64)
    bias = a["logit_bias"].double()
    assert torch.allclose(torch.sort(bias, descending=True).values,
                          -1.5 * torch.log(torch.arange(1, 129, dtype=torch.float64)),
                          atol=1e-6)


# ---------------------------------------------------------------------------
# Planted mistakes: every one of them must make at least one pin fail.
# ---------------------------------------------------------------------------
PINS = [pin_worked_example, pin_router_library, pin_router_ties, pin_counts, pin_permute,
        pin_combine_identity, pin_single_expert, pin_brute_force]


class _Mutant:
    """A copy of the oracle module with one function replaced."""

    def __init__(self, **repl):
        for name in om.__all__:
            setattr(self, name, getattr(om, name))
        self.brute_force_layer = om.brute_force_layer
        for k, v in repl.items():
            setattr(self, k, v)
        # layer_forward must route through the mutated pieces
        self.layer_forward = lambda *a, **kw: _layer_forward_via(self, *a, **kw)


def _layer_forward_via(o, x, w_router, w_gate_up, w_down, top_k, ep_size=1,
                       e_begin=0, e_end=None, logit_bias=None, norm_topk=True,
                       shared_gate_up=None, shared_down=None, routing=None,
                       residual=True):
    E = w_router.shape[0]
    e_end = E if e_end is None else e_end
    r = o.router(x, w_router, top_k, logit_bias, norm_topk)
    idx, w = r["topk_idx"], r["topk_w"]
    c = o.counts_offsets_splits(idx, e_begin, e_end, E, ep_size)
    p = o.permute(x, idx, e_begin, e_end)
    y = o.expert_ffn(p["x_perm"], c["offsets"], w_gate_up, w_down)
    shared = None if shared_gate_up is None else o.swiglu_ffn(x, shared_gate_up, shared_down)
    out = o.combine(y, p["pos"], w, x if residual else None, shared)
    res = dict(r)
    res.update(c)
    res.update(p)
    res.update(out=out, y_perm=y)
    return res


def _mut_router_no_renorm(x, w_router, top_k, logit_bias=None, norm_topk=True):
    return om.router(x, w_router, top_k, logit_bias, norm_topk=False)


def _mut_router_high_id_ties(x, w_router, top_k, logit_bias=None, norm_topk=True):
    r = om.router(x, w_router, top_k, logit_bias, norm_topk)
    lg = r["logits"]
    E = lg.shape[1]
    order = np.argsort(-lg[:, ::-1], axis=1, kind="stable")
    idx = (E - 1 - order[:, :top_k]).astype(np.int32)
    r = dict(r)
    p = r["probs"][np.arange(len(lg))[:, None], idx]
    r["topk_idx"], r["topk_w"] = idx, (p / p.sum(1, keepdims=True) if norm_topk else p)
    return r


def _mut_router_transposed(x, w_router, top_k, logit_bias=None, norm_topk=True):
    # a transposed gate weight (only shape-compatible when D == E, else wrong shape)
    wt = np.asarray(w_router)
    if wt.shape[0] == wt.shape[1]:
        wt = wt.T
    else:
        wt = wt[::-1]
    return om.router(x, np.ascontiguousarray(wt), top_k, logit_bias, norm_topk)


def _mut_swiglu_swapped(rows, w_gate_up, w_down):
    inter = w_gate_up.shape[1] // 2
    sw = np.concatenate([w_gate_up[:, inter:], w_gate_up[:, :inter]], axis=1)
    return om.swiglu_ffn(rows, sw, w_down)


def _mut_swiglu_sign(rows, w_gate_up, w_down):
    r = np.asarray(rows, np.float64)
    wgu = np.asarray(w_gate_up, np.float64)
    inter = wgu.shape[1] // 2
    g = r @ wgu[:, :inter]
    u = r @ wgu[:, inter:]
    return (g / (1.0 + np.exp(g)) * u) @ np.asarray(w_down, np.float64)


def _mut_ffn(swiglu):
    def f(x_perm, offsets, w_gate_up, w_down):
        y = np.zeros((x_perm.shape[0], w_down.shape[2]))
        for j in range(len(offsets) - 1):
            a, b = int(offsets[j]), int(offsets[j + 1])
            if b > a:
                y[a:b] = swiglu(x_perm[a:b], w_gate_up[j], w_down[j])
        return y
    return f


def _mut_ffn_off_by_one(x_perm, offsets, w_gate_up, w_down):
    y = np.zeros((x_perm.shape[0], w_down.shape[2]))
    n = len(offsets) - 1
    for j in range(n):
        a, b = int(offsets[j]), int(offsets[j + 1])
        if b > a:
            y[a:b] = om.swiglu_ffn(x_perm[a:b], w_gate_up[(j + 1) % n], w_down[(j + 1) % n])
    return y


def _mut_combine_no_weights(y_perm, pos, topk_w, residual=None, shared=None, res_begin=0):
    return om.combine(y_perm, pos, np.ones_like(np.asarray(topk_w, np.float64)) / pos.shape[1],
                      residual, shared, res_begin)


def _mut_combine_no_residual(y_perm, pos, topk_w, residual=None, shared=None, res_begin=0):
    return om.combine(y_perm, pos, topk_w, None, shared, res_begin)


def _mut_combine_shared_weighted(y_perm, pos, topk_w, residual=None, shared=None, res_begin=0):
    s = None if shared is None else 0.5 * np.asarray(shared)
    return om.combine(y_perm, pos, topk_w, residual, s, res_begin)


def _mut_permute_descending(x, topk_idx, e_begin, e_end):
    T, k = topk_idx.shape
    pos = np.full((T, k), -1, dtype=np.int64)
    src = []
    for e in range(e_begin, e_end):
        hit_t, hit_j = np.nonzero(topk_idx == e)
        hit_t, hit_j = hit_t[::-1], hit_j[::-1]
        base = len(src)
        pos[hit_t, hit_j] = base + np.arange(len(hit_t))
        src.extend(hit_t.tolist())
    perm_src = np.asarray(src, dtype=np.int64)
    return dict(x_perm=x[perm_src], perm_src=perm_src, pos=pos)


def _mut_split_local_index(topk_idx, e_begin, e_end, E, ep_size):
    c = om.counts_offsets_splits(topk_idx, e_begin, e_end, E, ep_size)
    split = np.zeros(ep_size, np.int64)
    for j in range(e_end - e_begin):
        split[(e_begin + j) % ep_size] += c["counts"][j]
    c["split"] = split
    return c


def _mut_rank_mod(e, E, ep_size):
    e_loc = E // ep_size
    return np.asarray(e) % ep_size, np.asarray(e) // ep_size


MUTANTS = {
    "no_renorm": dict(router=_mut_router_no_renorm),
    "ties_to_higher_id": dict(router=_mut_router_high_id_ties),
    "transposed_gate": dict(router=_mut_router_transposed),
    "gate_up_swapped": dict(swiglu_ffn=_mut_swiglu_swapped,
                            expert_ffn=_mut_ffn(_mut_swiglu_swapped)),
    "silu_sign": dict(swiglu_ffn=_mut_swiglu_sign, expert_ffn=_mut_ffn(_mut_swiglu_sign)),
    "wrong_expert_weights": dict(expert_ffn=_mut_ffn_off_by_one),
    "combine_ignores_weights": dict(combine=_mut_combine_no_weights),
    "combine_drops_residual": dict(combine=_mut_combine_no_residual),
    "shared_weighted": dict(combine=_mut_combine_shared_weighted),
    "permute_descending_tokens": dict(permute=_mut_permute_descending),
    "split_by_modulo": dict(counts_offsets_splits=_mut_split_local_index),
    "rank_by_modulo": dict(expert_rank=_mut_rank_mod),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    o = _Mutant(**MUTANTS[name])
    caught = []
    for pin in PINS:
        try:
            pin(o)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name!r} passed every pin"


# ---------------------------------------------------------------------------
# Router dtype: the rounding to bf16 / fp16 against library conversions
# ---------------------------------------------------------------------------
def test_round_to_format_matches_library_conversions():
    rng = np.random.default_rng(4)
    v = np.concatenate([rng.normal(size=20000) * 10.0 ** rng.integers(-9, 5, size=20000),
                        [0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, 2.0 ** -24, 2.0 ** -25,
                         3 * 2.0 ** -26, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11]])
    # fp16: numpy's float64 -> float16 conversion rounds to nearest even directly
    h = om.round_to_format(v, "fp16")
    ref = v.astype(np.float16).astype(np.float64)
    assert np.array_equal(h, ref, equal_nan=True)
    # bf16: torch's fp32 -> bf16 conversion rounds to nearest even; on values
    # exact in fp32 it is the rounding of the value itself
    v32 = v.astype(np.float32).astype(np.float64)
    b = om.round_to_format(v32, "bf16")
    ref = torch.from_numpy(v32.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.array_equal(b, ref)
    # ties to even at one
    assert om.round_to_format(1.0 + 2.0 ** -8, "bf16") == 1.0
    assert om.round_to_format(1.0 + 3 * 2.0 ** -8, "bf16") == 1.0 + 2.0 ** -6


def test_router_dtype_rounds_the_logits():
    x, wr, _, _ = _small(T=50, D=24, E=8, seed=9, dtype=torch.bfloat16)
    for fmt in ("bf16", "fp16"):
        w16 = om.round_to_format(wr, fmt)
        bias = np.linspace(-0.3, 0.2, 8)
        r = om.router(x, w16, 2, bias, router_dtype=fmt)
        exact = x.astype(np.float64) @ w16.T
        expect = om.round_to_format(om.round_to_format(exact, fmt) + bias, fmt)
        assert np.array_equal(r["logits"].astype(np.float64), expect)
        # the choice is the stable descending order of those logits
        order = np.argsort(-expect, axis=1, kind="stable")[:, :2]
        assert np.array_equal(r["topk_idx"], order)
