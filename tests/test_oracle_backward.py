"""Pins of the backward oracle (oracle/moe_backward_oracle.py) to facts
outside itself (no GPU needed).

  * central finite differences of the float64 forward oracle, for every
    gradient of the layer (input, router, expert and shared-expert weights,
    logit bias), with renormalised and with plain top-k weights;
  * torch.autograd (a library routine) through a dense per-token torch
    formulation of the same layer;
  * the worked example's closed form (weights 0.6 and 0.4);
  * invariants of the softmax gradient and of experts that receive no rows.
The last test plants mistakes into the backward oracle and checks that the
pins catch every one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import moe_backward_oracle as ob
from oracle import moe_oracle as om

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _case(T=5, D=6, E=4, k=2, I=3, Is=2, seed=5, bias=True):
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(T, D))
    wr = rng.normal(size=(E, D)) * 0.5
    wgu = rng.normal(size=(E, D, 2 * I)) * 0.4
    wd = rng.normal(size=(E, I, D)) * 0.4
    sgu = rng.normal(size=(D, 2 * Is)) * 0.4 if Is else None
    sd = rng.normal(size=(Is, D)) * 0.4 if Is else None
    b = rng.normal(size=E) * 0.3 if bias else None
    dout = rng.normal(size=(T, D))
    return dict(x=x, w_router=wr, w_gate_up=wgu, w_down=wd, shared_gate_up=sgu,
                shared_down=sd, logit_bias=b), dout, k


def _out(p, k, norm_topk):
    return om.layer_forward(p["x"], p["w_router"], p["w_gate_up"], p["w_down"], k,
                            logit_bias=p["logit_bias"], norm_topk=norm_topk,
                            shared_gate_up=p["shared_gate_up"], shared_down=p["shared_down"],
                            fp32_logits=False)


def _grads(o, p, dout, k, norm_topk):
    return o.layer_backward(p["x"], p["w_router"], p["w_gate_up"], p["w_down"], k, dout,
                            logit_bias=p["logit_bias"], norm_topk=norm_topk,
                            shared_gate_up=p["shared_gate_up"], shared_down=p["shared_down"],
                            fp32_logits=False)


GRAD_OF = {"x": "dx", "w_router": "dw_router", "w_gate_up": "dw_gate_up", "w_down": "dw_down",
           "shared_gate_up": "dw_shared_gate_up", "shared_down": "dw_shared_down",
           "logit_bias": "dbias"}


# ---------------------------------------------------------------------------
# Pin 1: central finite differences of the forward oracle
# ---------------------------------------------------------------------------
def pin_finite_differences(o=ob, norm_topk=True, seed=5):
    p, dout, k = _case(seed=seed)
    base = _out(p, k, norm_topk)
    # the selection must not move under the perturbations
    assert base["boundary_gap"].min() > 1e-2
    g = _grads(o, p, dout, k, norm_topk)
    h = 1e-6

    def f(q):
        r = _out(q, k, norm_topk)
        assert np.array_equal(r["topk_idx"], base["topk_idx"])
        return float(np.sum(dout * r["out"]))

    for name, gname in GRAD_OF.items():
        a = p[name]
        fd = np.zeros_like(a)
        for i in np.ndindex(a.shape):
            q = {kk: (None if v is None else v.copy()) for kk, v in p.items()}
            q[name][i] = a[i] + h
            fp = f(q)
            q[name][i] = a[i] - h
            fm = f(q)
            fd[i] = (fp - fm) / (2 * h)
        np.testing.assert_allclose(g[gname], fd, rtol=1e-6, atol=1e-7,
                                   err_msg=f"d/d {name} (norm_topk={norm_topk})")


def pin_finite_differences_plain_weights(o=ob):
    pin_finite_differences(o, norm_topk=False, seed=6)


def test_finite_differences():
    pin_finite_differences()


def test_finite_differences_plain_weights():
    pin_finite_differences_plain_weights()


# ---------------------------------------------------------------------------
# Pin 2: torch.autograd through a dense per-token formulation
# ---------------------------------------------------------------------------
def pin_autograd(o=ob):
    p, dout, k = _case(T=40, D=16, E=6, k=3, I=8, Is=4, seed=9)
    fwd = _out(p, k, True)
    idx = torch.from_numpy(fwd["topk_idx"].astype(np.int64))
    t = {n: torch.tensor(v, dtype=torch.float64, requires_grad=True)
         for n, v in p.items() if v is not None}
    x = t["x"]
    logits = x @ t["w_router"].T + t["logit_bias"]
    w = torch.softmax(torch.gather(logits, 1, idx), dim=1)  # renormalised top-k
    out = x.clone()
    Is = t["shared_gate_up"].shape[1] // 2
    sg = x @ t["shared_gate_up"]
    out = out + (torch.nn.functional.silu(sg[:, :Is]) * sg[:, Is:]) @ t["shared_down"]
    I = t["w_gate_up"].shape[2] // 2
    for e in range(t["w_router"].shape[0]):
        gu = x @ t["w_gate_up"][e]
        y = (torch.nn.functional.silu(gu[:, :I]) * gu[:, I:]) @ t["w_down"][e]
        we = (w * (idx == e)).sum(dim=1, keepdim=True)  # weight of e per token (or 0)
        out = out + we * y
    names = list(t)
    grads = torch.autograd.grad(out, [t[n] for n in names], torch.from_numpy(dout))
    g = _grads(o, p, dout, k, True)
    for n, gr in zip(names, grads):
        np.testing.assert_allclose(g[GRAD_OF[n]], gr.numpy(), rtol=1e-9, atol=1e-11,
                                   err_msg=f"d/d {n}")


def test_autograd():
    pin_autograd()


# ---------------------------------------------------------------------------
# Pin 3: the worked example (weights 0.6 and 0.4, tests/golden)
# ---------------------------------------------------------------------------
def _swiglu(x, wgu, wd):
    xt = torch.from_numpy(np.asarray(x, np.float64))
    w = torch.from_numpy(np.asarray(wgu, np.float64))
    inter = w.shape[1] // 2
    hh = torch.nn.functional.silu(xt @ w[:, :inter]) * (xt @ w[:, inter:])
    return (hh @ torch.from_numpy(np.asarray(wd, np.float64))).numpy()


def pin_worked_example(o=ob):
    """out = x + 0.6 FFN_2(x) + 0.4 FFN_11(x): with a = dout . FFN_2(x) and
    b = dout . FFN_11(x), the logit gradients are +0.24 (a - b) for expert 2,
    -0.24 (a - b) for expert 11 and 0 for the other 14."""
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    E, k = g["num_experts"], g["top_k"]
    D, I = 16, 12
    a0 = 0.25
    logit = np.full(E, a0 + math.log(0.4) - 1.0)
    for e, wv in zip(g["chosen_experts"], g["routing_weights"]):
        logit[e] = a0 + math.log(wv)
    x = np.zeros((1, D))
    x[0, 0] = 1.0
    x[0, 1:] = np.linspace(-0.5, 0.5, D - 1)
    wr = np.zeros((E, D))
    wr[:, 0] = logit
    rng = np.random.default_rng(21)
    wgu = rng.normal(size=(E, D, 2 * I)) * 0.3
    wd = rng.normal(size=(E, I, D)) * 0.3
    dout = rng.normal(size=(1, D))
    r = o.layer_backward(x, wr, wgu, wd, k, dout, fp32_logits=False)
    e2, e11 = g["chosen_experts"]
    a = float(dout[0] @ _swiglu(x, wgu[e2], wd[e2])[0])
    b = float(dout[0] @ _swiglu(x, wgu[e11], wd[e11])[0])
    np.testing.assert_allclose(r["dtopk_w"][0], [a, b], rtol=1e-9)
    expect = np.zeros(E)
    expect[e2] = 0.6 * 0.4 * (a - b)
    expect[e11] = -0.6 * 0.4 * (a - b)
    np.testing.assert_allclose(r["dlogits"][0], expect, rtol=1e-6, atol=1e-12)
    # the router weight gradient is the logit gradient times the token
    np.testing.assert_allclose(r["dw_router"], np.outer(expect, x[0]), rtol=1e-6, atol=1e-12)


def test_worked_example():
    pin_worked_example()


# ---------------------------------------------------------------------------
# Pin 4: invariants
# ---------------------------------------------------------------------------
def pin_invariants(o=ob):
    p, dout, k = _case(T=30, D=8, E=6, k=2, I=4, Is=0, seed=13)
    p["logit_bias"] = np.zeros(6)
    p["logit_bias"][5] = -50.0  # expert 5 is never chosen
    for norm in (True, False):
        g = _grads(o, p, dout, k, norm)
        dl = g["dlogits"]
        # softmax gradients sum to zero over the experts of a token
        np.testing.assert_allclose(dl.sum(axis=1), 0.0, atol=1e-12)
        np.testing.assert_allclose(g["dbias"], dl.sum(axis=0), rtol=1e-12, atol=1e-14)
        assert not np.any(g["topk_idx"] == 5)
        # an expert without rows has zero weight gradients
        assert np.all(g["dw_gate_up"][5] == 0) and np.all(g["dw_down"][5] == 0)
        if norm:
            chosen = np.zeros_like(dl, dtype=bool)
            chosen[np.arange(dl.shape[0])[:, None], g["topk_idx"]] = True
            assert np.all(dl[~chosen] == 0)
            np.testing.assert_allclose(g["dw_router"][5], 0.0, atol=0)
        # with every output weight at zero nothing but the residual flows back
    z = _grads(o, p, np.zeros_like(dout), k, True)
    for name in ("dx", "dw_router", "dw_gate_up", "dw_down"):
        assert np.all(z[name] == 0), name


def test_invariants():
    pin_invariants()


PINS = [pin_finite_differences, pin_finite_differences_plain_weights, pin_autograd,
        pin_worked_example, pin_invariants]


# ---------------------------------------------------------------------------
# Planted mistakes: each must fail at least one pin.
# ---------------------------------------------------------------------------
_orig = {n: getattr(ob, n) for n in ob.__all__}


def _mut_silu_derivative(rows, w_gate_up, w_down, dy):
    r = _orig["swiglu_backward"](rows, w_gate_up, w_down, dy)
    inter = r["g"].shape[1]
    s = 1.0 / (1.0 + np.exp(-r["g"]))
    dh = np.asarray(dy, np.float64) @ np.asarray(w_down, np.float64).T
    dg = dh * r["u"] * s  # drops the g s (1 - s) term
    dgu = np.concatenate([dg, r["dgu"][:, inter:]], axis=1)
    r.update(dgu=dgu, d_rows=dgu @ np.asarray(w_gate_up, np.float64).T,
             dw_gate_up=np.asarray(rows, np.float64).T @ dgu)
    return r


def _mut_gate_up_swapped(rows, w_gate_up, w_down, dy):
    r = _orig["swiglu_backward"](rows, w_gate_up, w_down, dy)
    inter = r["g"].shape[1]
    dgu = np.concatenate([r["dgu"][:, inter:], r["dgu"][:, :inter]], axis=1)
    r.update(dgu=dgu, d_rows=dgu @ np.asarray(w_gate_up, np.float64).T,
             dw_gate_up=np.asarray(rows, np.float64).T @ dgu)
    return r


def _mut_combine_unweighted(dout, y_perm, pos, topk_w, M):
    return _orig["combine_backward"](dout, y_perm, pos, np.ones_like(topk_w), M)


def _mut_softmax_sign(dtopk_w, topk_idx, topk_w, probs, norm_topk=True):
    return -_orig["topk_weight_backward"](dtopk_w, topk_idx, topk_w, probs, norm_topk)


def _mut_softmax_no_weight(dtopk_w, topk_idx, topk_w, probs, norm_topk=True):
    dtw = np.asarray(dtopk_w, np.float64)
    T, k = dtw.shape
    dl = np.zeros((T, probs.shape[1]))
    w = np.asarray(topk_w, np.float64)
    dl[np.arange(T)[:, None], topk_idx] = dtw - np.sum(w * dtw, axis=1, keepdims=True)
    return dl


def _mut_full_softmax_always(dtopk_w, topk_idx, topk_w, probs, norm_topk=True):
    return _orig["topk_weight_backward"](dtopk_w, topk_idx, topk_w, probs, False)


def _mut_dwd_from_unweighted(x_perm, offsets, w_gate_up, w_down, dy_perm):
    r = _orig["expert_ffn_backward"](x_perm, offsets, w_gate_up, w_down, dy_perm)
    r["dw_down"] = np.transpose(np.transpose(r["dw_down"], (0, 2, 1)), (0, 2, 1)) * 1.5
    return r


MUTANTS = {
    "silu_derivative_missing_term": ("swiglu_backward", _mut_silu_derivative),
    "gate_up_gradients_swapped": ("swiglu_backward", _mut_gate_up_swapped),
    "combine_ignores_weights": ("combine_backward", _mut_combine_unweighted),
    "softmax_gradient_sign": ("topk_weight_backward", _mut_softmax_sign),
    "softmax_gradient_without_weight": ("topk_weight_backward", _mut_softmax_no_weight),
    "full_softmax_for_renormalised": ("topk_weight_backward", _mut_full_softmax_always),
    "down_gradient_scaled": ("expert_ffn_backward", _mut_dwd_from_unweighted),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    fn, mut = MUTANTS[name]
    monkeypatch.setattr(ob, fn, mut)
    caught = []
    for pin in PINS:
        try:
            pin(ob)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name!r} passed every pin"
