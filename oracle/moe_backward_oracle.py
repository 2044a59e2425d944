"""Plain CPU oracle of the MoE layer's backward pass (gradients of the layer
forward of ``moe_oracle`` with respect to its input and its weights).

TEST INFRASTRUCTURE ONLY. Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this module. It shares no code with
the HIP path and imports nothing from it.

Sources (cited by page title and section):
  [EP]   "Expert Parallel (EP)" (twinkle-kit docs): Overview (expert
         parallelism is training middleware), Communication Pattern (the
         4-stage forward whose steps are differentiated here).
  [WE]   "Worked Example: Tracing a Token Through Expert Parallelism",
         Steps 1-5 (softmax, top-k, weighted combine, residual).
  [OVL]  torchtitan issue 5554 (shared-expert stream overlap): autograd runs
         each branch's backward on its own forward stream, and the input
         gradient adds the shared, routed and router contributions in the
         original order, (shared + routed) + router.
  [DBG]  twinkle pull request 198, commit notes: the expert-parallel
         forward returns the permuted tokens so that the backward all-to-all
         path is kept (the permuted rows are an input of the backward).

What is computed. The pages define the forward only; the backward here is the
exact derivative of that forward (a plain definition), evaluated in float64:
  out[t] = x[t] + S(x[t]) + sum_j w[t,j] * FFN_{e(t,j)}(x[t]),
  FFN_e(z) = (SiLU(z Wg_e) * (z Wu_e)) Wd_e,  S = the shared expert's FFN,
  w[t,:] = softmax over the k chosen logits (renormalised top-k weights; with
  norm_topk=False the plain softmax probabilities of the chosen experts),
  logits = x W_r^T (+ bias).
Readings (listed with the others in the design notes):
  * the top-k choice is piecewise constant: it has no derivative, and the
    chosen set is that of the forward;
  * the fp32 rounding of the router logits is not differentiated (taken as
    the identity);
  * the gradient of the logit bias is reported (dbias) but it is synthetic
    routing skew, not a weight of the layer;
  * the input gradient sums (shared + routed) + router, then the residual's
    gradient.

Parity pins (tests/test_oracle_backward.py): central finite differences of
the float64 forward on tiny inputs for every gradient; torch.autograd of the
dense per-token layer; the worked example's closed form; invariants of the
softmax gradient. None is "parity unpinned".
"""
from __future__ import annotations

from typing import Dict

import numpy as np

from . import moe_oracle as om

__all__ = ["swiglu_backward", "expert_ffn_backward", "combine_backward",
           "topk_weight_backward", "layer_backward"]

f64 = np.float64


def _as64(a) -> np.ndarray:
    return np.asarray(a, dtype=f64)


def _sigmoid(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


# ---------------------------------------------------------------------------
# One expert: [EP] Communication Pattern stage 3; [WE] Step 3.
# ---------------------------------------------------------------------------
def swiglu_backward(rows, w_gate_up, w_down, dy) -> Dict[str, np.ndarray]:
    """Gradients of y = (SiLU(rows Wg) * (rows Wu)) Wd.

    rows [m, D], w_gate_up [D, 2I] (gate = columns [0, I), up = [I, 2I)),
    w_down [I, D], dy [m, D] (gradient of y). With g = rows Wg, u = rows Wu,
    s = sigmoid(g), h = g s u:
      dh = dy Wd^T;  dWd = h^T dy
      dg = dh u s (1 + g (1 - s))   (d SiLU(g) / dg = s + g s (1 - s))
      du = dh g s
      d_rows = [dg | du] Wgu^T;  dWgu = rows^T [dg | du]
    Returns d_rows, dw_gate_up, dw_down and the intermediates g, u, h, dh, dgu.
    """
    r = _as64(rows)
    wgu = _as64(w_gate_up)
    wd = _as64(w_down)
    d = _as64(dy)
    inter = wgu.shape[1] // 2
    g = r @ wgu[:, :inter]
    u = r @ wgu[:, inter:]
    s = _sigmoid(g)
    h = g * s * u
    dh = d @ wd.T
    dg = dh * u * (s + g * s * (1.0 - s))
    du = dh * g * s
    dgu = np.concatenate([dg, du], axis=1)
    return dict(d_rows=dgu @ wgu.T, dw_gate_up=r.T @ dgu, dw_down=h.T @ d,
                g=g, u=u, h=h, dh=dh, dgu=dgu)


def expert_ffn_backward(x_perm, offsets, w_gate_up, w_down, dy_perm) -> Dict[str, np.ndarray]:
    """swiglu_backward on each expert's segment [offsets[j], offsets[j+1]).

    Returns dx_perm [M, D], dw_gate_up [n, D, 2I], dw_down [n, I, D] (zero for
    an expert without rows), h [M, I] and dgu [M, 2I].
    """
    x = _as64(x_perm)
    wgu = _as64(w_gate_up)
    wd = _as64(w_down)
    n = len(offsets) - 1
    M, D = x.shape
    inter = wgu.shape[2] // 2
    dx = np.zeros((M, D))
    dwgu = np.zeros_like(wgu)
    dwd = np.zeros_like(wd)
    h = np.zeros((M, inter))
    dgu = np.zeros((M, 2 * inter))
    for j in range(n):
        a, b = int(offsets[j]), int(offsets[j + 1])
        if b <= a:
            continue
        r = swiglu_backward(x[a:b], wgu[j], wd[j], _as64(dy_perm[a:b]))
        dx[a:b] = r["d_rows"]
        dwgu[j] = r["dw_gate_up"]
        dwd[j] = r["dw_down"]
        h[a:b] = r["h"]
        dgu[a:b] = r["dgu"]
    return dict(dx_perm=dx, dw_gate_up=dwgu, dw_down=dwd, h=h, dgu=dgu)


# ---------------------------------------------------------------------------
# Combine: [EP] Communication Pattern stage 4; [WE] Steps 4 and 5.
# ---------------------------------------------------------------------------
def combine_backward(dout, y_perm, pos, topk_w, M: int) -> Dict[str, np.ndarray]:
    """Gradients of out[t] = ... + sum_j w[t,j] y_perm[pos[t,j]].

      dtopk_w[t,j]      = dout[t] . y_perm[pos[t,j]]   (0 for pos < 0)
      dy_perm[pos[t,j]] = w[t,j] dout[t]
    """
    T, k = pos.shape
    g = _as64(dout)
    y = _as64(y_perm)
    w = _as64(topk_w)
    dtw = np.zeros((T, k))
    dy = np.zeros((M, g.shape[1]))
    for j in range(k):
        ok = pos[:, j] >= 0
        p = pos[ok, j]
        dtw[ok, j] = np.sum(g[ok] * y[p], axis=1)
        dy[p] = w[ok, j][:, None] * g[ok]
    return dict(dtopk_w=dtw, dy_perm=dy)


# ---------------------------------------------------------------------------
# Routing weights: [WE] Step 1 (softmax over the logits, top-k selection).
# ---------------------------------------------------------------------------
def topk_weight_backward(dtopk_w, topk_idx, topk_w, probs, norm_topk=True) -> np.ndarray:
    """Gradient of the logits [T, E] from the gradient of the top-k weights.

    Renormalised weights are the softmax of the chosen logits, so
      dl[t, e_j] = w_j (dw_j - sum_i w_i dw_i)
    and the other logits get 0. Plain probabilities (norm_topk=False) are the
    full softmax: dl = p (dp - sum_e p_e dp_e) with dp = dtopk_w at the chosen
    experts and 0 elsewhere.
    """
    dtw = _as64(dtopk_w)
    T, k = dtw.shape
    E = probs.shape[1]
    rows = np.arange(T)[:, None]
    dl = np.zeros((T, E))
    if norm_topk:
        w = _as64(topk_w)
        dl[rows, topk_idx] = w * (dtw - np.sum(w * dtw, axis=1, keepdims=True))
    else:
        p = _as64(probs)
        dp = np.zeros((T, E))
        dp[rows, topk_idx] = dtw
        dl = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
    return dl


# ---------------------------------------------------------------------------
# The whole layer (all experts on this GPU).
# ---------------------------------------------------------------------------
def layer_backward(x, w_router, w_gate_up, w_down, top_k, dout, logit_bias=None,
                   norm_topk=True, shared_gate_up=None, shared_down=None, routing=None,
                   residual=True, fp32_logits=True) -> Dict[str, np.ndarray]:
    """Forward (moe_oracle.layer_forward over every expert) then backward.

    Returns the forward's intermediates and
      dx [T, D], dw_router [E, D], dbias [E], dw_gate_up [E, D, 2I],
      dw_down [E, I, D], dw_shared_gate_up / dw_shared_down (or None),
      dtopk_w [T, k], dlogits [T, E], dy_perm [M, D], dx_perm [M, D],
      dx_shared / dx_routed / dx_router [T, D].
    ``routing`` may supply (topk_idx, topk_w) as for the forward.
    """
    E = w_router.shape[0]
    f = om.layer_forward(x, w_router, w_gate_up, w_down, top_k, ep_size=1,
                         logit_bias=logit_bias, norm_topk=norm_topk,
                         shared_gate_up=shared_gate_up, shared_down=shared_down,
                         routing=routing, residual=residual, fp32_logits=fp32_logits)
    x64 = _as64(x)
    g = _as64(dout)
    T, D = x64.shape
    idx, w, pos = f["topk_idx"], f["topk_w"], f["pos"]
    M = int(f["offsets"][-1])
    cb = combine_backward(g, f["y_perm"], pos, w, M)
    fb = expert_ffn_backward(f["x_perm"], f["offsets"], w_gate_up, w_down, cb["dy_perm"])
    dx_routed = np.zeros((T, D))
    for j in range(pos.shape[1]):
        ok = pos[:, j] >= 0
        dx_routed[ok] += fb["dx_perm"][pos[ok, j]]
    dl = topk_weight_backward(cb["dtopk_w"], idx, w, f["probs"], norm_topk)
    wr = _as64(w_router)
    dx_router = dl @ wr
    dx_shared = np.zeros((T, D))
    dws_gu = dws_d = None
    if shared_gate_up is not None:
        sb = swiglu_backward(x64, shared_gate_up, shared_down, g)
        dx_shared = sb["d_rows"]
        dws_gu, dws_d = sb["dw_gate_up"], sb["dw_down"]
    # [OVL]: (shared + routed) + router, then the residual's gradient
    dx = (dx_shared + dx_routed) + dx_router
    if residual:
        dx = dx + g
    res = dict(f)
    res.update(dx=dx, dw_router=dl.T @ x64, dbias=dl.sum(axis=0),
               dw_gate_up=fb["dw_gate_up"], dw_down=fb["dw_down"],
               dw_shared_gate_up=dws_gu, dw_shared_down=dws_d,
               dtopk_w=cb["dtopk_w"], dlogits=dl, dy_perm=cb["dy_perm"],
               dx_perm=fb["dx_perm"], h=fb["h"], dgu=fb["dgu"], dx_shared=dx_shared,
               dx_routed=dx_routed, dx_router=dx_router)
    assert dl.shape == (T, E)
    return res
