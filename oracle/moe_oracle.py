"""Plain CPU oracle of the MoE layer forward (one GPU's share of the work).

TEST INFRASTRUCTURE ONLY. Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this module. It shares no code with
the HIP path and imports nothing from it; it is written from the pages alone.

Sources (cited by page title and section):
  [EP]   "Expert Parallel (EP)" (twinkle-kit docs): Configuration,
         Communication Pattern (the 4-stage forward), Requirements.
  [GATE] "[Question] How does the gate coordinate across ranks in expert
         parallelism?" (Tutel issue 278): each rank gates its own local batch
         with a full [num_experts, embedding_dim] gate weight.
  [WE]   "Worked Example: Tracing a Token Through Expert Parallelism",
         Steps 1-5.
  [OVL]  torchtitan issue 5554 (shared-expert stream overlap): the shared
         expert's output joins the routed output before the combination.

Precision. Everything is float64 except where the pages fix the precision:
[EP] Configuration sets the router dtype to fp32, so the router logits are
the fp32 rounding of the (float64) dot product, and the top-k choice is made
on those fp32 values. Inputs arrive as float32 numpy arrays (bf16 inputs are
widened exactly by the caller); they are widened to float64 here.

Readings taken where the pages are silent (each also listed in the design
notes of the repository):
  * top-k weights are renormalised over the chosen experts (the worked
    example's 0.6 and 0.4 add up to 1);
  * selection is on the fp32 logits, ties go to the lower expert id, slots
    are ordered by descending logit;
  * within one expert's segment, pairs are ordered by ascending source token;
  * gate_up_proj [D, 2I]: columns [0, I) are the gate, [I, 2I) the up
    projection; h = SiLU(gate) * up with SiLU(z) = z / (1 + exp(-z));
    no biases in the expert linears;
  * the routing weights scale expert outputs at the combine; the shared
    expert's output and the residual are added unweighted;
  * an optional per-expert logit bias is added to the fp32 logits in fp32
    before the softmax and the selection;
  * router_dtype 'bf16' / 'fp16' ([EP] Configuration lists 'fp32', 'bf16'
    and 'fp16'): the gate weight holds values of that dtype, each logit is
    the exact dot product rounded once to nearest even to that dtype, a bias
    is added to the rounded value and the sum rounded again; softmax and
    top-k follow on those values.

Parity pins: every function here is pinned by the CPU tests (worked example,
invariants, brute force, library special cases); none is "parity unpinned".
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

__all__ = [
    "NEAR_TIE",
    "round_to_format",
    "router",
    "expert_rank",
    "counts_offsets_splits",
    "permute",
    "swiglu_ffn",
    "expert_ffn",
    "combine",
    "layer_forward",
    "ffn_rows",
    "brute_force_layer",
]

f64 = np.float64
f32 = np.float32

# Tokens whose k-th and (k+1)-th fp32 logits are closer than this are
# "near ties": their selection is reported, not required to match bit for bit.
NEAR_TIE = 1e-6


def _as64(a) -> np.ndarray:
    return np.asarray(a, dtype=f64)


# Floating-point formats of the router dtype: (significant bits, exponent of
# the smallest normal, largest finite value).
FORMATS = {"bf16": (8, -126, 3.3895313892515355e38), "fp16": (11, -14, 65504.0)}


def round_to_format(v, fmt: str) -> np.ndarray:
    """Round float64 values to nearest (ties to even) in format fmt.

    A value m 2^e (0.5 <= |m| < 1) keeps p significant bits: its quantum is
    2^(e - p), and 2^(emin + 1 - p) below the normal range (subnormals).
    Magnitudes past the largest finite value become infinite.
    """
    p, emin, big = FORMATS[fmt]
    v = _as64(v)
    m, e = np.frexp(v)
    q = np.maximum(e, emin + 1) - p
    r = np.ldexp(np.rint(np.ldexp(m, e - q)), q)
    r = np.where(v == 0, v, r)
    return np.where(np.abs(r) > big, np.copysign(np.inf, r), r)


# ---------------------------------------------------------------------------
# Router: [GATE] (gate weight [E, D] on every rank, each rank gates its own
# tokens), [WE] Step 1 (logits for all experts, softmax, top-k selection),
# [EP] Configuration (fp32 router).
# ---------------------------------------------------------------------------
def router(x: np.ndarray, w_router: np.ndarray, top_k: int,
           logit_bias: Optional[np.ndarray] = None,
           norm_topk: bool = True, fp32_logits: bool = True,
           router_dtype: str = "fp32") -> Dict[str, np.ndarray]:
    """Route tokens x [T, D] over E experts with gate weight w_router [E, D].

    fp32_logits=False keeps the logits in float64 (no fp32 rounding): the
    router as a smooth function of its inputs, for derivative checks.
    router_dtype 'bf16' / 'fp16': logits rounded to that format instead
    (w_router must hold values of that format).

    Returns
      logits   [T, E] float32: fp32 rounding of sum_d x[t,d] * W[e,d]
               (summed in float64), plus the bias in fp32 if given
      probs    [T, E] float64: softmax over all E experts of the fp32 logits
      topk_idx [T, k] int32: experts by descending logit, ties to lower id
      topk_w   [T, k] float64: probs of the chosen experts, divided by their
               sum when norm_topk (else the plain probs)
      boundary_gap [T] float64: logit of the k-th minus the (k+1)-th choice
               (inf when k == E)
      slot_gap [T] float64: smallest gap between adjacent chosen logits
               (inf when k == 1)
    """
    x64 = _as64(x)
    w64 = _as64(w_router)
    T = x64.shape[0]
    E = w64.shape[0]
    if not 1 <= top_k <= E:
        raise ValueError("top_k must lie in [1, E]")
    if router_dtype != "fp32":
        logits = round_to_format(x64 @ w64.T, router_dtype)
        if logit_bias is not None:
            logits = round_to_format(logits + _as64(logit_bias), router_dtype)
        logits = logits.astype(f32)  # exact: the values fit the format
    elif fp32_logits:
        logits = (x64 @ w64.T).astype(f32)  # one rounding to fp32
        if logit_bias is not None:
            logits = (logits + np.asarray(logit_bias, dtype=f32)).astype(f32)
    else:
        logits = x64 @ w64.T
        if logit_bias is not None:
            logits = logits + _as64(logit_bias)

    l64 = logits.astype(f64)
    shifted = np.exp(l64 - l64.max(axis=1, keepdims=True))
    probs = shifted / shifted.sum(axis=1, keepdims=True)

    # Descending logit, ties to the lower expert id: a stable sort of the
    # negated logits keeps equal values in ascending id order.
    order = np.argsort(-logits, axis=1, kind="stable")
    topk_idx = order[:, :top_k].astype(np.int32)
    rows = np.arange(T)[:, None]
    p_sel = probs[rows, topk_idx]
    topk_w = p_sel / p_sel.sum(axis=1, keepdims=True) if norm_topk else p_sel

    sorted_l = l64[rows, order]
    if top_k < E:
        boundary_gap = sorted_l[:, top_k - 1] - sorted_l[:, top_k]
    else:
        boundary_gap = np.full(T, np.inf)
    if top_k > 1:
        slot_gap = np.min(sorted_l[:, : top_k - 1] - sorted_l[:, 1:top_k], axis=1)
    else:
        slot_gap = np.full(T, np.inf)
    return dict(logits=logits, probs=probs, topk_idx=topk_idx, topk_w=topk_w,
                boundary_gap=boundary_gap, slot_gap=slot_gap)


def expert_rank(e, E: int, ep_size: int):
    """Owner rank and local index of expert e when E experts are split evenly
    over ep_size ranks ([EP] Overview: experts are split evenly; Requirements:
    E divisible by ep_size; [WE] Step 2: expert 11 of 16 on 4 devices is local
    index 11 mod 4 = 3 on device 2)."""
    if E % ep_size:
        raise ValueError("num_experts must be divisible by ep_size")
    e_loc = E // ep_size
    return np.asarray(e) // e_loc, np.asarray(e) % e_loc


# ---------------------------------------------------------------------------
# Preprocess: [EP] Communication Pattern, stage 1 (per-expert token counts
# and split sizes).
# ---------------------------------------------------------------------------
def counts_offsets_splits(topk_idx: np.ndarray, e_begin: int, e_end: int,
                          E: int, ep_size: int) -> Dict[str, np.ndarray]:
    """Counts of (token, expert) pairs for experts in [e_begin, e_end).

    counts[j]  = pairs whose expert is e_begin + j
    offsets    = exclusive prefix sum of counts, length n + 1 (no padding)
    split[q]   = sum of counts over the in-range experts owned by rank q
    """
    n = e_end - e_begin
    counts = np.zeros(n, dtype=np.int64)
    for e in range(e_begin, e_end):
        counts[e - e_begin] = int(np.count_nonzero(topk_idx == e))
    offsets = np.zeros(n + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    owner, _ = expert_rank(np.arange(e_begin, e_end), E, ep_size)
    split = np.zeros(ep_size, dtype=np.int64)
    for j in range(n):
        split[owner[j]] += counts[j]
    return dict(counts=counts, offsets=offsets, split=split)


# ---------------------------------------------------------------------------
# Permute: [EP] Communication Pattern, stage 2 (permute tokens by expert
# assignment); [WE] Step 2 (one dispatch entry per chosen expert).
# ---------------------------------------------------------------------------
def permute(x: np.ndarray, topk_idx: np.ndarray, e_begin: int,
            e_end: int) -> Dict[str, np.ndarray]:
    """Expert-contiguous copy of the pairs whose expert lies in [e_begin, e_end).

    Rows are ordered by expert, then by ascending source token.
      x_perm   [M, D] copy of x[perm_src[p]] (same dtype as x; None if x is None)
      perm_src [M] source token of row p
      pos      [T, k] row of pair (t, j), -1 when its expert is out of range
    """
    T, k = topk_idx.shape
    pos = np.full((T, k), -1, dtype=np.int64)
    src = []
    for e in range(e_begin, e_end):
        hit_t, hit_j = np.nonzero(topk_idx == e)  # row-major: t ascending
        base = len(src)
        pos[hit_t, hit_j] = base + np.arange(len(hit_t))
        src.extend(hit_t.tolist())
    perm_src = np.asarray(src, dtype=np.int64)
    x_perm = None if x is None else x[perm_src]
    return dict(x_perm=x_perm, perm_src=perm_src, pos=pos)


# ---------------------------------------------------------------------------
# Expert compute: [EP] Communication Pattern, stage 3 and Requirements
# (tensor-style gate_up_proj / down_proj); [WE] Step 3 (a two-layer
# feed-forward network per expert).
# ---------------------------------------------------------------------------
def swiglu_ffn(rows: np.ndarray, w_gate_up: np.ndarray,
               w_down: np.ndarray) -> np.ndarray:
    """(SiLU(rows @ Wg) * (rows @ Wu)) @ Wd in float64.

    rows [M, D]; w_gate_up [D, 2I] with gate = columns [0, I) and
    up = columns [I, 2I); w_down [I, D].
    """
    r = _as64(rows)
    wgu = _as64(w_gate_up)
    inter = wgu.shape[1] // 2
    gate = r @ wgu[:, :inter]
    up = r @ wgu[:, inter:]
    with np.errstate(over="ignore"):
        silu = gate / (1.0 + np.exp(-gate))
    return (silu * up) @ _as64(w_down)


def expert_ffn(x_perm: np.ndarray, offsets: np.ndarray, w_gate_up: np.ndarray,
               w_down: np.ndarray) -> np.ndarray:
    """Apply local expert j to rows [offsets[j], offsets[j+1]) of x_perm.

    w_gate_up [n, D, 2I] and w_down [n, I, D] are indexed by local expert.
    """
    M = x_perm.shape[0]
    D = w_down.shape[2]
    y = np.zeros((M, D), dtype=f64)
    for j in range(len(offsets) - 1):
        a, b = int(offsets[j]), int(offsets[j + 1])
        if b > a:
            y[a:b] = swiglu_ffn(x_perm[a:b], w_gate_up[j], w_down[j])
    return y


# ---------------------------------------------------------------------------
# Combine: [EP] Communication Pattern, stage 4 (unpermute, apply routing
# weights); [WE] Step 4 (weighted sum of the expert outputs) and Step 5
# (add the residual); [OVL] (shared expert output added before the combine).
# ---------------------------------------------------------------------------
def combine(y_perm: np.ndarray, pos: np.ndarray, topk_w: np.ndarray,
            residual: Optional[np.ndarray] = None,
            shared: Optional[np.ndarray] = None,
            res_begin: int = 0) -> np.ndarray:
    """out[t] = residual[t] + shared[t] + sum_j w[t,j] * y_perm[pos[t,j]].

    Slots with pos < 0 contribute nothing. residual and shared, when given,
    cover rows [res_begin, res_begin + len(residual)) of the output and are
    added unweighted. Summed in float64.
    """
    T, k = pos.shape
    D = y_perm.shape[1]
    out = np.zeros((T, D), dtype=f64)
    for j in range(k):
        ok = pos[:, j] >= 0
        if np.any(ok):
            out[ok] += _as64(topk_w)[ok, j][:, None] * _as64(y_perm)[pos[ok, j]]
    for extra in (residual, shared):
        if extra is not None:
            out[res_begin:res_begin + extra.shape[0]] += _as64(extra)
    return out


# ---------------------------------------------------------------------------
# The whole layer on one GPU's share.
# ---------------------------------------------------------------------------
def layer_forward(x, w_router, w_gate_up, w_down, top_k, ep_size=1,
                  e_begin=0, e_end=None, logit_bias=None, norm_topk=True,
                  shared_gate_up=None, shared_down=None, routing=None,
                  residual=True, fp32_logits=True) -> Dict[str, np.ndarray]:
    """Router -> counts/splits -> permute -> expert FFN -> combine.

    x [T, D]; local experts [e_begin, e_end) use w_gate_up[j] / w_down[j]
    for expert e_begin + j. ``routing`` may supply (topk_idx, topk_w) to run
    the later stages on a given routing. Returns every intermediate.
    """
    E = w_router.shape[0]
    e_end = E if e_end is None else e_end
    r = router(x, w_router, top_k, logit_bias, norm_topk, fp32_logits)
    idx, w = (r["topk_idx"], r["topk_w"]) if routing is None else routing
    c = counts_offsets_splits(idx, e_begin, e_end, E, ep_size)
    p = permute(x, idx, e_begin, e_end)
    y = expert_ffn(p["x_perm"], c["offsets"], w_gate_up, w_down)
    shared = None
    if shared_gate_up is not None:
        shared = swiglu_ffn(x, shared_gate_up, shared_down)
    out = combine(y, p["pos"], w, x if residual else None, shared)
    res = dict(r)
    res.update(c)
    res.update(p)
    res.update(topk_idx=idx, topk_w=w, y_perm=y, shared=shared, out=out)
    return res


def ffn_rows(x_rows: np.ndarray, idx_rows: np.ndarray, w_rows: np.ndarray,
             w_gate_up: np.ndarray, w_down: np.ndarray, e_begin: int = 0,
             e_end: Optional[int] = None) -> np.ndarray:
    """Weighted expert sum for a few tokens, one token at a time.

    For sampled outputs of large workloads: returns sum over the token's
    in-range slots of w * FFN_e(x), without residual or shared expert.
    """
    e_end = w_gate_up.shape[0] + e_begin if e_end is None else e_end
    out = np.zeros((x_rows.shape[0], x_rows.shape[1]), dtype=f64)
    for e in np.unique(idx_rows):
        if not e_begin <= e < e_end:
            continue
        t_hit, j_hit = np.nonzero(idx_rows == e)
        y = swiglu_ffn(x_rows[t_hit], w_gate_up[e - e_begin], w_down[e - e_begin])
        for row, (t, j) in enumerate(zip(t_hit, j_hit)):
            out[t] += float(w_rows[t, j]) * y[row]
    return out


def brute_force_layer(x, topk_idx, topk_w, w_gate_up, w_down,
                      shared_gate_up=None, shared_down=None) -> np.ndarray:
    """Direct per-token loop with no counts, permutation or positions
    ([WE] Steps 3-5 for each token on its own): out[t] = x[t] (+ shared)
    + sum_j w[t,j] * FFN_{idx[t,j]}(x[t]). Tiny inputs only."""
    T, D = x.shape
    out = np.zeros((T, D), dtype=f64)
    for t in range(T):
        xt = _as64(x[t])
        acc = xt.copy()
        if shared_gate_up is not None:
            acc += _ffn_one(xt, shared_gate_up, shared_down)
        for j in range(topk_idx.shape[1]):
            e = int(topk_idx[t, j])
            acc += float(topk_w[t, j]) * _ffn_one(xt, w_gate_up[e], w_down[e])
        out[t] = acc
    return out


def _ffn_one(xt: np.ndarray, wgu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    wgu = _as64(wgu)
    inter = wgu.shape[1] // 2
    h = np.empty(inter, dtype=f64)
    for i in range(inter):
        g = float(np.dot(xt, wgu[:, i]))
        u = float(np.dot(xt, wgu[:, inter + i]))
        with np.errstate(over="ignore"):
            h[i] = g / (1.0 + np.exp(f64(-g))) * u
    return h @ _as64(wd)
