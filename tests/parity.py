"""Comparison helpers shared by the GPU parity tests (test infrastructure).

Acceptance (see the design notes):
  * expert indices, counts, offsets, split sizes, perm_src and pos: bit-exact,
    except tokens whose k-th and (k+1)-th oracle fp32 logits differ by less
    than 1e-6 ("near ties"), which are counted and checked for validity;
  * router probabilities and routing weights: within 1e-5 absolute;
  * layer outputs: |gpu - ref| <= 1e-2 + 2e-2 * |ref| elementwise.
"""
from __future__ import annotations

import numpy as np

from oracle import moe_oracle as om

OUT_RTOL = 2e-2
OUT_ATOL = 1e-2
PROB_ATOL = 1e-5


def np32(t):
    return None if t is None else t.detach().float().cpu().numpy()


def npi(t):
    return t.detach().cpu().numpy().astype(np.int64)


def to_dev(inp: dict, device="cuda") -> dict:
    return {k: (None if v is None else v.to(device)) for k, v in inp.items()}


def assert_out_close(gpu: np.ndarray, ref: np.ndarray, what="output",
                     rtol=OUT_RTOL, atol=OUT_ATOL):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    err = np.abs(gpu - ref)
    bad = err > atol + rtol * np.abs(ref)
    if bad.any():
        i = np.unravel_index(np.argmax(err - (atol + rtol * np.abs(ref))), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} elements outside tolerance; worst at {i}: "
            f"gpu={gpu[i]!r} ref={ref[i]!r} (max abs err {err.max():.3e})")
    return float(err.max())


def check_routing(gpu_idx: np.ndarray, gpu_w: np.ndarray, ref: dict, norm_topk=True):
    """Compare GPU routing with the oracle's. Returns (routing to use
    downstream, report).

    Near ties (the oracle's fp32 logits): a boundary near tie is a token
    whose k-th and (k+1)-th logits differ by less than 1e-6; a slot-order
    near tie one where two adjacent chosen logits do. Such tokens may route
    differently; the GPU's choice is then checked to be a valid top-k of the
    oracle logits within the band (every chosen logit at least the k-th
    minus 1e-6, slots descending within 1e-6) and substituted, so that every
    later step is compared on the same routing. Any other difference fails.
    The report counts both kinds of near tie and the substituted tokens."""
    ref_idx = ref["topk_idx"].astype(np.int64)
    near_b = ref["boundary_gap"] < om.NEAR_TIE
    near_s = ref["slot_gap"] < om.NEAR_TIE
    near = near_b | near_s
    same = np.all(gpu_idx == ref_idx, axis=1)
    bad = ~same & ~near
    assert not bad.any(), (
        f"{int(bad.sum())} tokens route differently outside the near-tie band; first "
        f"{np.nonzero(bad)[0][:5].tolist()}: gpu {gpu_idx[bad][:2].tolist()} "
        f"ref {ref_idx[bad][:2].tolist()}")
    idx = ref_idx.copy()
    diff = np.nonzero(~same)[0]
    lg = ref["logits"].astype(np.float64)
    k = ref_idx.shape[1]
    for t in diff:
        g = gpu_idx[t]
        assert len(set(g.tolist())) == k and g.min() >= 0 and g.max() < lg.shape[1]
        kth = np.sort(lg[t])[::-1][k - 1]
        assert np.all(lg[t, g] >= kth - om.NEAR_TIE), f"token {t}: GPU choice not a near-tie top-k"
        assert np.all(lg[t, g[:-1]] >= lg[t, g[1:]] - om.NEAR_TIE), (
            f"token {t}: GPU slots not in descending logit order")
        idx[t] = g
    p_sel = ref["probs"][np.arange(len(idx))[:, None], idx]
    w = p_sel / p_sel.sum(1, keepdims=True) if norm_topk else p_sel
    werr = float(np.abs(gpu_w - w).max()) if gpu_w.size else 0.0
    assert werr <= PROB_ATOL, f"routing weights differ by {werr:.3e}"
    report = dict(tokens=int(len(idx)), boundary_near_ties=int(near_b.sum()),
                  slot_order_near_ties=int(near_s.sum()), substituted=int(len(diff)),
                  weight_err=werr)
    assert report["substituted"] <= int(near.sum())
    return (idx, w), report


def print_report(name: str, report: dict, split=None):
    """One line per workload: the near-tie counts (reported apart from the
    bit-exact comparison) and, when given, the per-logical-rank split sizes."""
    extra = f" split={list(map(int, split))}" if split is not None else ""
    print(f"[parity] {name}: " + " ".join(f"{k}={v}" for k, v in report.items()) + extra,
          flush=True)


def check_logits(gpu_logits: np.ndarray, ref_logits: np.ndarray):
    """fp32 logits: within 1e-5 + 1e-5|l|; also count exact (bitwise) agreement."""
    d = np.abs(gpu_logits.astype(np.float64) - ref_logits.astype(np.float64))
    tol = 1e-5 + 1e-5 * np.abs(ref_logits.astype(np.float64))
    assert np.all(d <= tol), f"logits differ by up to {d.max():.3e}"
    return float(np.mean(gpu_logits == ref_logits))
