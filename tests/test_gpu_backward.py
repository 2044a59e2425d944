"""GPU parity of the backward pass (include/moe_backward.h) against the
backward oracle (oracle/moe_backward_oracle.py). Needs an MI355X.

Tolerances, from the arithmetic of the HIP path (bf16 operands and fp32
accumulation on the matrix cores; G | U recomputed in fp32; dy_perm, dG | dU
and H rounded to bf16, whose unit roundoff is u = 2^-8 (8 significant bits);
the fp64 oracle rounds nothing):
  * an fp32 sum of n products: |gpu - ref| <= n 2^-24 sum |products|;
  * one bf16 rounding of a value computed in fp32: |gpu - ref| <= 2u |ref|
    (a factor 2 over the rounding) plus the fp32 terms (the sigmoid from the
    hardware exp and reciprocal, relative error ~1e-6);
  * a contraction of bf16-rounded operands: elementwise bounds propagated
    through |A| @ |B| from the operands' own bounds, with a factor 1.5
    (expert FFN tests; the worst measured error is below half the bound);
  * the whole layer, where the forward's own rounding (H in fp16, y_perm)
    enters through the routing-weight gradient: |gpu - ref| <= 2e-2 |ref| +
    1e-2 rms(ref) elementwise and a relative Frobenius error below 1e-2.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_fp32_amd as moe
from oracle import moe_backward_oracle as ob
from oracle import moe_oracle as om
import workloads as wl
from parity import check_routing, np32, npi, to_dev

pytestmark = pytest.mark.gpu

bf16 = torch.bfloat16
GRAD_RTOL = 2e-2
GRAD_ATOL_RMS = 1e-2
GRAD_FROB = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu_and_library():
    assert torch.cuda.is_available(), "no GPU visible"
    moe.load_library()
    yield
    torch.cuda.synchronize()


def _align(n):
    return (n + 255) // 256 * 256


def assert_grad_close(gpu, ref, what, rms_of=None, rtol=GRAD_RTOL, atol_rms=GRAD_ATOL_RMS,
                      frob=GRAD_FROB):
    """|gpu - ref| <= rtol |ref| + atol_rms rms(rms_of or ref), and the
    relative Frobenius error of (gpu - ref) below frob. Returns that error."""
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    base = r if rms_of is None else np.asarray(rms_of, np.float64)
    rms = float(np.sqrt(np.mean(base ** 2))) if base.size else 0.0
    err = np.abs(g - r)
    tol = rtol * np.abs(r) + atol_rms * rms
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; worst "
                             f"at {i}: gpu={g[i]!r} ref={r[i]!r} (rms {rms:.3e})")
    den = float(np.linalg.norm(base))
    rel = float(np.linalg.norm(g - r)) / den if den > 0 else float(np.linalg.norm(g - r))
    assert rel < frob, f"{what}: relative Frobenius error {rel:.3e}"
    print(f"[grad] {what}: rel Frobenius error {rel:.2e}", flush=True)
    return rel


def _bf(t):
    return t.to(bf16)


# ---------------------------------------------------------------------------
# Expert FFN backward on ragged segments
# ---------------------------------------------------------------------------
def _ffn_case(counts, D, I, seed, wscale=0.05, dtype=bf16):
    g = torch.Generator().manual_seed(seed)
    n = len(counts)
    M = int(sum(counts))
    x = torch.randn(M, D, generator=g).to(dtype)
    wgu = (torch.randn(n, D, 2 * I, generator=g) * wscale).to(dtype)
    wd = (torch.randn(n, I, D, generator=g) * wscale).to(dtype)
    dy = torch.randn(M, D, generator=g).to(dtype)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return x, wgu, wd, dy, offsets


def _run_ffn_bwd(x, wgu, wd, dy, offsets, D, I, extra_rows=0, gu_saved=None):
    n = wgu.shape[0]
    M = x.shape[0]
    cap = M + extra_rows
    dt = x.dtype
    d = moe.make_desc(T=max(M, 1), D=D, E=n, top_k=1, I=I,
                      dtype="bf16" if dt == bf16 else "f32")
    dev = "cuda"
    xd = torch.zeros(cap, D, dtype=dt, device=dev)
    xd[:M] = x.to(dev)
    dyd = torch.zeros(cap, D, dtype=dt, device=dev)
    dyd[:M] = dy.to(dev)
    off = torch.tensor(offsets, dtype=torch.int32, device=dev) if offsets is not None else None
    dx = torch.full((cap, D), -3.0, device=dev)
    dwgu = torch.full((n, D, 2 * I), -5.0, device=dev)
    dwd = torch.full((n, I, D), -5.0, device=dev)
    ws = moe.workspace(moe.moe_ffn_backward_workspace_size(d, I, cap))
    moe.moe_expert_ffn_backward(d, n, I, cap, xd, off, wgu.to(dev), wd.to(dev), dyd, dx, dwgu, dwd,
                                ws, gu_saved=gu_saved)
    torch.cuda.synchronize()
    es = dt.itemsize
    r4, r2 = cap * I * 4, cap * 2 * I * es
    dh = ws[:r4].view(torch.float32).view(cap, I)
    dgu = ws[_align(r4):_align(r4) + r2].view(dt).view(cap, 2 * I)
    o = _align(r4) + _align(r2)
    h = ws[o:o + cap * I * es].view(dt).view(cap, I)
    return dict(dx=dx.cpu().numpy(), dwgu=dwgu.cpu().numpy(), dwd=dwd.cpu().numpy(),
                dh=dh.cpu().numpy() if gu_saved is None else None,  # dH unused when saved
                dgu=dgu.float().cpu().numpy(), h=h.float().cpu().numpy())


def _expert_bounds(rows, wgu, wd, dy, dy_rounded, ub=2.0 ** -8):
    """The oracle's gradients of one expert on `rows` and elementwise bounds of
    the HIP path's errors, propagated from its roundings:
      G, U, dH: fp32 sums (D 2^-24 of the sum of |products|), plus u = 2^-8
        of |dy| @ |Wd|^T in dH when the GPU's dy is a bf16 rounding (the
        layer's dy_perm = bf16(w dout));
      H, dG, dU: those errors through |SiLU'| <= 1.1 and |SiLU''| <= 0.5,
        the hardware sigmoid (~2e-6 relative), and their own bf16 rounding;
      dX, dWgu, dWd: contractions of those operands (bf16 x and weights are
        exact) plus the fp32 sums' bound."""
    x = np.asarray(rows, np.float64)
    w1 = np.asarray(wgu, np.float64)
    w2 = np.asarray(wd, np.float64)
    d = np.asarray(dy, np.float64)
    D = x.shape[1]
    I = w1.shape[1] // 2
    n = x.shape[0]
    r = ob.swiglu_backward(x, w1, w2, d)
    g, u, dh, h = r["g"], r["u"], r["dh"], r["h"]
    dg, du = r["dgu"][:, :I], r["dgu"][:, I:]
    ax, a1, a2, ad = np.abs(x), np.abs(w1), np.abs(w2), np.abs(d)
    mag_gu = ax @ a1
    mg, mu = D * 2.0 ** -24 * mag_gu[:, :I], D * 2.0 ** -24 * mag_gu[:, I:]
    mag_dh = ad @ a2.T
    # ub: unit roundoff of the stored intermediates (bf16 2^-8; fp32 layers 2^-24)
    e_dh = (D * 2.0 ** -24 + (ub if dy_rounded else 0.0)) * mag_dh
    eps = 2e-6
    e_h = 2 * ub * np.abs(h) + 1.1 * mg * np.abs(u) + mu * np.abs(g) + eps * np.abs(g * u)
    e_dg = (2 * ub * np.abs(dg) + 1.1 * e_dh * np.abs(u) + 0.5 * mg * np.abs(dh * u)
            + 1.1 * mu * np.abs(dh) + eps * np.abs(dh * u) * (1 + np.abs(g)))
    e_du = (2 * ub * np.abs(du) + 1.1 * e_dh * np.abs(g) + 1.1 * mg * np.abs(dh)
            + eps * np.abs(dh * g))
    e_dgu = np.concatenate([e_dg, e_du], axis=1)
    a_dgu = np.abs(r["dgu"])
    f = 1.5  # margin over the first-order propagation
    b_dx = f * (e_dgu @ a1.T + 2 * I * 2.0 ** -24 * (a_dgu @ a1.T))
    b_wgu = f * (ax.T @ e_dgu + n * 2.0 ** -24 * (ax.T @ a_dgu))
    b_wd = f * (e_h.T @ ad + (ub if dy_rounded else 0.0) * (np.abs(h).T @ ad)
                + n * 2.0 ** -24 * (np.abs(h).T @ ad))
    return dict(r=r, b_dh=e_dh, e_h=e_h, e_dgu=e_dgu, b_dx=b_dx, b_wgu=b_wgu, b_wd=b_wd)


def _within(got, want, bound, what):
    err = np.abs(np.asarray(got, np.float64) - want)
    bad = err > bound + 1e-30
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside the bound; worst "
                           f"excess {float((err - bound).max()):.3e}")
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(want), 1e-300))
    print(f"[grad] {what}: max err / bound {float((err / (bound + 1e-30)).max()):.3f}, "
          f"rel Frobenius {rel:.2e}", flush=True)


def _check_ffn_bwd(x, wgu, wd, dy, offsets, D, I, out, tag):
    n = wgu.shape[0]
    M = x.shape[0]
    ub = 2.0 ** -8 if x.dtype == bf16 else 2.0 ** -24
    for j in range(n):
        a, b = int(offsets[j]), int(offsets[j + 1])
        if b == a:
            assert np.all(out["dwgu"][j] == 0) and np.all(out["dwd"][j] == 0), f"expert {j}"
            continue
        eb = _expert_bounds(np32(x[a:b]), np32(wgu[j]), np32(wd[j]), np32(dy[a:b]), False, ub)
        r = eb["r"]
        t = f"{tag} expert {j}"
        _within(out["dh"][a:b], r["dh"], eb["b_dh"], f"{t} dH")
        _within(out["h"][a:b], r["h"], eb["e_h"], f"{t} H")
        _within(out["dgu"][a:b], r["dgu"], eb["e_dgu"], f"{t} dG|dU")
        _within(out["dx"][a:b], r["d_rows"], eb["b_dx"], f"{t} dx_perm")
        _within(out["dwgu"][j], r["dw_gate_up"], eb["b_wgu"], f"{t} dW_gate_up")
        _within(out["dwd"][j], r["dw_down"], eb["b_wd"], f"{t} dW_down")
    assert np.all(out["dx"][M:] == -3.0), "rows past the segments were written"


@pytest.mark.parametrize("counts,D,I", [
    ([300, 0, 17, 330], 320, 192),        # ragged tiles in every dimension, an empty expert
    ([1, 64, 0, 0, 511, 2], 256, 256),
    ([5, 70, 0, 33], 64, 64),             # weight-gradient tiles mostly past P and Q
])
def test_expert_ffn_backward_ragged(counts, D, I):
    x, wgu, wd, dy, offsets = _ffn_case(counts, D, I, seed=sum(counts))
    out = _run_ffn_bwd(x, wgu, wd, dy, offsets, D, I, extra_rows=7)
    _check_ffn_bwd(x, wgu, wd, dy, offsets, D, I, out, f"ffn {counts}")


def test_split_backward_entry_points_match():
    """moe_expert_gate_up_backward (fed the dH that the one-call backward
    leaves in its workspace) and moe_expert_weight_grad reproduce
    moe_expert_ffn_backward bit for bit (the same kernels)."""
    counts, D, I = [130, 0, 257, 64], 256, 192
    x, wgu, wd, dy, offsets = _ffn_case(counts, D, I, seed=77)
    M = x.shape[0]
    full = _run_ffn_bwd(x, wgu, wd, dy, offsets, D, I)
    n = len(counts)
    d = moe.make_desc(T=M, D=D, E=n, top_k=1, I=I)
    dev = "cuda"
    off = torch.tensor(offsets, dtype=torch.int32, device=dev)
    dh = torch.from_numpy(full["dh"]).to(dev)
    dgu = torch.empty(M, 2 * I, dtype=bf16, device=dev)
    h = torch.empty(M, I, dtype=bf16, device=dev)
    moe.moe_expert_gate_up_backward(d, n, I, M, x.to(dev), off, wgu.to(dev), dh, dgu, h)
    dwd = torch.full((n, I, D), 3.0, device=dev)
    dwgu = torch.full((n, D, 2 * I), 3.0, device=dev)
    moe.moe_expert_weight_grad(d, n, M, h, I, dy.to(dev), D, off, dwd)
    moe.moe_expert_weight_grad(d, n, M, x.to(dev), D, dgu, 2 * I, off, dwgu)
    torch.cuda.synchronize()
    assert np.array_equal(dgu.float().cpu().numpy(), full["dgu"])
    assert np.array_equal(h.float().cpu().numpy(), full["h"])
    assert np.array_equal(dwd.cpu().numpy(), full["dwd"])
    assert np.array_equal(dwgu.cpu().numpy(), full["dwgu"])


@pytest.mark.parametrize("counts,D,I", [
    ([300, 0, 17, 330], 320, 192),   # ragged segments, an empty expert, rows past the last
    ([389], 192, 128),               # offsets NULL (the shared expert's form)
    # enough row blocks for the wide tiles of the gate_up GEMM
    ([12000], 128, 512),
    ([3000, 5100, 4000, 0, 6000, 3900, 4000, 6000], 128, 512),
])
def test_saved_gate_up_matches_recompute(counts, D, I):
    """moe_expert_ffn_train gives moe_expert_ffn's y_perm bit for bit and the
    fp32 G | U within the fp32 sums' bound (D 2^-24 sum |products|) of the
    oracle's; the backward fed that G | U gives the recomputing backward's
    dG | dU, H and every gradient bit for bit."""
    x, wgu, wd, dy, offsets = _ffn_case(counts, D, I, seed=5 + sum(counts))
    n, M = len(counts), x.shape[0]
    dense = n == 1
    extra = 0 if dense else 6
    cap = M + extra
    d = moe.make_desc(T=M, D=D, E=n, top_k=1, I=I)
    dev = "cuda"
    xd = torch.zeros(cap, D, dtype=bf16, device=dev)
    xd[:M] = x.to(dev)
    off = None if dense else torch.tensor(offsets, dtype=torch.int32, device=dev)
    wgud, wdd = wgu.to(dev), wd.to(dev)
    ws = moe.workspace(moe.moe_ffn_workspace_size(d, I, cap))
    y0 = torch.full((cap, D), -1.0, device=dev)
    moe.moe_expert_ffn(d, n, I, cap, xd, off, wgud, wdd, y0, ws)
    y1 = torch.full((cap, D), -1.0, device=dev)
    gu = torch.full((cap, 2 * I), -7.0, device=dev)
    moe.moe_expert_ffn_train(d, n, I, cap, xd, off, wgud, wdd, y1, gu, ws)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1), "training forward's y_perm differs"
    gu_c = gu.cpu().numpy()
    assert np.all(gu_c[M:] == -7.0), "rows past the segments were written"
    for j in range(n):
        a, b = int(offsets[j]), int(offsets[j + 1])
        xs = np32(x[a:b]).astype(np.float64)
        w1 = np32(wgu[j]).astype(np.float64)
        bound = D * 2.0 ** -24 * (np.abs(xs) @ np.abs(w1)) + 1e-30
        assert np.all(np.abs(gu_c[a:b] - xs @ w1) <= bound), f"G | U of expert {j}"
    rec = _run_ffn_bwd(x, wgu, wd, dy, None if dense else offsets, D, I, extra_rows=extra)
    sav = _run_ffn_bwd(x, wgu, wd, dy, None if dense else offsets, D, I, extra_rows=extra,
                       gu_saved=gu)
    for key in ("dgu", "h", "dx", "dwgu", "dwd"):
        assert np.array_equal(rec[key][:M] if key in ("dgu", "h") else rec[key],
                              sav[key][:M] if key in ("dgu", "h") else sav[key]), key


@pytest.mark.parametrize("counts,D,I", [([90, 0, 13, 151], 128, 192), ([389], 64, 128)])
def test_expert_ffn_backward_f32(counts, D, I):
    """fp32 layers: fp32 throughout, bounds with the fp32 unit roundoff."""
    x, wgu, wd, dy, offsets = _ffn_case(counts, D, I, seed=3 + sum(counts), dtype=torch.float32)
    out = _run_ffn_bwd(x, wgu, wd, dy, offsets if len(counts) > 1 else None, D, I,
                       extra_rows=5 if len(counts) > 1 else 0)
    _check_ffn_bwd(x, wgu, wd, dy, offsets, D, I, out, f"f32 ffn {counts}")


def test_expert_ffn_backward_dense():
    """offsets NULL: one expert owning every row (the shared expert's form)."""
    x, wgu, wd, dy, offsets = _ffn_case([389], 192, 128, seed=4)
    out = _run_ffn_bwd(x, wgu, wd, dy, None, 192, 128)
    _check_ffn_bwd(x, wgu, wd, dy, offsets, 192, 128, out, "dense ffn")


# ---------------------------------------------------------------------------
# Combine, router and input adjoints
# ---------------------------------------------------------------------------
def _routing(T, D, E, k, seed):
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(T, D)).astype(np.float32)
    wr = (rng.normal(size=(E, D)) * 0.1).astype(np.float32)
    r = om.router(x, wr, k)
    p = om.permute(None, r["topk_idx"], 0, E)
    c = om.counts_offsets_splits(r["topk_idx"], 0, E, E, 1)
    return r, p, c


def test_combine_backward():
    T, D, E, k = 203, 192, 6, 2
    r, p, c = _routing(T, D, E, k, seed=1)
    M = T * k
    g = torch.Generator().manual_seed(2)
    dout = _bf(torch.randn(T, D, generator=g))
    y = torch.randn(M, D, generator=g)
    d = moe.make_desc(T=T, D=D, E=E, top_k=k, I=64)
    dev = "cuda"
    pos = torch.tensor(p["pos"], dtype=torch.int32, device=dev)
    tw = torch.tensor(r["topk_w"], dtype=torch.float32, device=dev)
    dy = torch.zeros(M, D, dtype=bf16, device=dev)
    dtw = torch.empty(T, k, device=dev)
    dl = torch.empty(T, k, device=dev)
    dlp = torch.full((M,), 7.0, device=dev)
    moe.moe_combine_backward(d, dout.to(dev), y.to(dev), pos, tw, dy, dtw, dl, dlp)
    torch.cuda.synchronize()
    w32 = tw.cpu().numpy().astype(np.float64)
    ref = ob.combine_backward(np32(dout), y.numpy(), p["pos"], w32, M)
    dref = ob.topk_weight_backward(ref["dtopk_w"], r["topk_idx"], w32, r["probs"])
    dy_g = dy.float().cpu().numpy()
    # bf16 of the fp32 product: unit roundoffs 2^-8 and 2^-24
    assert np.all(np.abs(dy_g - ref["dy_perm"]) <= (2 ** -8 + 2 ** -23) * np.abs(ref["dy_perm"]))
    # fp32 dots of D products
    mag = np.zeros((T, k))
    for j in range(k):
        mag[:, j] = np.sum(np.abs(np32(dout) * y.numpy()[p["pos"][:, j]]), axis=1)
    bound = D * 2.0 ** -24 * mag + 1e-30
    assert np.all(np.abs(dtw.cpu().numpy() - ref["dtopk_w"]) <= bound)
    dl_ref = dref[np.arange(T)[:, None], r["topk_idx"]]
    assert np.all(np.abs(dl.cpu().numpy() - dl_ref) <= 2 * bound.max(axis=1, keepdims=True) + 1e-7)
    assert np.array_equal(dlp.cpu().numpy()[p["pos"]], dl.cpu().numpy())
    np.testing.assert_allclose(dl.cpu().numpy().sum(axis=1), 0.0, atol=1e-5)


def test_router_backward():
    counts = [0, 45, 1, 0, 100, 31, 64, 0, 7, 200, 3, 0]
    E, D = len(counts), 448
    M = sum(counts)
    cap = M + 10
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    g = torch.Generator().manual_seed(8)
    x = _bf(torch.randn(cap, D, generator=g))
    dlp = torch.randn(cap, generator=g)
    d = moe.make_desc(T=M, D=D, E=E, top_k=1, I=64)
    dev = "cuda"
    off = torch.tensor(offsets, dtype=torch.int32, device=dev)
    ws = moe.workspace(moe.moe_router_backward_workspace_size(d, cap))
    outs = []
    for _ in range(2):
        dw = torch.full((E, D), 9.0, device=dev)
        moe.moe_router_backward(d, cap, x.to(dev), off, dlp.to(dev), dw, ws)
        torch.cuda.synchronize()
        outs.append(dw.cpu().numpy())
    assert np.array_equal(outs[0], outs[1]), "not deterministic"
    xs = np32(x).astype(np.float64)
    ls = dlp.numpy().astype(np.float64)
    for e in range(E):
        a, b = offsets[e], offsets[e + 1]
        ref = (ls[a:b, None] * xs[a:b]).sum(axis=0)
        mag = np.abs(ls[a:b, None] * xs[a:b]).sum(axis=0)
        assert np.all(np.abs(outs[0][e] - ref) <= max(b - a, 1) * 2.0 ** -24 * mag + 1e-30), e
        if b == a:
            assert np.all(outs[0][e] == 0)


@pytest.mark.parametrize("with_shared,with_dout", [(True, True), (False, False)])
def test_input_backward(with_shared, with_dout):
    T, D, E, k = 150, 192, 7, 3
    r, p, c = _routing(T, D, E, k, seed=3)
    M = T * k
    g = torch.Generator().manual_seed(4)
    dxp = torch.randn(M, D, generator=g)
    dl = torch.randn(T, k, generator=g)
    wr = torch.randn(E, D, generator=g) * 0.1
    dsh = torch.randn(T, D, generator=g) if with_shared else None
    dout = _bf(torch.randn(T, D, generator=g)) if with_dout else None
    d = moe.make_desc(T=T, D=D, E=E, top_k=k, I=64)
    dev = "cuda"
    dx = torch.empty(T, D, dtype=bf16, device=dev)
    moe.moe_input_backward(d, dxp.to(dev), torch.tensor(p["pos"], dtype=torch.int32, device=dev),
                           torch.tensor(r["topk_idx"], dtype=torch.int32, device=dev), dl.to(dev),
                           wr.to(dev), None if dsh is None else dsh.to(dev),
                           None if dout is None else dout.to(dev), dx)
    torch.cuda.synchronize()
    routed = np.zeros((T, D))
    router = np.zeros((T, D))
    mag = np.zeros((T, D))
    for j in range(k):
        routed += dxp.numpy()[p["pos"][:, j]]
        router += dl.numpy()[:, j:j + 1].astype(np.float64) * wr.numpy()[r["topk_idx"][:, j]]
        mag += np.abs(dxp.numpy()[p["pos"][:, j]]) + np.abs(
            dl.numpy()[:, j:j + 1] * wr.numpy()[r["topk_idx"][:, j]])
    ref = routed + router
    if dsh is not None:
        ref += dsh.numpy()
        mag += np.abs(dsh.numpy())
    if dout is not None:
        ref += np32(dout)
        mag += np.abs(np32(dout))
    got = dx.float().cpu().numpy()
    # fp32 sum of 2k + 2 terms (each rounding <= 2^-24 of the running |sum|),
    # then one bf16 rounding (2^-8 of the computed value)
    fp32_err = (2 * k + 3) * 2.0 ** -24 * mag
    assert np.all(np.abs(got - ref) <= 2 ** -8 * np.abs(ref) + 2 * fp32_err)


# ---------------------------------------------------------------------------
# The whole layer backward
# ---------------------------------------------------------------------------
LAYERS = {
    "ragged": (wl.Workload("ragged_bwd", T=333, D=192, E=12, k=3, I=320, ep_size=3), 1.0),
    "zipf": (wl.Workload("zipf_bwd", T=600, D=128, E=32, k=4, I=128, zipf_s=3.0), 1.0),
    "shared_strong": (wl.Workload("shared_bwd", T=200, D=128, E=8, k=2, I=192, I_shared=128),
                      5.0),
    "one_expert": (wl.Workload("one_expert_bwd", T=65, D=64, E=1, k=1, I=64), 5.0),
    "k_equals_E": (wl.Workload("k_equals_E_bwd", T=130, D=128, E=4, k=4, I=192), 5.0),
    "tiny_fp32": (wl.WORKLOADS["tiny_fp32"], 1.0),
    "f32_shared": (wl.Workload("f32_shared_bwd", T=97, D=64, E=6, k=2, I=128, dtype="f32",
                               I_shared=64), 5.0),
}


def _layer(w, inp):
    d = moe.make_desc(T=w.T, D=w.D, E=w.E, top_k=w.k, I=w.I, ep_size=w.ep_size,
                      I_shared=w.I_shared, dtype=w.dtype)
    dv = to_dev(inp)
    lay = moe.LayerTrain(d, dv["w_router"], dv["w_gate_up"], dv["w_down"],
                         logit_bias=dv["logit_bias"], shared_gate_up=dv["shared_gate_up"],
                         shared_down=dv["shared_down"])
    lay.forward(dv["x"])
    return lay


def _scaled_inputs(w, seed, wscale):
    inp = wl.make_inputs(w, seed=seed)
    for kname in ("w_gate_up", "w_down", "shared_gate_up", "shared_down"):
        if inp[kname] is not None and wscale != 1.0:
            inp[kname] = (inp[kname].float() * wscale).to(inp[kname].dtype)
    return inp


@pytest.mark.parametrize("name", sorted(LAYERS))
def test_layer_backward(name):
    w, wscale = LAYERS[name]
    inp = _scaled_inputs(w, seed=11, wscale=wscale)
    lay = _layer(w, inp)
    g = torch.Generator().manual_seed(12)
    dout = torch.randn(w.T, w.D, generator=g).to(w.torch_dtype)
    lay.backward(dout.cuda())
    torch.cuda.synchronize()
    x = np32(inp["x"])
    ref_r = om.router(x, np32(inp["w_router"]), w.k, np32(inp["logit_bias"]))
    routing, _ = check_routing(npi(lay.topk_idx), np32(lay.topk_w), ref_r)
    ref = ob.layer_backward(x, np32(inp["w_router"]), np32(inp["w_gate_up"]),
                            np32(inp["w_down"]), w.k, np32(dout),
                            logit_bias=np32(inp["logit_bias"]),
                            shared_gate_up=np32(inp["shared_gate_up"]),
                            shared_down=np32(inp["shared_down"]), routing=routing)
    # fp32 layers: fp32 arithmetic throughout (unit roundoff 2^-24)
    f32 = w.dtype == "f32"
    ub = 2.0 ** -24 if f32 else 2.0 ** -8
    tols = dict(rtol=1e-4, atol_rms=1e-4, frob=1e-4) if f32 else {}
    # dx: one rounding of the whole sum, plus the layer part's tolerance
    moe_part = ref["dx"] - np32(dout)
    got = np32(lay.dx)
    err = np.abs(got - ref["dx"])
    rms = float(np.sqrt(np.mean(moe_part ** 2)))
    tol = (ub * np.abs(ref["dx"]) + tols.get("rtol", GRAD_RTOL) * np.abs(moe_part)
           + tols.get("atol_rms", GRAD_ATOL_RMS) * rms)
    assert np.all(err <= tol), f"dx: worst excess {float((err - tol).max()):.3e}"
    assert_grad_close(np32(lay.dw_router), ref["dw_router"], f"{name} dW_router", **tols)
    # expert weight gradients: the propagated bounds, with the GPU's dy_perm a
    # bf16 rounding of w dout
    wgu, wd = np32(inp["w_gate_up"]), np32(inp["w_down"])
    off = ref["offsets"]
    for e in range(w.E):
        a, b = int(off[e]), int(off[e + 1])
        if b == a:
            assert np.all(np32(lay.dw_gate_up[e]) == 0) and np.all(np32(lay.dw_down[e]) == 0)
            continue
        eb = _expert_bounds(ref["x_perm"][a:b], wgu[e], wd[e], ref["dy_perm"][a:b], True, ub)
        _within(np32(lay.dw_gate_up[e]), eb["r"]["dw_gate_up"], eb["b_wgu"],
                f"{name} dW_gate_up[{e}]")
        _within(np32(lay.dw_down[e]), eb["r"]["dw_down"], eb["b_wd"], f"{name} dW_down[{e}]")
    assert_grad_close(np32(lay.dw_gate_up), ref["dw_gate_up"], f"{name} dW_gate_up",
                      rtol=1.0, atol_rms=1.0)
    if w.I_shared:
        eb = _expert_bounds(x, np32(inp["shared_gate_up"]), np32(inp["shared_down"]),
                            np32(dout), False, ub)
        _within(np32(lay.dw_shared_gate_up), ref["dw_shared_gate_up"], eb["b_wgu"],
                f"{name} dW_shared_gate_up")
        _within(np32(lay.dw_shared_down), ref["dw_shared_down"], eb["b_wd"],
                f"{name} dW_shared_down")


@pytest.mark.parametrize("name", ["ragged", "shared_strong", "k_equals_E"])
def test_layer_backward_saved_matches_recompute(name):
    """LayerTrain with the forward's G | U saved (the default for bf16 layers)
    and with G | U recomputed: the same output and gradients, bit for bit."""
    w, wscale = LAYERS[name]
    inp = _scaled_inputs(w, seed=21, wscale=wscale)
    d = moe.make_desc(T=w.T, D=w.D, E=w.E, top_k=w.k, I=w.I, ep_size=w.ep_size,
                      I_shared=w.I_shared, dtype=w.dtype)
    dv = to_dev(inp)
    dout = torch.randn(w.T, w.D, generator=torch.Generator().manual_seed(22)).to(bf16).cuda()
    res = []
    for save in (True, False):
        lay = moe.LayerTrain(d, dv["w_router"], dv["w_gate_up"], dv["w_down"],
                             logit_bias=dv["logit_bias"], shared_gate_up=dv["shared_gate_up"],
                             shared_down=dv["shared_down"], save_gu=save)
        assert (lay.gu is not None) == save
        out = lay.forward(dv["x"]).clone()
        lay.backward(dout)
        torch.cuda.synchronize()
        ts = [out, lay.dx, lay.dw_router, lay.dw_gate_up, lay.dw_down]
        if w.I_shared:
            ts += [lay.dw_shared_gate_up, lay.dw_shared_down]
        res.append([t.clone() for t in ts])
    for i, (a, b) in enumerate(zip(*res)):
        assert torch.equal(a, b), f"tensor {i}"


def test_layer_backward_is_deterministic():
    w, wscale = LAYERS["zipf"]
    inp = _scaled_inputs(w, seed=2, wscale=wscale)
    lay = _layer(w, inp)
    dout = _bf(torch.randn(w.T, w.D, generator=torch.Generator().manual_seed(3))).cuda()
    res = []
    for _ in range(2):
        lay.backward(dout)
        torch.cuda.synchronize()
        res.append([t.clone() for t in (lay.dx, lay.dw_router, lay.dw_gate_up, lay.dw_down)])
    for a, b in zip(*res):
        assert torch.equal(a, b)


def test_layer_backward_full_size_sampled():
    """The worked-example geometry (T = 4096, D = 1024, E = 16, top-2, I = 2048)
    in the launch configuration the benchmark uses: weight gradients of two
    experts, the router gradient of those experts and the input gradient of
    64 tokens, each computed by the oracle from the tokens it depends on."""
    w = wl.WORKLOADS["worked_example_geometry"]
    inp = wl.make_inputs(w, seed=0)
    lay = _layer(w, inp)
    dout = _bf(torch.randn(w.T, w.D, generator=torch.Generator().manual_seed(5)))
    lay.backward(dout.cuda())
    torch.cuda.synchronize()
    x = np32(inp["x"])
    wr = np32(inp["w_router"])
    wgu, wd = np32(inp["w_gate_up"]), np32(inp["w_down"])
    g = np32(dout)
    ref_r = om.router(x, wr, w.k, None)
    (idx, wts), _ = check_routing(npi(lay.topk_idx), np32(lay.topk_w), ref_r)
    experts = [0, 11]
    rng = np.random.default_rng(0)
    tokens = np.sort(rng.choice(w.T, size=64, replace=False))
    need = set(tokens.tolist())
    for e in experts:
        need |= set(np.nonzero((idx == e).any(axis=1))[0].tolist())
    need = np.array(sorted(need))
    # per (token, slot) in the needed set: y, then dtopk_w and dlogit
    y = {}
    for e in range(w.E):
        ts, js = np.nonzero(idx[need] == e)
        if len(ts):
            ye = om.swiglu_ffn(x[need[ts]], wgu[e], wd[e])
            for r_, (t, j) in enumerate(zip(need[ts], js)):
                y[(t, j)] = ye[r_]
    dl = {}
    for t in need:
        dtw = np.array([float(g[t] @ y[(t, j)]) for j in range(w.k)])
        s = float(np.sum(wts[t] * dtw))
        for j in range(w.k):
            dl[(t, j)] = wts[t, j] * (dtw[j] - s)
    for e in experts:
        ts, js = np.nonzero(idx == e)
        rows = x[ts]
        dy = wts[ts, js][:, None] * g[ts]
        eb = _expert_bounds(rows, wgu[e], wd[e], dy, True)
        r = eb["r"]
        _within(np32(lay.dw_gate_up[e]), r["dw_gate_up"], eb["b_wgu"], f"full dW_gate_up[{e}]")
        _within(np32(lay.dw_down[e]), r["dw_down"], eb["b_wd"], f"full dW_down[{e}]")
        dwr = sum(dl[(t, j)] * x[t].astype(np.float64) for t, j in zip(ts, js))
        assert_grad_close(np32(lay.dw_router[e]), dwr, f"full dW_router[{e}]")
    dx_ref = np.zeros((len(tokens), w.D))
    for i, t in enumerate(tokens):
        acc = np.zeros(w.D)
        for j in range(w.k):
            e = int(idx[t, j])
            r = ob.swiglu_backward(x[t:t + 1], wgu[e], wd[e], wts[t, j] * g[t:t + 1])
            acc += r["d_rows"][0]
        for j in range(w.k):
            acc += dl[(t, j)] * wr[int(idx[t, j])].astype(np.float64)
        dx_ref[i] = acc + g[t]
    got = np32(lay.dx)[tokens]
    moe_part = dx_ref - g[tokens]
    rms = float(np.sqrt(np.mean(moe_part ** 2)))
    tol = 2 ** -8 * np.abs(dx_ref) + GRAD_RTOL * np.abs(moe_part) + GRAD_ATOL_RMS * rms
    assert np.all(np.abs(got - dx_ref) <= tol)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_layer_backward_no_tokens(dtype):
    """T = 0: every weight gradient is written as zero, nothing else is read."""
    w = wl.Workload("empty_bwd", T=0, D=128, E=4, k=2, I=128, dtype=dtype, I_shared=64)
    inp = wl.make_inputs(w, seed=1)
    lay = _layer(w, inp)
    for t in (lay.dw_router, lay.dw_gate_up, lay.dw_down, lay.dw_shared_gate_up,
              lay.dw_shared_down):
        t.fill_(7.0)
    lay.backward(torch.empty(0, w.D, dtype=w.torch_dtype, device="cuda"))
    torch.cuda.synchronize()
    for t in (lay.dw_router, lay.dw_gate_up, lay.dw_down, lay.dw_shared_gate_up,
              lay.dw_shared_down):
        assert torch.all(t == 0)
