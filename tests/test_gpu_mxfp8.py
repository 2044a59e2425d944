"""GPU parity of the MXFP8 expert FFN (include/moe_mxfp8.h) against the MXFP8
oracle: quantization and weight packing bit-exact (byte work), the FFN's
output within a bound derived from the arithmetic.

The bound: gfx950's block-scaled FP8 instruction (v_mfma_scale_f32_32x32x64_
f8f6f4) does not sum a 64-product group exactly: measured on random E4M3
operands over the whole range with random scales, its error reaches
2^-11.5 of the sum of the |products| (mean 2^-15), then the group sums are
accumulated in fp32. So an element of a K-long MX GEMM is within
2^-10 * sum_k |a_k w_k| of the exact value (a factor 2.8 of margin)."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_fp32_amd as moe
from oracle import moe_oracle as om
from oracle import mxfp8_oracle as mo
import workloads as wl
from parity import assert_out_close, check_routing, np32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_and_library():
    assert torch.cuda.is_available(), "no GPU visible"
    moe.load_library()
    yield
    torch.cuda.synchronize()


def _mixed_rows(rows, K, seed):
    """bf16 rows whose 32-blocks span many magnitudes, with all-zero blocks,
    blocks near E4M3 saturation and bf16 subnormals."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(rows, K, generator=g)
    blk = torch.exp2(torch.randint(-30, 30, (rows, K // 32), generator=g).float())
    x = x * blk.repeat_interleave(32, dim=1)
    x[0, :64] = 0.0                                   # zero blocks
    if rows > 3:
        x[1, :32] = torch.linspace(-1.0, 1.0, 32) * 2.0 ** 12
        x[2, 32:64] = 2.0 ** -130 * torch.arange(1, 33).float()  # subnormal block
        x[3, :32] = -0.0
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("rows,K", [(37, 64), (300, 1024), (1, 2048)])
def test_quantize_rows_bit_exact(rows, K):
    x = _mixed_rows(rows, K, seed=rows + K)
    codes = torch.empty(rows, K, dtype=torch.uint8, device="cuda")
    scales = torch.empty(rows, K // 32, dtype=torch.uint8, device="cuda")
    moe.moe_mxfp8_quantize_rows(x.cuda(), codes, scales)
    torch.cuda.synchronize()
    q_ref, s_ref = mo.mx_quantize(x.float().numpy())
    assert np.array_equal(scales.cpu().numpy(), s_ref)
    assert np.array_equal(codes.cpu().numpy(), q_ref)


def test_pack_weights_bit_exact():
    g = torch.Generator().manual_seed(11)
    w = (torch.randn(3, 256, 200, generator=g) * 0.02).to(torch.bfloat16)
    w[1, :32, 5] = 0.0
    codes = torch.empty(3, 200, 256, dtype=torch.uint8, device="cuda")
    scales = torch.empty(3, 200, 8, dtype=torch.uint8, device="cuda")
    moe.moe_mxfp8_pack_weights(w.cuda(), codes, scales)
    torch.cuda.synchronize()
    q_ref, s_ref = mo.pack_weights(w.float().numpy())
    assert np.array_equal(scales.cpu().numpy(), s_ref)
    assert np.array_equal(codes.cpu().numpy(), q_ref)


def _align(n):
    return (n + 255) // 256 * 256


def _run_ffn(x_perm, offsets, w_gu, w_d, D, I):
    """x_perm [M, D], weights [n, D, 2I] / [n, I, D] (bf16, CPU) -> GPU results:
    y [M, D], the bf16 H [M, I] and its MXFP8 codes / scales (from the
    workspace: H, then codes, then scales, each 256-byte aligned), and the
    activation codes."""
    M = x_perm.shape[0]
    n = w_gu.shape[0]
    d = moe.make_desc(T=max(M, 1), D=D, E=n, top_k=1, I=I, dtype="bf16")
    xq = torch.empty(M, D, dtype=torch.uint8, device="cuda")
    xs = torch.empty(M, D // 32, dtype=torch.uint8, device="cuda")
    moe.moe_mxfp8_quantize_rows(x_perm.cuda(), xq, xs)
    guq = torch.empty(n, 2 * I, D, dtype=torch.uint8, device="cuda")
    gus = torch.empty(n, 2 * I, D // 32, dtype=torch.uint8, device="cuda")
    dq = torch.empty(n, D, I, dtype=torch.uint8, device="cuda")
    ds = torch.empty(n, D, I // 32, dtype=torch.uint8, device="cuda")
    moe.moe_mxfp8_pack_weights(w_gu.cuda(), guq, gus)
    moe.moe_mxfp8_pack_weights(w_d.cuda(), dq, ds)
    y = torch.full((M, D), -7.0, device="cuda")
    ws = moe.workspace(moe.moe_ffn_mxfp8_workspace_size(d, I, M))
    off = torch.tensor(offsets, dtype=torch.int32, device="cuda")
    moe.moe_expert_ffn_mxfp8(d, n, I, M, xq, xs, off, guq, gus, dq, ds, y, ws)
    torch.cuda.synchronize()
    hb = M * I * 2
    h = ws[:hb].view(torch.bfloat16).view(M, I).float().cpu().numpy()
    hq = ws[_align(hb):_align(hb) + M * I].view(M, I).cpu().numpy()
    o = _align(hb) + _align(M * I)
    hs = ws[o:o + M * I // 32].view(M, I // 32).cpu().numpy()
    return dict(y=y.cpu().numpy(), h=h, hq=hq, hs=hs, xq=xq.cpu().numpy())


def _check_ffn(gpu, rows, x, expert_of, w_gu, w_d, what):
    """Compare the GPU FFN on the given rows with the oracle.

    H: within a tolerance of the oracle's H (fp32 vs float64 sums, each rounded
    to bf16). The quantization of H is a decision taken on H's bf16 values, so
    it is compared on the GPU's own H: the oracle quantizes that H (its codes
    and scales must match the GPU's bit for bit) and runs GEMM 2 on them (tight
    tolerance: fp32 accumulation only). End to end, Y is within the format's
    aggregate error of the oracle's own pipeline (a bf16 H that differs by one
    ulp can move a block's scale and requantize that block)."""
    MFMA_REL = 2.0 ** -10
    wgu = w_gu.float().numpy()
    wd = w_d.float().numpy()
    xf = x.float().numpy()
    D, I = wd.shape[2], wd.shape[1]
    dq, ds = mo.pack_weights(wd)
    y_ref = np.zeros((len(rows), D))
    h_ref = np.zeros((len(rows), I))
    y_own = np.zeros((len(rows), D))
    bound = np.zeros((len(rows), D))
    q_own, s_own = mo.mx_quantize(gpu["h"][rows])
    for e in np.unique(expert_of):
        sel = expert_of == e
        r = mo.expert_ffn_mxfp8(xf[rows[sel]], np.array([0, int(sel.sum())]), wgu[e:e + 1],
                                wd[e:e + 1])
        y_ref[sel] = r["y"]
        h_ref[sel] = r["h"]
        assert np.array_equal(gpu["xq"][rows[sel]], r["xq"]), what
        y_own[sel] = mo.mx_gemm(q_own[sel], s_own[sel], dq[e], ds[e])
        bound[sel] = MFMA_REL * (np.abs(mo.mx_dequantize(q_own[sel], s_own[sel]))
                                 @ np.abs(mo.mx_dequantize(dq[e], ds[e])).T)
    scale_h = float(np.sqrt(np.mean(h_ref ** 2)))
    assert_out_close(gpu["h"][rows], h_ref, f"{what} H", rtol=1e-2, atol=1e-3 * scale_h)
    assert np.array_equal(gpu["hs"][rows], s_own), f"{what}: H scales"
    assert np.array_equal(gpu["hq"][rows], q_own), f"{what}: H codes"
    err = np.abs(gpu["y"][rows] - y_own)
    bad = err > bound
    assert not bad.any(), (f"{what} Y (GEMM 2 on the GPU's H): {int(bad.sum())} of {bad.size} "
                           f"beyond 2^-10 sum|terms|; worst ratio {float((err / bound).max()):.2f}")
    rel = np.linalg.norm(gpu["y"][rows] - y_ref) / np.linalg.norm(y_ref)
    assert rel < 5e-3, f"{what}: Y differs from the oracle pipeline by {rel:.2e} (relative)"


def test_expert_ffn_mxfp8_small_ragged():
    # 4 experts (one empty), segments spanning several 320-row tiles and ragged tails
    D, I = 256, 384
    counts = [700, 0, 33, 345]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    M = int(offsets[-1])
    g = torch.Generator().manual_seed(21)
    x = torch.randn(M, D, generator=g).to(torch.bfloat16)
    w_gu = (torch.randn(4, D, 2 * I, generator=g) * 0.05).to(torch.bfloat16)
    w_d = (torch.randn(4, I, D, generator=g) * 0.05).to(torch.bfloat16)
    gpu = _run_ffn(x, offsets, w_gu, w_d, D, I)
    rows = np.arange(M)
    _check_ffn(gpu, rows, x, np.searchsorted(offsets, rows, side="right") - 1, w_gu, w_d,
               "mxfp8 small")


def test_expert_ffn_mxfp8_worked_example_geometry_sampled():
    """16 experts x ~512 rows, D = 1024, I = 2048 (the full routed shape of the
    16-expert top-2 layer); the oracle recomputes a sample of rows (each row's
    output depends only on its own row and its expert's weights)."""
    w = wl.WORKLOADS["worked_example_geometry"]
    D, I = w.D, w.I
    inp = wl.make_inputs(w, seed=0)
    counts = [504, 517, 477, 510, 489, 547, 528, 510, 509, 538, 488, 579, 510, 492, 539, 455]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    M = int(offsets[-1])
    g = torch.Generator().manual_seed(5)
    x = torch.randn(M, D, generator=g).to(torch.bfloat16)
    gpu = _run_ffn(x, offsets, inp["w_gate_up"], inp["w_down"], D, I)
    assert np.all(np.isfinite(gpu["y"]))
    rng = np.random.default_rng(9)
    rows = np.sort(rng.choice(M, size=192, replace=False))
    _check_ffn(gpu, rows, x, np.searchsorted(offsets, rows, side="right") - 1,
               inp["w_gate_up"], inp["w_down"], "mxfp8 C2 sampled")


def test_split_entry_points_match_ffn():
    """gate_up -> quantize H -> down through the split entry points gives the
    one-call FFN's output bit for bit (the same kernels)."""
    D, I = 256, 256
    counts = [100, 0, 290, 37]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    M = int(offsets[-1])
    g = torch.Generator().manual_seed(31)
    x = torch.randn(M, D, generator=g).to(torch.bfloat16)
    w_gu = (torch.randn(4, D, 2 * I, generator=g) * 0.05).to(torch.bfloat16)
    w_d = (torch.randn(4, I, D, generator=g) * 0.05).to(torch.bfloat16)
    full = _run_ffn(x, offsets, w_gu, w_d, D, I)
    d = moe.make_desc(T=M, D=D, E=4, top_k=1, I=I, dtype="bf16")
    u8 = torch.uint8
    xq = torch.empty(M, D, dtype=u8, device="cuda")
    xs = torch.empty(M, D // 32, dtype=u8, device="cuda")
    moe.moe_mxfp8_quantize_rows(x.cuda(), xq, xs)
    guq = torch.empty(4, 2 * I, D, dtype=u8, device="cuda")
    gus = torch.empty(4, 2 * I, D // 32, dtype=u8, device="cuda")
    dq = torch.empty(4, D, I, dtype=u8, device="cuda")
    ds = torch.empty(4, D, I // 32, dtype=u8, device="cuda")
    moe.moe_mxfp8_pack_weights(w_gu.cuda(), guq, gus)
    moe.moe_mxfp8_pack_weights(w_d.cuda(), dq, ds)
    off = torch.tensor(offsets, dtype=torch.int32, device="cuda")
    h = torch.zeros(M, I, dtype=torch.bfloat16, device="cuda")
    hq = torch.empty(M, I, dtype=u8, device="cuda")
    hs = torch.empty(M, I // 32, dtype=u8, device="cuda")
    y = torch.full((M, D), -7.0, device="cuda")
    moe.moe_expert_gate_up_mxfp8(d, 4, I, M, xq, xs, off, guq, gus, h)
    moe.moe_mxfp8_quantize_rows(h, hq, hs)
    moe.moe_expert_down_mxfp8(d, 4, I, M, hq, hs, off, dq, ds, y)
    torch.cuda.synchronize()
    assert np.array_equal(h.float().cpu().numpy(), full["h"])
    assert np.array_equal(y.cpu().numpy(), full["y"])


def test_layer_forward_mxfp8_small():
    """The layer with the MXFP8 expert FFN against the oracle pipeline (router,
    permute, MXFP8 FFN, combine) at the layer's tolerance."""
    w = wl.scaled(wl.WORKLOADS["worked_example_geometry"], T=300, D=256, E=8, k=2, I=256)
    inp = wl.make_inputs(w, seed=3)
    d = moe.make_desc(T=w.T, D=w.D, E=w.E, top_k=w.k, I=w.I, ep_size=w.ep_size, dtype="bf16")
    dv = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    lay = moe.LayerForwardMXFP8(d, dv["w_router"], dv["w_gate_up"], dv["w_down"])
    out = lay(dv["x"])
    torch.cuda.synchronize()
    x = np32(inp["x"])
    ref_r = om.router(x, np32(inp["w_router"]), w.k, None)
    routing, _ = check_routing(lay.topk_idx.cpu().numpy(), lay.topk_w.cpu().numpy(), ref_r)
    p = om.permute(x, routing[0], 0, w.E)
    c = om.counts_offsets_splits(routing[0], 0, w.E, w.E, w.ep_size)
    ffn = mo.expert_ffn_mxfp8(p["x_perm"], c["offsets"], np32(inp["w_gate_up"]),
                              np32(inp["w_down"]))
    M = w.T * w.k
    assert torch.equal(lay.x_perm.cpu(), inp["x"][torch.from_numpy(p["perm_src"])])
    xq, xs = mo.mx_quantize(np32(lay.x_perm))
    assert np.array_equal(lay.xq.cpu().numpy(), xq)
    assert np.array_equal(lay.xs.cpu().numpy(), xs)
    # expert outputs: the residual dominates the layer output, so they are
    # checked on their own (relative Frobenius error, as for the FFN alone)
    y = np32(lay.y_perm)[:M]
    rel = np.linalg.norm(y - ffn["y"]) / np.linalg.norm(ffn["y"])
    assert rel < 5e-3, rel
    ref = om.combine(ffn["y"], p["pos"], routing[1], residual=x)
    assert_out_close(np32(out), ref, "mxfp8 layer")

