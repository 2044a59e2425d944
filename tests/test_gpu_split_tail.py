"""The grouped GEMMs' split-K tail (needs MI355X). With wide tiles one
workgroup runs per CU, so R tiles take ceil(R / CUs) rounds; when a
workspace holds the part buffer, the tiles of the last, partial round are cut
along K into parts and a second launch sums them in part order (and, for the
gated GEMM, applies the SiLU gate). Cases built to have such a tail: the
calls with a part buffer (split) against the calls without one (whole
tiles), repeated calls against each other, and the oracle."""
import math

import numpy as np
import pytest
import torch

import mixture_experts_layer_fp32_amd as moe
from oracle import moe_oracle as om
from parity import assert_out_close, np32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu_and_library():
    assert torch.cuda.is_available(), "no GPU visible"
    moe.load_library()
    yield
    torch.cuda.synchronize()


def _split(counts, D, I, cus):
    """Host replica of the kernel's decision: tiles, tail tiles, parts."""
    R = sum(math.ceil(c / 256) for c in counts) * math.ceil(D / 256)
    r = R % cus
    parts = min(8, cus // r, (I // 64) // 32) if r else 0
    return R, r, parts


@pytest.mark.parametrize("packed,y_fp16", [(False, False), (True, False), (True, True)])
def test_down_split_tail(packed, y_fp16):
    E, D, I = 8, 4096, 4096
    counts = [2100] * 7 + [2050]
    M = sum(counts)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    R, rem, parts = _split(counts, D, I, cus)
    d = moe.make_desc(T=M, D=D, E=E, top_k=1, I=I, packed=packed, y_fp16=y_fp16)
    assert moe.moe_ffn_tile_shape(d, E, I, M, True, 1) == (256, 256)
    assert rem > 0 and parts >= 2, (R, rem, parts)  # the case has a split tail

    g = torch.Generator().manual_seed(5)
    xp = torch.randn(M, D, generator=g).to(torch.bfloat16)
    gu = (torch.randn(E, D, 2 * I, generator=g) * 0.02).to(torch.bfloat16)
    dn = (torch.randn(E, I, D, generator=g) * 0.02).to(torch.bfloat16)
    off_h = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    off = torch.from_numpy(off_h).cuda()
    xd, gud, dnd = xp.cuda(), gu.cuda(), dn.cuda()
    if packed:
        gud, dnd = moe.pack_expert_weights(d, gud, dnd)
    ydt = torch.float16 if y_fp16 else torch.float32

    y_split = torch.empty(M, D, dtype=ydt, device="cuda")
    ws = moe.workspace(moe.moe_ffn_workspace_size(d, I, M))
    moe.moe_expert_ffn(d, E, I, M, xd, off, gud, dnd, y_split, ws)
    h = torch.empty(M, I, dtype=torch.float16, device="cuda")
    y_whole = torch.empty_like(y_split)
    moe.moe_expert_gate_up(d, E, I, M, xd, off, gud, h)
    moe.moe_expert_down(d, E, I, M, h, off, dnd, y_whole)
    # the same call again gives the same bits (parts summed in a fixed order),
    # and so does the down GEMM called on its own with a part buffer
    y_again = torch.empty_like(y_split)
    moe.moe_expert_ffn(d, E, I, M, xd, off, gud, dnd, y_again, ws)
    y_down_ws = torch.empty_like(y_split)
    moe.moe_expert_down(d, E, I, M, h, off, dnd, y_down_ws,
                        ws=moe.workspace(moe.moe_down_workspace_size(d, M)))
    torch.cuda.synchronize()
    assert torch.equal(y_split.view(torch.int16), y_again.view(torch.int16))
    assert torch.equal(y_split.view(torch.int16), y_down_ws.view(torch.int16))

    # split and whole tiles differ only in the order of the fp32 sums
    a, b = y_split.float().cpu().numpy(), y_whole.float().cpu().numpy()
    scale = float(np.sqrt(np.mean(b.astype(np.float64) ** 2)))
    rt = 2e-3 if y_fp16 else 1e-5  # fp16: one rounding of a sum that moved by ~1e-7
    assert_out_close(a, b, "split tail vs whole tiles", rtol=rt, atol=1e-5 * scale)
    assert not np.array_equal(a, b) or y_fp16  # the tail really ran in parts

    # the last expert's first 256 rows (their tiles are in the tail) against
    # the oracle
    lo = int(off_h[-2])
    sub_off = np.array([0, 256], dtype=np.int64)
    ref = om.expert_ffn(np32(xp[lo:lo + 256]), sub_off, np32(gu[-1:]), np32(dn[-1:]))
    assert_out_close(a[lo:lo + 256], ref, "split-tail expert rows", rtol=2e-2, atol=1e-2 * scale)


KPART = 256 * 1024                 # bytes of one part
HDR = 16 * (256 + 1)               # header after the parts


def _split_gu(counts, I, D, cus):
    """Host replica of the gated GEMM's decision (256 x 128 H-column tiles,
    parts of at least 20 K-steps of 64)."""
    R = sum(math.ceil(c / 256) for c in counts) * math.ceil(I / 128)
    r = R % cus
    parts = min(8, cus // r, (D // 64) // 20) if r else 0
    return R, r, parts


def test_gate_up_split_tail():
    E, D, I = 8, 4096, 4096
    counts = [2100] * 7 + [2400]  # 73 row blocks x 32 column blocks: a 32-tile tail
    M = sum(counts)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    R, rem, parts = _split_gu(counts, I, D, cus)
    d = moe.make_desc(T=M, D=D, E=E, top_k=1, I=I, packed=True)
    assert moe.moe_ffn_tile_shape(d, E, I, M, True, 0) == (256, 256)
    assert rem > 0 and parts >= 2, (R, rem, parts)

    g = torch.Generator().manual_seed(6)
    xp = torch.randn(M, D, generator=g).to(torch.bfloat16)
    gu = (torch.randn(E, D, 2 * I, generator=g) * 0.02).to(torch.bfloat16)
    dn = (torch.randn(E, I, D, generator=g) * 0.02).to(torch.bfloat16)
    off_h = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    off = torch.from_numpy(off_h).cuda()
    xd = xp.cuda()
    gud, dnd = moe.pack_expert_weights(d, gu.cuda(), dn.cuda())

    nbytes = moe.moe_gate_up_workspace_size(d, I, M)
    ws = moe.workspace(nbytes)
    h_split = torch.empty(M, I, dtype=torch.float16, device="cuda")
    moe.moe_expert_gate_up(d, E, I, M, xd, off, gud, h_split, ws=ws)
    torch.cuda.synchronize()
    # the header after the parts says the tail ran split as the host decided
    cap = (nbytes - HDR) // KPART
    hdr = ws[cap * KPART: cap * KPART + 8].view(torch.int32).cpu().tolist()
    assert hdr == [rem, parts], (hdr, rem, parts)

    h_whole = torch.empty_like(h_split)
    moe.moe_expert_gate_up(d, E, I, M, xd, off, gud, h_whole)
    h_again = torch.empty_like(h_split)
    moe.moe_expert_gate_up(d, E, I, M, xd, off, gud, h_again, ws=ws)
    # the fused FFN splits both GEMMs in its own workspace: the same H, so the
    # same Y as the down GEMM (with its part buffer) on the split H
    y_fused = torch.empty(M, D, dtype=torch.float32, device="cuda")
    moe.moe_expert_ffn(d, E, I, M, xd, off, gud, dnd, y_fused,
                       moe.workspace(moe.moe_ffn_workspace_size(d, I, M)))
    y_sep = torch.empty_like(y_fused)
    moe.moe_expert_down(d, E, I, M, h_split, off, dnd, y_sep,
                        ws=moe.workspace(moe.moe_down_workspace_size(d, M)))
    torch.cuda.synchronize()
    assert torch.equal(h_split.view(torch.int16), h_again.view(torch.int16))
    assert torch.equal(y_fused.view(torch.int32), y_sep.view(torch.int32))

    # split and whole tiles differ only in the order of the fp32 sums of G
    # and U: H within two fp16 steps
    a, b = h_split.float().cpu().numpy(), h_whole.float().cpu().numpy()
    scale = float(np.sqrt(np.mean(b.astype(np.float64) ** 2)))
    assert_out_close(a, b, "split tail vs whole tiles (H)", rtol=2e-3, atol=1e-5 * scale)

    # the last expert's last 256 rows (their tiles hold the tail) against
    # the oracle, through Y
    lo = int(off_h[-1]) - 256
    sub_off = np.array([0, 256], dtype=np.int64)
    ref = om.expert_ffn(np32(xp[lo:lo + 256]), sub_off, np32(gu[-1:]), np32(dn[-1:]))
    y = y_sep.cpu().numpy()
    yscale = float(np.sqrt(np.mean(ref ** 2)))
    assert_out_close(y[lo:lo + 256], ref, "split-tail expert rows", rtol=2e-2, atol=1e-2 * yscale)
