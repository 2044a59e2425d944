"""The C ABI library on a machine without a GPU: it loads, exports every
symbol include/*.h declares, and rejects bad arguments on the host before
any HIP call (so none of these calls needs a device)."""
import ctypes
import glob
import os
import re
import subprocess

import pytest
import torch

import mixture_experts_layer_fp32_amd as moe
from mixture_experts_layer_fp32_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):  # build only when nothing is built yet
        from mixture_experts_layer_fp32_amd import build
        build.build()
    return B.load_library()


def _declared():
    text = "\n".join(open(h).read() for h in HEADERS)
    return set(re.findall(r"^\s*(?:moe_status|size_t|const char\*|int32_t)\s+(moe_\w+)\(",
                          text, re.M))


def test_header_declarations_match_binding():
    assert _declared() == set(B.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in nm.splitlines() if " T " in ln and "moe_" in ln}
    assert _declared() <= exported
    assert {s for s in exported if s.startswith("moe_")} == _declared()


def _desc(**kw):
    base = dict(T=64, D=128, E=16, top_k=2, I=256, ep_size=4, ep_rank=0, dtype="bf16")
    base.update(kw)
    return B.make_desc(**base)


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails its checks


@pytest.mark.parametrize("kw,code", [
    (dict(E=15), B.MOE_ERR_INVALID_ARG),          # E not divisible by ep_size
    (dict(top_k=0), B.MOE_ERR_INVALID_ARG),
    (dict(top_k=17, E=32), B.MOE_ERR_UNSUPPORTED),
    (dict(top_k=20, E=16), B.MOE_ERR_INVALID_ARG),  # k > E
    (dict(ep_rank=4), B.MOE_ERR_INVALID_ARG),
    (dict(T=-1), B.MOE_ERR_INVALID_ARG),
    (dict(D=100), B.MOE_ERR_UNSUPPORTED),
    (dict(I=96), B.MOE_ERR_UNSUPPORTED),
    (dict(E=2048, ep_size=1), B.MOE_ERR_UNSUPPORTED),
    (dict(D=0), B.MOE_ERR_INVALID_ARG),
    (dict(D=B.MOE_MAX_WIDTH + 64), B.MOE_ERR_UNSUPPORTED),
    (dict(I=B.MOE_MAX_WIDTH + 64), B.MOE_ERR_UNSUPPORTED),
])
def test_route_rejects_bad_descriptor(lib, kw, code):
    d = _desc(**kw)
    st = lib.moe_route(ctypes.byref(d), FAKE, FAKE, None, None, None, FAKE, FAKE, None, 0, None)
    assert st == code, (kw, st)


def test_bad_dtype_and_norm(lib):
    d = _desc()
    d.act_dtype = 7
    assert lib.moe_route(ctypes.byref(d), FAKE, FAKE, None, None, None, FAKE, FAKE,
                         None, 0, None) == B.MOE_ERR_UNSUPPORTED
    d = _desc()
    d.norm_topk = 2
    assert lib.moe_route(ctypes.byref(d), FAKE, FAKE, None, None, None, FAKE, FAKE,
                         None, 0, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_route(None, FAKE, FAKE, None, None, None, FAKE, FAKE,
                         None, 0, None) == B.MOE_ERR_INVALID_ARG


def test_null_required_pointers(lib):
    d = _desc()
    assert lib.moe_route(ctypes.byref(d), None, FAKE, None, None, None, FAKE, FAKE,
                         None, 0, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_route(ctypes.byref(d), FAKE, FAKE, None, None, None, FAKE, None,
                         None, 0, None) == B.MOE_ERR_INVALID_ARG
    ws = lib.moe_permute_workspace_size(ctypes.byref(d), 0, 16)
    assert lib.moe_permute(ctypes.byref(d), FAKE, None, 0, 16, 128, FAKE, FAKE, None, FAKE, FAKE,
                           None, FAKE, ws, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_unpermute_combine(ctypes.byref(d), FAKE, None, FAKE, None, None, 0, 0, FAKE,
                                     None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_ffn(ctypes.byref(d), 4, 256, 128, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                              1 << 30, None) == B.MOE_ERR_INVALID_ARG


def test_permute_noalloc_checks(lib):
    """The no-workspace permute runs moe_permute's argument checks on the
    host before it looks up its scratch (so none of these needs a GPU)."""
    d = _desc()
    call = lambda eb, ee, cap, idx: lib.moe_permute_noalloc(  # noqa: E731
        ctypes.byref(d), FAKE, idx, eb, ee, cap, FAKE, FAKE, None, FAKE, FAKE, FAKE, None)
    assert call(8, 4, 128, FAKE) == B.MOE_ERR_INVALID_ARG
    assert call(4, 8, 127, FAKE) == B.MOE_ERR_CAPACITY
    assert call(4, 8, 128, None) == B.MOE_ERR_INVALID_ARG
    bad = _desc(E=15)
    assert lib.moe_permute_noalloc(ctypes.byref(bad), FAKE, FAKE, 0, 15, 128, FAKE, FAKE, None,
                                   FAKE, FAKE, FAKE, None) == B.MOE_ERR_INVALID_ARG


def test_permute_range_capacity_workspace(lib):
    d = _desc()
    ws = lib.moe_permute_workspace_size(ctypes.byref(d), 4, 8)
    args = lambda eb, ee, cap, wsb: lib.moe_permute(  # noqa: E731
        ctypes.byref(d), FAKE, FAKE, eb, ee, cap, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, wsb,
        None)
    assert args(8, 4, 128, ws) == B.MOE_ERR_INVALID_ARG      # empty range
    assert args(-1, 4, 128, ws) == B.MOE_ERR_INVALID_ARG
    assert args(4, 17, 128, ws) == B.MOE_ERR_INVALID_ARG     # past E
    assert args(4, 8, 127, ws) == B.MOE_ERR_CAPACITY        # T*min(k, n) = 128
    assert args(4, 5, 63, ws) == B.MOE_ERR_CAPACITY         # one expert: T*1 = 64
    assert args(4, 8, 128, ws - 1) == B.MOE_ERR_WORKSPACE


def test_ffn_and_combine_checks(lib):
    d = _desc()
    need = lib.moe_ffn_workspace_size(ctypes.byref(d), 256, 128)
    assert need >= 128 * 256 * 2
    ffn = lambda n, inter, cap, wsb: lib.moe_expert_ffn(  # noqa: E731
        ctypes.byref(d), n, inter, cap, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, wsb, None)
    assert ffn(0, 256, 128, need) == B.MOE_ERR_INVALID_ARG
    assert ffn(4, 100, 128, need) == B.MOE_ERR_UNSUPPORTED
    assert ffn(4, 256, -1, need) == B.MOE_ERR_INVALID_ARG
    assert ffn(4, 256, 128, need - 1) == B.MOE_ERR_WORKSPACE
    assert ffn(4, 256, 0, 0) == B.MOE_OK  # nothing to do
    comb = lambda rb, rr, res: lib.moe_unpermute_combine(  # noqa: E731
        ctypes.byref(d), FAKE, FAKE, FAKE, res, None, rb, rr, FAKE, None)
    assert comb(-1, 4, None) == B.MOE_ERR_INVALID_ARG
    assert comb(60, 5, FAKE) == B.MOE_ERR_INVALID_ARG       # rows past T
    assert comb(0, 0, FAKE) == B.MOE_ERR_INVALID_ARG        # residual with no rows


def test_down_workspace(lib):
    """moe_expert_down's optional part buffer: moe_down_workspace_size gives
    its bytes (none for fp32 layers, part of moe_ffn_workspace_size), a
    smaller buffer is WORKSPACE; the checks run before any HIP call."""
    d, d32 = _desc(), _desc(dtype="f32")
    need = lib.moe_down_workspace_size(ctypes.byref(d), 128)
    assert need > 0 and lib.moe_down_workspace_size(ctypes.byref(d32), 128) == 0
    assert lib.moe_ffn_workspace_size(ctypes.byref(d), 256, 128) >= need + 128 * 256 * 2
    assert lib.moe_expert_down(ctypes.byref(d), 4, 256, 128, FAKE, FAKE, FAKE, FAKE, FAKE,
                               need - 1, None) == B.MOE_ERR_WORKSPACE
    assert lib.moe_down_workspace_size(None, 128) == 0


def test_gate_up_workspace(lib):
    """moe_expert_gate_up's optional part buffer: moe_gate_up_workspace_size
    gives its bytes (none for fp32 layers or inter < 1), the FFN workspace
    holds the larger of the two GEMMs' part buffers, a smaller buffer is
    WORKSPACE; the checks run before any HIP call."""
    d, d32 = _desc(), _desc(dtype="f32")
    need = lib.moe_gate_up_workspace_size(ctypes.byref(d), 256, 128)
    assert need > 0 and lib.moe_gate_up_workspace_size(ctypes.byref(d32), 256, 128) == 0
    assert lib.moe_gate_up_workspace_size(ctypes.byref(d), 0, 128) == 0
    assert lib.moe_gate_up_workspace_size(None, 256, 128) == 0
    down = lib.moe_down_workspace_size(ctypes.byref(d), 128)
    assert lib.moe_ffn_workspace_size(ctypes.byref(d), 256, 128) >= max(need, down) + 128 * 256 * 2
    assert lib.moe_expert_gate_up(ctypes.byref(d), 4, 256, 128, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  need - 1, None) == B.MOE_ERR_WORKSPACE


def test_ffn_offsets_required_for_several_experts(lib):
    """offsets == NULL means one dense expert: every FFN entry point rejects
    it with more than one expert instead of running expert 0 over all rows."""
    d = _desc()
    need = lib.moe_ffn_workspace_size(ctypes.byref(d), 256, 128)
    assert lib.moe_expert_ffn(ctypes.byref(d), 4, 256, 128, FAKE, None, FAKE, FAKE, FAKE, FAKE,
                              need, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_gate_up(ctypes.byref(d), 4, 256, 128, FAKE, None, FAKE, FAKE, None, 0,
                                  None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_down(ctypes.byref(d), 4, 256, 128, FAKE, None, FAKE, FAKE, None, 0,
                               None) == B.MOE_ERR_INVALID_ARG
    # one expert without offsets is the dense case (zero rows: no launch)
    assert lib.moe_expert_ffn(ctypes.byref(d), 1, 256, 0, None, None, None, None, None, None,
                              0, None) == B.MOE_OK


def test_route_workspace(lib):
    """bf16 activations with more than 16 experts route through a workspace
    of moe_route_workspace_size() bytes (partial logits, row norms, the split
    gate weight): WORKSPACE when it is missing or smaller. At most 16 experts
    (one workgroup per 16 tokens does it all) and fp32 activations need
    none."""
    assert lib.moe_route_workspace_size(ctypes.byref(_desc())) == 0  # E = 16
    d = _desc(E=32)
    need = lib.moe_route_workspace_size(ctypes.byref(d))
    assert need >= d.T * d.E * 4 + d.T * 8
    assert lib.moe_route(ctypes.byref(d), FAKE, FAKE, None, None, None, FAKE, FAKE,
                         None, 0, None) == B.MOE_ERR_WORKSPACE
    assert lib.moe_route(ctypes.byref(d), FAKE, FAKE, None, None, None, FAKE, FAKE,
                         FAKE, need - 1, None) == B.MOE_ERR_WORKSPACE
    assert lib.moe_route_workspace_size(ctypes.byref(_desc(dtype="f32"))) == 0
    d0 = _desc(T=0)
    assert lib.moe_route_workspace_size(ctypes.byref(d0)) == 0
    assert lib.moe_route(ctypes.byref(d0), FAKE, FAKE, None, None, None, FAKE, FAKE,
                         None, 0, None) == B.MOE_OK


def test_expert_out_dtype_checks(lib):
    """expert_out_dtype: fp32 or fp16 (bf16 layers only); the backward, the
    training forward and the MXFP8 FFN take fp32 expert outputs only."""
    d = _desc()
    d.expert_out_dtype = 5
    assert lib.moe_route(ctypes.byref(d), FAKE, FAKE, None, None, None, FAKE, FAKE,
                         None, 0, None) == B.MOE_ERR_INVALID_ARG
    d32 = _desc(dtype="f32")
    d32.expert_out_dtype = B.MOE_F16
    assert lib.moe_route(ctypes.byref(d32), FAKE, FAKE, None, None, None, FAKE, FAKE,
                         None, 0, None) == B.MOE_ERR_UNSUPPORTED
    dh = _desc(y_fp16=True)
    fneed = lib.moe_ffn_workspace_size(ctypes.byref(dh), 256, 128)
    assert lib.moe_expert_ffn_train(ctypes.byref(dh), 4, 256, 128, FAKE, FAKE, FAKE, FAKE, FAKE,
                                    FAKE, FAKE, fneed, None) == B.MOE_ERR_UNSUPPORTED
    assert lib.moe_combine_backward(ctypes.byref(dh), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                    None, None) == B.MOE_ERR_UNSUPPORTED
    dh.D, dh.I = 256, 256
    assert lib.moe_expert_gate_up_mxfp8(ctypes.byref(dh), 4, 256, 128, FAKE, FAKE, FAKE, FAKE,
                                        FAKE, FAKE, None) == B.MOE_ERR_UNSUPPORTED
    # the layer workspace holds fp16 expert outputs: smaller than with fp32
    full = _desc(I_shared=128)
    half = _desc(I_shared=128, y_fp16=True)
    M = 64 * 2
    assert (lib.moe_workspace_size(ctypes.byref(full)) - lib.moe_workspace_size(ctypes.byref(half))
            >= (M * 128 + 64 * 128) * 2)


def test_ffn_tile_shape_query(lib):
    """The tile-shape query is host arithmetic: wide 256 x 256 tiles for many
    rows per expert, 320-row narrow tiles when wide ones would leave CUs idle,
    64 x 64 for fp32 layers."""
    d = _desc(D=1536, I=1536)
    r, c = ctypes.c_int32(), ctypes.c_int32()
    q = lambda dd, n, inter, cap, off, gemm: lib.moe_ffn_tile_shape(  # noqa: E731
        ctypes.byref(dd), n, inter, cap, off, gemm, ctypes.byref(r), ctypes.byref(c))
    assert q(d, 8, 1536, 10000, 1, 0) == B.MOE_OK and (r.value, c.value) == (256, 256)
    assert q(d, 8, 1536, 10000, 1, 1) == B.MOE_OK and (r.value, c.value) == (256, 256)
    d2 = _desc(D=1024, I=2048)
    assert q(d2, 16, 2048, 8192, 1, 0) == B.MOE_OK and (r.value, c.value) == (320, 128)
    assert q(_desc(dtype="f32"), 4, 256, 128, 1, 1) == B.MOE_OK and (r.value, c.value) == (64, 64)
    assert q(d, 8, 1536, 10000, 1, 2) == B.MOE_ERR_INVALID_ARG
    assert q(d, 8, 1536, 10000, 0, 0) == B.MOE_ERR_INVALID_ARG   # dense needs one expert
    assert q(d, 8, 96, 10000, 1, 0) == B.MOE_ERR_UNSUPPORTED
    assert lib.moe_ffn_tile_shape(ctypes.byref(d), 8, 1536, 100, 1, 0, None,
                                  ctypes.byref(c)) == B.MOE_ERR_INVALID_ARG


def test_mxfp8_checks(lib):
    q = lambda rows, K, x: lib.moe_mxfp8_quantize_rows(rows, K, x, FAKE, FAKE, None)  # noqa: E731
    assert q(-1, 64, FAKE) == B.MOE_ERR_INVALID_ARG
    assert q(4, 48, FAKE) == B.MOE_ERR_INVALID_ARG        # K not a multiple of 32
    assert q(4, 64, None) == B.MOE_ERR_INVALID_ARG
    assert q(0, 64, None) == B.MOE_OK                     # nothing to do
    assert q(1 << 36, 1 << 10, FAKE) == B.MOE_ERR_UNSUPPORTED
    pk = lambda n, K, N, w: lib.moe_mxfp8_pack_weights(n, K, N, w, FAKE, FAKE, None)  # noqa: E731
    assert pk(2, 33, 8, FAKE) == B.MOE_ERR_INVALID_ARG
    assert pk(2, 64, 0, FAKE) == B.MOE_ERR_INVALID_ARG
    assert pk(-1, 64, 8, FAKE) == B.MOE_ERR_INVALID_ARG
    assert pk(2, 64, 8, None) == B.MOE_ERR_INVALID_ARG
    assert pk(0, 64, 8, None) == B.MOE_OK
    d = _desc()
    d.D, d.I = 256, 256
    need = lib.moe_ffn_mxfp8_workspace_size(ctypes.byref(d), 256, 128)
    assert need >= 128 * 256 * 3 + 128 * 256 // 32
    ffn = lambda dd, inter, cap, off, wsb: lib.moe_expert_ffn_mxfp8(  # noqa: E731
        ctypes.byref(dd), 4, inter, cap, FAKE, FAKE, off, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
        wsb, None)
    assert ffn(d, 192, 128, FAKE, need) == B.MOE_ERR_UNSUPPORTED   # inter not a multiple of 128
    assert ffn(d, 256, 128, None, need) == B.MOE_ERR_INVALID_ARG   # offsets required
    assert ffn(d, 256, 128, FAKE, need - 1) == B.MOE_ERR_WORKSPACE
    assert ffn(d, 256, 0, None, 0) == B.MOE_OK                     # nothing to do
    d32 = _desc()
    d32.D, d32.I, d32.act_dtype = 256, 256, B.MOE_F32
    assert ffn(d32, 256, 128, FAKE, need) == B.MOE_ERR_UNSUPPORTED  # bf16 layers only
    d64 = _desc()
    d64.D, d64.I = 192, 256
    assert ffn(d64, 256, 128, FAKE, need) == B.MOE_ERR_UNSUPPORTED  # D not a multiple of 128
    gu = lambda dd, off, h: lib.moe_expert_gate_up_mxfp8(  # noqa: E731
        ctypes.byref(dd), 4, 256, 128, FAKE, FAKE, off, FAKE, FAKE, h, None)
    dn = lambda dd, off, y: lib.moe_expert_down_mxfp8(  # noqa: E731
        ctypes.byref(dd), 4, 256, 128, FAKE, FAKE, off, FAKE, FAKE, y, None)
    assert gu(d, FAKE, None) == B.MOE_ERR_INVALID_ARG
    assert gu(d, None, FAKE) == B.MOE_ERR_INVALID_ARG
    assert gu(d32, FAKE, FAKE) == B.MOE_ERR_UNSUPPORTED
    assert dn(d, FAKE, None) == B.MOE_ERR_INVALID_ARG
    assert dn(d64, FAKE, FAKE) == B.MOE_ERR_UNSUPPORTED


def test_backward_checks(lib):
    d = _desc()
    d32 = _desc(dtype="f32")
    dplain = _desc(norm_topk=False)
    cb = lambda dd, dout, dl: lib.moe_combine_backward(  # noqa: E731
        ctypes.byref(dd), dout, FAKE, FAKE, FAKE, FAKE, None, dl, None, None)
    assert cb(d, None, FAKE) == B.MOE_ERR_INVALID_ARG
    assert cb(d, FAKE, None) == B.MOE_ERR_INVALID_ARG
    assert cb(dplain, FAKE, FAKE) == B.MOE_ERR_UNSUPPORTED   # renormalised weights only
    need = lib.moe_ffn_backward_workspace_size(ctypes.byref(d), 256, 128)
    assert need >= 128 * 256 * (4 + 4 + 2)                    # dH fp32, dG|dU and H bf16
    fb = lambda dd, n, inter, cap, off, wsb, gs=None: lib.moe_expert_ffn_backward(  # noqa: E731
        ctypes.byref(dd), n, inter, cap, FAKE, off, FAKE, FAKE, FAKE, gs, FAKE, FAKE, FAKE, FAKE,
        wsb, None)
    assert fb(d, 4, 256, 128, FAKE, need - 1) == B.MOE_ERR_WORKSPACE
    assert fb(d, 4, 256, 128, None, need) == B.MOE_ERR_INVALID_ARG   # one expert without offsets
    assert fb(d, 4, 96, 128, FAKE, need) == B.MOE_ERR_UNSUPPORTED
    assert fb(dplain, 4, 256, 128, FAKE, need) == B.MOE_ERR_UNSUPPORTED
    need32 = lib.moe_ffn_backward_workspace_size(ctypes.byref(d32), 256, 128)
    assert need32 >= 128 * 256 * (4 + 8 + 4)                  # fp32 layers: fp32 intermediates
    assert fb(d32, 4, 256, 128, FAKE, need32 - 1) == B.MOE_ERR_WORKSPACE
    assert fb(d32, 4, 256, 128, FAKE, need32, FAKE) == B.MOE_ERR_UNSUPPORTED  # saved G|U: bf16
    assert fb(d, 4, 256, 128, FAKE, need - 1, FAKE) == B.MOE_ERR_WORKSPACE
    assert fb(d, 4, 256, 1 << 20, FAKE, 1 << 40) == B.MOE_ERR_UNSUPPORTED  # rows x 2I >= 2^30 B
    assert fb(d, 0, 256, 128, FAKE, need) == B.MOE_ERR_INVALID_ARG
    gub = lambda dd, off, dh: lib.moe_expert_gate_up_backward(  # noqa: E731
        ctypes.byref(dd), 4, 256, 128, FAKE, off, FAKE, dh, FAKE, FAKE, None)
    assert gub(d, FAKE, None) == B.MOE_ERR_INVALID_ARG
    assert gub(d, None, FAKE) == B.MOE_ERR_INVALID_ARG
    assert gub(dplain, FAKE, FAKE) == B.MOE_ERR_UNSUPPORTED
    wg = lambda n, cap, P, Q, off, c: lib.moe_expert_weight_grad(  # noqa: E731
        ctypes.byref(d), n, cap, FAKE, P, FAKE, Q, off, c, None)
    assert wg(4, 128, 96, 256, FAKE, FAKE) == B.MOE_ERR_UNSUPPORTED   # P not a multiple of 64
    assert wg(4, 128, 256, 0, FAKE, FAKE) == B.MOE_ERR_INVALID_ARG
    assert wg(4, 128, 256, 256, None, FAKE) == B.MOE_ERR_INVALID_ARG  # offsets required
    assert wg(4, 128, 256, 256, FAKE, None) == B.MOE_ERR_INVALID_ARG
    assert wg(4, 1 << 22, 256, 256, FAKE, FAKE) == B.MOE_ERR_UNSUPPORTED
    assert wg(1, 1, (1 << 24) + 64, 64, FAKE, FAKE) == B.MOE_ERR_UNSUPPORTED  # row offsets
    rneed = lib.moe_router_backward_workspace_size(ctypes.byref(d), 128)
    assert rneed >= (128 // 32 + 16) * 128 * 4
    rb = lambda dd, cap, off, wsb: lib.moe_router_backward(  # noqa: E731
        ctypes.byref(dd), cap, FAKE, off, FAKE, FAKE, FAKE, wsb, None)
    assert rb(d, 128, FAKE, rneed - 1) == B.MOE_ERR_WORKSPACE
    assert rb(d, 128, None, rneed) == B.MOE_ERR_INVALID_ARG
    assert rb(d, -1, FAKE, rneed) == B.MOE_ERR_INVALID_ARG
    ib = lambda dd, dxp, dl, wr: lib.moe_input_backward(  # noqa: E731
        ctypes.byref(dd), dxp, FAKE, FAKE, dl, wr, None, FAKE, FAKE, None)
    assert ib(d, None, FAKE, FAKE) == B.MOE_ERR_INVALID_ARG
    assert ib(d, FAKE, FAKE, None) == B.MOE_ERR_INVALID_ARG  # router term needs the weight
    bneed = lib.moe_backward_workspace_size(ctypes.byref(d))
    assert bneed > need
    lb = lambda dd, off, wsb, sgu=None, gs=None: lib.moe_layer_backward(  # noqa: E731
        ctypes.byref(dd), FAKE, FAKE, FAKE, FAKE, sgu, None, FAKE, FAKE, off, FAKE, FAKE, FAKE,
        gs, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, wsb, None)
    assert lb(d, FAKE, bneed - 1) == B.MOE_ERR_WORKSPACE
    assert lb(d, None, bneed) == B.MOE_ERR_INVALID_ARG
    assert lb(dplain, FAKE, bneed) == B.MOE_ERR_UNSUPPORTED
    dsh = _desc(I_shared=128)
    assert lb(dsh, FAKE, 1 << 40, FAKE) == B.MOE_ERR_INVALID_ARG   # shared gradients required
    assert lb(d32, FAKE, 1 << 40, None, FAKE) == B.MOE_ERR_UNSUPPORTED  # saved G|U: bf16 only
    # the training forward (saves G | U)
    fneed = lib.moe_ffn_workspace_size(ctypes.byref(d), 256, 128)
    ft = lambda dd, n, off, gs, wsb: lib.moe_expert_ffn_train(  # noqa: E731
        ctypes.byref(dd), n, 256, 128, FAKE, off, FAKE, FAKE, FAKE, gs, FAKE, wsb, None)
    assert ft(d, 4, FAKE, None, fneed) == B.MOE_ERR_INVALID_ARG
    assert ft(d, 4, None, FAKE, fneed) == B.MOE_ERR_INVALID_ARG    # several experts need offsets
    assert ft(d, 4, FAKE, FAKE, fneed - 1) == B.MOE_ERR_WORKSPACE
    assert ft(d32, 4, FAKE, FAKE, fneed) == B.MOE_ERR_UNSUPPORTED   # bf16 layers only
    assert ft(d, 0, FAKE, FAKE, fneed) == B.MOE_ERR_INVALID_ARG
    # no rows: nothing to do, no buffer needed
    assert lib.moe_expert_ffn_train(ctypes.byref(d), 4, 256, 0, None, FAKE, FAKE, FAKE, None,
                                    None, None, 0, None) == B.MOE_OK


def test_variant_checks(lib):
    d = _desc()
    rt = lambda dd, dt, x: lib.moe_route_typed(  # noqa: E731
        ctypes.byref(dd), dt, x, FAKE, None, None, None, FAKE, FAKE, None)
    assert rt(d, 3, FAKE) == B.MOE_ERR_INVALID_ARG        # not a router dtype
    assert rt(d, B.MOE_F16, None) == B.MOE_ERR_INVALID_ARG
    assert rt(_desc(dtype="f32", D=128), -1, FAKE) == B.MOE_ERR_INVALID_ARG
    need = lib.moe_ffn_workspace_size(ctypes.byref(d), 256, 128)
    fp = lambda dd, n, off, gu, wsb: lib.moe_expert_ffn_ptrs(  # noqa: E731
        ctypes.byref(dd), n, 256, 128, FAKE, off, gu, FAKE, FAKE, FAKE, wsb, None)
    assert fp(d, 4, FAKE, None, need) == B.MOE_ERR_INVALID_ARG
    assert fp(d, 4, None, FAKE, need) == B.MOE_ERR_INVALID_ARG   # several experts need offsets
    assert fp(d, 4, FAKE, FAKE, need - 1) == B.MOE_ERR_WORKSPACE
    assert fp(_desc(dtype="f32"), 4, FAKE, FAKE, need) == B.MOE_ERR_UNSUPPORTED


def test_layer_forward_checks(lib):
    d = _desc(I_shared=128)
    need = lib.moe_workspace_size(ctypes.byref(d))
    M = 64 * 2
    assert need >= M * (128 + 256 + 128) * 2 + 64 * (128 + 128) * 2
    call = lambda sgu, wsb: lib.moe_layer_forward(  # noqa: E731
        ctypes.byref(d), FAKE, FAKE, None, FAKE, FAKE, sgu, FAKE, FAKE, None, FAKE, FAKE, FAKE,
        FAKE, None, None, None, FAKE, wsb, None)
    assert call(None, need) == B.MOE_ERR_INVALID_ARG         # shared expert without weights
    assert call(FAKE, need - 1) == B.MOE_ERR_WORKSPACE
    d.E = 0
    assert lib.moe_workspace_size(ctypes.byref(d)) == 0


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, 42):
        assert isinstance(lib.moe_status_str(code), bytes)
    assert lib.moe_last_hip_error() == 0


def test_binding_refuses_host_tensors(lib):
    d = _desc(T=4, D=64)
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        moe.moe_route(d, x, torch.zeros(16, 64), None, None, None,
                      torch.zeros(4, 2, dtype=torch.int32), torch.zeros(4, 2))


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(ImportError):
        B.load_library(str(tmp_path / "libmoe.so"))
