"""ctypes binding of libmoe (include/moe.h, include/moe_mxfp8.h,
include/moe_backward.h, include/moe_variants.h): one Python function per C entry
point, with the same name. Arguments are torch tensors (device memory) or
None; the binding checks their device, dtype, shape and contiguity, passes
their addresses and torch's current HIP stream, and raises MoeError on a
non-OK status. All arithmetic runs in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_CAPACITY = -4
MOE_ERR_HIP = -5

MOE_F32 = 0
MOE_BF16 = 1
MOE_F16 = 2  # router dtype only
MOE_MAX_EXPERTS = 1024
MOE_MAX_TOPK = 16
MOE_MAX_WIDTH = 262144

# Every symbol include/*.h declares.
EXPORTS = (
    "moe_route", "moe_route_workspace_size", "moe_permute", "moe_permute_workspace_size",
    "moe_expert_ffn",
    "moe_ffn_workspace_size", "moe_expert_gate_up", "moe_expert_down", "moe_down_workspace_size",
    "moe_gate_up_workspace_size",
    "moe_unpermute_combine", "moe_layer_forward", "moe_workspace_size", "moe_status_str",
    "moe_last_hip_error", "moe_ffn_tile_shape", "moe_pack_expert_weights",
    "moe_permute_noalloc",
    # MXFP8 variant of the expert FFN
    "moe_mxfp8_quantize_rows", "moe_mxfp8_pack_weights", "moe_expert_ffn_mxfp8",
    "moe_ffn_mxfp8_workspace_size", "moe_expert_gate_up_mxfp8", "moe_expert_down_mxfp8",
    # backward pass
    "moe_expert_ffn_train",
    "moe_combine_backward", "moe_expert_ffn_backward", "moe_ffn_backward_workspace_size",
    "moe_expert_gate_up_backward", "moe_expert_weight_grad",
    "moe_router_backward", "moe_router_backward_workspace_size", "moe_input_backward",
    "moe_layer_backward", "moe_backward_workspace_size",
    # interface variants
    "moe_route_typed", "moe_expert_ffn_ptrs",
)


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str, hip_error: int = 0):
        extra = f" (hipError {hip_error})" if status == MOE_ERR_HIP else ""
        super().__init__(f"{fn}: {msg}{extra} [status {status}]")
        self.status = status


MOE_WEIGHTS_STACKED = 0
MOE_WEIGHTS_PACKED = 1


class moe_desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("T", "D", "E", "top_k", "I", "ep_size", "ep_rank", "act_dtype",
                 "norm_topk", "I_shared", "weight_layout", "expert_out_dtype")]


def make_desc(T: int, D: int, E: int, top_k: int, I: int, ep_size: int = 1, ep_rank: int = 0,
              dtype: str = "bf16", norm_topk: bool = True, I_shared: int = 0,
              packed: bool = False, y_fp16: bool = False) -> moe_desc:
    """packed: expert weights (routed and shared) in the layout of
    moe_pack_expert_weights; y_fp16: expert outputs (y_perm, shared_out) in
    fp16 (both bf16 layers only)."""
    return moe_desc(T, D, E, top_k, I, ep_size, ep_rank,
                    MOE_BF16 if dtype == "bf16" else MOE_F32, int(bool(norm_topk)), I_shared,
                    MOE_WEIGHTS_PACKED if packed else MOE_WEIGHTS_STACKED,
                    MOE_F16 if y_fp16 else MOE_F32)


_P = ctypes.c_void_p
_D = ctypes.POINTER(moe_desc)
_SIGS = {
    "moe_route": (ctypes.c_int32, [_D, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_route_workspace_size": (ctypes.c_size_t, [_D]),
    "moe_permute": (ctypes.c_int32, [_D, _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                     _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_permute_workspace_size": (ctypes.c_size_t, [_D, ctypes.c_int32, ctypes.c_int32]),
    "moe_permute_noalloc": (ctypes.c_int32, [_D, _P, _P, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_int64, _P, _P, _P, _P, _P, _P, _P]),
    "moe_expert_ffn": (ctypes.c_int32, [_D, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                        _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_ffn_workspace_size": (ctypes.c_size_t, [_D, ctypes.c_int32, ctypes.c_int64]),
    "moe_expert_gate_up": (ctypes.c_int32, [_D, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                            _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_gate_up_workspace_size": (ctypes.c_size_t, [_D, ctypes.c_int32, ctypes.c_int64]),
    "moe_expert_down": (ctypes.c_int32, [_D, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                         _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_down_workspace_size": (ctypes.c_size_t, [_D, ctypes.c_int64]),
    "moe_pack_expert_weights": (ctypes.c_int32, [_D, ctypes.c_int32, ctypes.c_int32, _P, _P, _P,
                                                 _P, _P]),
    "moe_ffn_tile_shape": (ctypes.c_int32, [_D, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                            ctypes.c_int32, ctypes.c_int32,
                                            ctypes.POINTER(ctypes.c_int32),
                                            ctypes.POINTER(ctypes.c_int32)]),
    "moe_unpermute_combine": (ctypes.c_int32, [_D, _P, _P, _P, _P, _P, ctypes.c_int32,
                                               ctypes.c_int32, _P, _P]),
    "moe_layer_forward": (ctypes.c_int32, [_D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                           _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_workspace_size": (ctypes.c_size_t, [_D]),
    "moe_status_str": (ctypes.c_char_p, [ctypes.c_int32]),
    "moe_last_hip_error": (ctypes.c_int32, []),
    "moe_mxfp8_quantize_rows": (ctypes.c_int32, [ctypes.c_int64, ctypes.c_int32, _P, _P, _P, _P]),
    "moe_mxfp8_pack_weights": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                _P, _P, _P, _P]),
    "moe_expert_ffn_mxfp8": (ctypes.c_int32, [_D, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                              _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                              ctypes.c_size_t, _P]),
    "moe_ffn_mxfp8_workspace_size": (ctypes.c_size_t, [_D, ctypes.c_int32, ctypes.c_int64]),
    "moe_expert_gate_up_mxfp8": (ctypes.c_int32, [_D, ctypes.c_int32, ctypes.c_int32,
                                                  ctypes.c_int64, _P, _P, _P, _P, _P, _P, _P]),
    "moe_expert_down_mxfp8": (ctypes.c_int32, [_D, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_int64, _P, _P, _P, _P, _P, _P, _P]),
    "moe_combine_backward": (ctypes.c_int32, [_D, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_expert_ffn_train": (ctypes.c_int32, [_D, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                              _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_expert_ffn_backward": (ctypes.c_int32, [_D, ctypes.c_int32, ctypes.c_int32,
                                                 ctypes.c_int64, _P, _P, _P, _P, _P, _P, _P, _P,
                                                 _P, _P, ctypes.c_size_t, _P]),
    "moe_ffn_backward_workspace_size": (ctypes.c_size_t, [_D, ctypes.c_int32, ctypes.c_int64]),
    "moe_expert_gate_up_backward": (ctypes.c_int32, [_D, ctypes.c_int32, ctypes.c_int32,
                                                     ctypes.c_int64, _P, _P, _P, _P, _P, _P, _P]),
    "moe_expert_weight_grad": (ctypes.c_int32, [_D, ctypes.c_int32, ctypes.c_int64, _P,
                                                ctypes.c_int32, _P, ctypes.c_int32, _P, _P, _P]),
    "moe_router_backward": (ctypes.c_int32, [_D, ctypes.c_int64, _P, _P, _P, _P, _P,
                                             ctypes.c_size_t, _P]),
    "moe_router_backward_workspace_size": (ctypes.c_size_t, [_D, ctypes.c_int64]),
    "moe_input_backward": (ctypes.c_int32, [_D, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_layer_backward": (ctypes.c_int32, [_D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                            _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                            ctypes.c_size_t, _P]),
    "moe_backward_workspace_size": (ctypes.c_size_t, [_D]),
    "moe_route_typed": (ctypes.c_int32, [_D, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_expert_ffn_ptrs": (ctypes.c_int32, [_D, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                             _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
}

_lib: Optional[ctypes.CDLL] = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libmoe.so (built by mixture_experts_layer_fp32_amd.build).

    Raises if it is missing: there is no fallback implementation.
    """
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing: build it with "
                          "`python -m mixture_experts_layer_fp32_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != MOE_OK:
        lib = load_library()
        raise MoeError(fn, status, lib.moe_status_str(status).decode(),
                       lib.moe_last_hip_error())


def _act_dtype(d: moe_desc) -> torch.dtype:
    return torch.bfloat16 if d.act_dtype == MOE_BF16 else torch.float32


def _y_dtype(d: moe_desc) -> torch.dtype:
    """dtype of the expert outputs y_perm and shared_out."""
    return torch.float16 if d.expert_out_dtype == MOE_F16 else torch.float32


def _wd_dtype(d: moe_desc) -> torch.dtype:
    """dtype of down_proj: fp16 when packed (moe_pack_expert_weights converts
    it), else the activation dtype. Packed tensors keep the stacked shapes."""
    return torch.float16 if d.weight_layout == MOE_WEIGHTS_PACKED else _act_dtype(d)


def _ptr(t: Optional[torch.Tensor], name: str, dtype: Optional[torch.dtype] = None,
         shape=None, min_numel: Optional[int] = None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name}: {t.numel()} elements, need at least {min_numel}")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A device byte buffer of at least nbytes (at least 256 bytes)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------
# Entry points (same names as include/moe.h)
# ---------------------------------------------------------------------------
def moe_route_workspace_size(d: moe_desc) -> int:
    return int(load_library().moe_route_workspace_size(ctypes.byref(d)))


def moe_route(d: moe_desc, x, w_router, logit_bias, logits, probs, topk_idx, topk_w,
              ws=None, stream=None):
    """ws: a byte buffer of at least moe_route_workspace_size(d) bytes; when
    None, one is allocated here (through torch) for this call."""
    lib = load_library()
    T, D, E, k = d.T, d.D, d.E, d.top_k
    if ws is None:
        need = moe_route_workspace_size(d)
        if need > 0:
            ws = workspace(need, device=x.device if isinstance(x, torch.Tensor) else "cuda")
    args = (
        _ptr(x, "x", _act_dtype(d), (T, D)),
        _ptr(w_router, "w_router", torch.float32, (E, D)),
        _ptr(logit_bias, "logit_bias", torch.float32, (E,)),
        _ptr(logits, "logits", torch.float32, (T, E)),
        _ptr(probs, "probs", torch.float32, (T, E)),
        _ptr(topk_idx, "topk_idx", torch.int32, (T, k)),
        _ptr(topk_w, "topk_w", torch.float32, (T, k)),
        _ptr(ws, "ws", torch.uint8),
        ws.numel() if ws is not None else 0,
    )
    _check("moe_route", lib.moe_route(ctypes.byref(d), *args, _stream(stream)))


def moe_permute_workspace_size(d: moe_desc, e_begin: int, e_end: int) -> int:
    return int(load_library().moe_permute_workspace_size(ctypes.byref(d), e_begin, e_end))


def moe_permute(d: moe_desc, x, topk_idx, e_begin, e_end, cap_rows, counts, offsets, split,
                perm_src, pos, x_perm, ws, stream=None):
    lib = load_library()
    T, D, k = d.T, d.D, d.top_k
    n = e_end - e_begin
    args = (
        _ptr(x, "x", _act_dtype(d), (T, D)),
        _ptr(topk_idx, "topk_idx", torch.int32, (T, k)),
        int(e_begin), int(e_end), int(cap_rows),
        _ptr(counts, "counts", torch.int32, (n,)),
        _ptr(offsets, "offsets", torch.int32, (n + 1,)),
        _ptr(split, "split", torch.int32, (d.ep_size,)),
        _ptr(perm_src, "perm_src", torch.int32, min_numel=cap_rows),
        _ptr(pos, "pos", torch.int32, (T, k)),
        _ptr(x_perm, "x_perm", _act_dtype(d), min_numel=cap_rows * D),
        _ptr(ws, "ws", torch.uint8),
        ws.numel() if ws is not None else 0,
    )
    _check("moe_permute", lib.moe_permute(ctypes.byref(d), *args, _stream(stream)))


def moe_permute_noalloc(d: moe_desc, x, topk_idx, e_begin, e_end, cap_rows, counts, offsets,
                        split, perm_src, pos, x_perm, stream=None):
    """moe_permute with the library's own static scratch (no workspace)."""
    lib = load_library()
    T, D, k = d.T, d.D, d.top_k
    n = e_end - e_begin
    args = (
        _ptr(x, "x", _act_dtype(d), (T, D)),
        _ptr(topk_idx, "topk_idx", torch.int32, (T, k)),
        int(e_begin), int(e_end), int(cap_rows),
        _ptr(counts, "counts", torch.int32, (n,)),
        _ptr(offsets, "offsets", torch.int32, (n + 1,)),
        _ptr(split, "split", torch.int32, (d.ep_size,)),
        _ptr(perm_src, "perm_src", torch.int32, min_numel=cap_rows),
        _ptr(pos, "pos", torch.int32, (T, k)),
        _ptr(x_perm, "x_perm", _act_dtype(d), min_numel=cap_rows * D),
    )
    _check("moe_permute_noalloc", lib.moe_permute_noalloc(ctypes.byref(d), *args,
                                                          _stream(stream)))


def moe_ffn_workspace_size(d: moe_desc, inter: int, cap_rows: int) -> int:
    return int(load_library().moe_ffn_workspace_size(ctypes.byref(d), inter, cap_rows))


def moe_expert_ffn(d: moe_desc, n_experts, inter, cap_rows, x_perm, offsets, w_gate_up, w_down,
                   y_perm, ws, stream=None):
    lib = load_library()
    D = d.D
    dt = _act_dtype(d)
    args = (
        int(n_experts), int(inter), int(cap_rows),
        _ptr(x_perm, "x_perm", dt, min_numel=cap_rows * D),
        _ptr(offsets, "offsets", torch.int32, (n_experts + 1,)),
        _ptr(w_gate_up, "w_gate_up", dt, min_numel=n_experts * D * 2 * inter),
        _ptr(w_down, "w_down", _wd_dtype(d), min_numel=n_experts * inter * D),
        _ptr(y_perm, "y_perm", _y_dtype(d), min_numel=cap_rows * D),
        _ptr(ws, "ws", torch.uint8),
        ws.numel() if ws is not None else 0,
    )
    _check("moe_expert_ffn", lib.moe_expert_ffn(ctypes.byref(d), *args, _stream(stream)))


def _h_dtype(d: moe_desc) -> torch.dtype:
    return torch.float16 if d.act_dtype == MOE_BF16 else torch.float32


def moe_gate_up_workspace_size(d: moe_desc, inter: int, cap_rows: int) -> int:
    return int(load_library().moe_gate_up_workspace_size(ctypes.byref(d), inter, cap_rows))


def moe_expert_gate_up(d: moe_desc, n_experts, inter, cap_rows, x_perm, offsets, w_gate_up, h,
                       stream=None, ws=None):
    """ws None: whole tiles; a workspace of moe_gate_up_workspace_size bytes
    lets the last partial round of tiles run split along K (packed weights,
    as moe_expert_ffn)."""
    lib = load_library()
    D = d.D
    dt = _act_dtype(d)
    args = (
        int(n_experts), int(inter), int(cap_rows),
        _ptr(x_perm, "x_perm", dt, min_numel=cap_rows * D),
        _ptr(offsets, "offsets", torch.int32, (n_experts + 1,)),
        _ptr(w_gate_up, "w_gate_up", dt, min_numel=n_experts * D * 2 * inter),
        _ptr(h, "h", _h_dtype(d), min_numel=cap_rows * inter),
        _ptr(ws, "ws", torch.uint8),
        ws.numel() if ws is not None else 0,
    )
    _check("moe_expert_gate_up", lib.moe_expert_gate_up(ctypes.byref(d), *args, _stream(stream)))


def moe_down_workspace_size(d: moe_desc, cap_rows: int) -> int:
    return int(load_library().moe_down_workspace_size(ctypes.byref(d), cap_rows))


def moe_expert_down(d: moe_desc, n_experts, inter, cap_rows, h, offsets, w_down, y_perm,
                    stream=None, ws=None):
    """ws None: whole tiles; a workspace of moe_down_workspace_size bytes lets
    the last partial round of tiles run split along K (as moe_expert_ffn)."""
    lib = load_library()
    D = d.D
    args = (
        int(n_experts), int(inter), int(cap_rows),
        _ptr(h, "h", _h_dtype(d), min_numel=cap_rows * inter),
        _ptr(offsets, "offsets", torch.int32, (n_experts + 1,)),
        _ptr(w_down, "w_down", _wd_dtype(d), min_numel=n_experts * inter * D),
        _ptr(y_perm, "y_perm", _y_dtype(d), min_numel=cap_rows * D),
        _ptr(ws, "ws", torch.uint8),
        ws.numel() if ws is not None else 0,
    )
    _check("moe_expert_down", lib.moe_expert_down(ctypes.byref(d), *args, _stream(stream)))


def moe_pack_expert_weights(d: moe_desc, n_experts, inter, w_gate_up, w_down, packed_gate_up,
                            packed_down, stream=None):
    """Stacked bf16 gate_up_proj [n, D, 2 inter] / down_proj [n, inter, D]
    -> the packed layout (same shapes; packed_down is fp16). Either pair may
    be None."""
    lib = load_library()
    D = d.D
    bf = torch.bfloat16
    args = (
        _ptr(w_gate_up, "w_gate_up", bf, min_numel=n_experts * D * 2 * inter),
        _ptr(w_down, "w_down", bf, min_numel=n_experts * inter * D),
        _ptr(packed_gate_up, "packed_gate_up", bf, min_numel=n_experts * D * 2 * inter),
        _ptr(packed_down, "packed_down", torch.float16, min_numel=n_experts * inter * D),
    )
    _check("moe_pack_expert_weights",
           lib.moe_pack_expert_weights(ctypes.byref(d), int(n_experts), int(inter), *args,
                                       _stream(stream)))


def pack_expert_weights(d: moe_desc, w_gate_up, w_down, inter=None):
    """Packed copies (new tensors) of stacked expert weights: w_gate_up
    [n, D, 2I] or [D, 2I] (one expert), w_down [n, I, D] or [I, D]."""
    one = w_gate_up.dim() == 2
    gu = w_gate_up.unsqueeze(0) if one else w_gate_up
    dn = w_down.unsqueeze(0) if one else w_down
    n = gu.shape[0]
    inter = gu.shape[2] // 2 if inter is None else inter
    pgu = torch.empty_like(gu)
    pdn = torch.empty(dn.shape, dtype=torch.float16, device=dn.device)
    moe_pack_expert_weights(d, n, inter, gu, dn, pgu, pdn)
    return (pgu[0], pdn[0]) if one else (pgu, pdn)


def moe_ffn_tile_shape(d: moe_desc, n_experts, inter, cap_rows, has_offsets, gemm):
    """(rows, product columns) of the workgroup tile the grouped GEMMs take."""
    lib = load_library()
    r, c = ctypes.c_int32(0), ctypes.c_int32(0)
    _check("moe_ffn_tile_shape",
           lib.moe_ffn_tile_shape(ctypes.byref(d), n_experts, inter, cap_rows,
                                  int(bool(has_offsets)), gemm, ctypes.byref(r), ctypes.byref(c)))
    return r.value, c.value


def moe_unpermute_combine(d: moe_desc, y_perm, pos, topk_w, residual, shared_out, res_begin,
                          res_rows, out, stream=None):
    lib = load_library()
    T, D, k = d.T, d.D, d.top_k
    dt = _act_dtype(d)
    args = (
        _ptr(y_perm, "y_perm", _y_dtype(d)),
        _ptr(pos, "pos", torch.int32, (T, k)),
        _ptr(topk_w, "topk_w", torch.float32, (T, k)),
        _ptr(residual, "residual", dt, (res_rows, D)),
        _ptr(shared_out, "shared_out", _y_dtype(d), (res_rows, D)),
        int(res_begin), int(res_rows),
        _ptr(out, "out", dt, (T, D)),
    )
    if y_perm is not None and y_perm.numel() % D:
        raise ValueError("y_perm: not a whole number of rows")
    _check("moe_unpermute_combine",
           lib.moe_unpermute_combine(ctypes.byref(d), *args, _stream(stream)))


def moe_workspace_size(d: moe_desc) -> int:
    return int(load_library().moe_workspace_size(ctypes.byref(d)))


def moe_layer_forward(d: moe_desc, x, w_router, logit_bias, w_gate_up, w_down, shared_gate_up,
                      shared_down, out, logits, topk_idx, topk_w, counts, offsets, split,
                      perm_src, pos, ws, stream=None):
    lib = load_library()
    T, D, E, k, I, Is = d.T, d.D, d.E, d.top_k, d.I, d.I_shared
    dt = _act_dtype(d)
    args = (
        _ptr(x, "x", dt, (T, D)),
        _ptr(w_router, "w_router", torch.float32, (E, D)),
        _ptr(logit_bias, "logit_bias", torch.float32, (E,)),
        _ptr(w_gate_up, "w_gate_up", dt, (E, D, 2 * I)),
        _ptr(w_down, "w_down", _wd_dtype(d), (E, I, D)),
        _ptr(shared_gate_up, "shared_gate_up", dt, (D, 2 * Is)),
        _ptr(shared_down, "shared_down", _wd_dtype(d), (Is, D)),
        _ptr(out, "out", dt, (T, D)),
        _ptr(logits, "logits", torch.float32, (T, E)),
        _ptr(topk_idx, "topk_idx", torch.int32, (T, k)),
        _ptr(topk_w, "topk_w", torch.float32, (T, k)),
        _ptr(counts, "counts", torch.int32, (E,)),
        _ptr(offsets, "offsets", torch.int32, (E + 1,)),
        _ptr(split, "split", torch.int32, (d.ep_size,)),
        _ptr(perm_src, "perm_src", torch.int32, min_numel=T * k),
        _ptr(pos, "pos", torch.int32, (T, k)),
        _ptr(ws, "ws", torch.uint8),
        ws.numel() if ws is not None else 0,
    )
    _check("moe_layer_forward", lib.moe_layer_forward(ctypes.byref(d), *args, _stream(stream)))


# ---------------------------------------------------------------------------
# MXFP8 variant (include/moe_mxfp8.h). Codes and scales are uint8 tensors.
# ---------------------------------------------------------------------------
def moe_mxfp8_quantize_rows(x, codes, scales, stream=None):
    """x [rows, K] bf16 -> codes [rows, K] uint8, scales [rows, K/32] uint8."""
    lib = load_library()
    if x.dim() != 2:
        raise ValueError("x: expected [rows, K]")
    rows, K = x.shape
    args = (
        _ptr(x, "x", torch.bfloat16),
        _ptr(codes, "codes", torch.uint8, (rows, K)),
        _ptr(scales, "scales", torch.uint8, (rows, K // 32)),
    )
    _check("moe_mxfp8_quantize_rows",
           lib.moe_mxfp8_quantize_rows(int(rows), int(K), *args, _stream(stream)))


def moe_mxfp8_pack_weights(w, codes, scales, stream=None):
    """w [n, K, N] bf16 -> codes [n, N, K] uint8, scales [n, N, K/32] uint8."""
    lib = load_library()
    if w.dim() != 3:
        raise ValueError("w: expected [n, K, N]")
    n, K, N = w.shape
    args = (
        _ptr(w, "w", torch.bfloat16),
        _ptr(codes, "codes", torch.uint8, (n, N, K)),
        _ptr(scales, "scales", torch.uint8, (n, N, K // 32)),
    )
    _check("moe_mxfp8_pack_weights",
           lib.moe_mxfp8_pack_weights(int(n), int(K), int(N), *args, _stream(stream)))


def moe_ffn_mxfp8_workspace_size(d: moe_desc, inter: int, cap_rows: int) -> int:
    return int(load_library().moe_ffn_mxfp8_workspace_size(ctypes.byref(d), inter, cap_rows))


def moe_expert_ffn_mxfp8(d: moe_desc, n_experts, inter, cap_rows, xq, xs, offsets, w_gu_q,
                         w_gu_s, w_d_q, w_d_s, y_perm, ws, stream=None):
    lib = load_library()
    D = d.D
    u8 = torch.uint8
    args = (
        _ptr(xq, "xq", u8, min_numel=cap_rows * D),
        _ptr(xs, "xs", u8, min_numel=cap_rows * D // 32),
        _ptr(offsets, "offsets", torch.int32, (n_experts + 1,)),
        _ptr(w_gu_q, "w_gu_q", u8, (n_experts, 2 * inter, D)),
        _ptr(w_gu_s, "w_gu_s", u8, (n_experts, 2 * inter, D // 32)),
        _ptr(w_d_q, "w_d_q", u8, (n_experts, D, inter)),
        _ptr(w_d_s, "w_d_s", u8, (n_experts, D, inter // 32)),
        _ptr(y_perm, "y_perm", torch.float32, min_numel=cap_rows * D),
        _ptr(ws, "ws", u8),
        ws.numel() if ws is not None else 0,
    )
    _check("moe_expert_ffn_mxfp8",
           lib.moe_expert_ffn_mxfp8(ctypes.byref(d), int(n_experts), int(inter), int(cap_rows),
                                    *args, _stream(stream)))


def moe_expert_gate_up_mxfp8(d: moe_desc, n_experts, inter, cap_rows, xq, xs, offsets, w_gu_q,
                             w_gu_s, h, stream=None):
    lib = load_library()
    D = d.D
    u8 = torch.uint8
    args = (
        _ptr(xq, "xq", u8, min_numel=cap_rows * D),
        _ptr(xs, "xs", u8, min_numel=cap_rows * D // 32),
        _ptr(offsets, "offsets", torch.int32, (n_experts + 1,)),
        _ptr(w_gu_q, "w_gu_q", u8, (n_experts, 2 * inter, D)),
        _ptr(w_gu_s, "w_gu_s", u8, (n_experts, 2 * inter, D // 32)),
        _ptr(h, "h", torch.bfloat16, min_numel=cap_rows * inter),
    )
    _check("moe_expert_gate_up_mxfp8",
           lib.moe_expert_gate_up_mxfp8(ctypes.byref(d), int(n_experts), int(inter),
                                        int(cap_rows), *args, _stream(stream)))


def moe_expert_down_mxfp8(d: moe_desc, n_experts, inter, cap_rows, hq, hs, offsets, w_d_q, w_d_s,
                          y_perm, stream=None):
    lib = load_library()
    D = d.D
    u8 = torch.uint8
    args = (
        _ptr(hq, "hq", u8, min_numel=cap_rows * inter),
        _ptr(hs, "hs", u8, min_numel=cap_rows * inter // 32),
        _ptr(offsets, "offsets", torch.int32, (n_experts + 1,)),
        _ptr(w_d_q, "w_d_q", u8, (n_experts, D, inter)),
        _ptr(w_d_s, "w_d_s", u8, (n_experts, D, inter // 32)),
        _ptr(y_perm, "y_perm", torch.float32, min_numel=cap_rows * D),
    )
    _check("moe_expert_down_mxfp8",
           lib.moe_expert_down_mxfp8(ctypes.byref(d), int(n_experts), int(inter), int(cap_rows),
                                     *args, _stream(stream)))


# ---------------------------------------------------------------------------
# Backward pass (include/moe_backward.h). Activations, dout and the bf16
# intermediates have the layer's activation dtype.
# ---------------------------------------------------------------------------
def moe_combine_backward(d: moe_desc, dout, y_perm, pos, topk_w, dy_perm, dtopk_w, dlogit,
                         dl_perm, stream=None):
    lib = load_library()
    T, D, k = d.T, d.D, d.top_k
    args = (
        _ptr(dout, "dout", _act_dtype(d), (T, D)),
        _ptr(y_perm, "y_perm", torch.float32),
        _ptr(pos, "pos", torch.int32, (T, k)),
        _ptr(topk_w, "topk_w", torch.float32, (T, k)),
        _ptr(dy_perm, "dy_perm", _act_dtype(d)),
        _ptr(dtopk_w, "dtopk_w", torch.float32, (T, k)),
        _ptr(dlogit, "dlogit", torch.float32, (T, k)),
        _ptr(dl_perm, "dl_perm", torch.float32),
    )
    for name, t in (("y_perm", y_perm), ("dy_perm", dy_perm)):
        if t is not None and t.numel() % D:
            raise ValueError(f"{name}: not a whole number of rows")
    if y_perm is not None and dy_perm is not None and dy_perm.numel() < y_perm.numel():
        raise ValueError("dy_perm: fewer rows than y_perm")
    _check("moe_combine_backward",
           lib.moe_combine_backward(ctypes.byref(d), *args, _stream(stream)))


def moe_ffn_backward_workspace_size(d: moe_desc, inter: int, cap_rows: int) -> int:
    return int(load_library().moe_ffn_backward_workspace_size(ctypes.byref(d), inter, cap_rows))


def moe_expert_ffn_train(d: moe_desc, n_experts, inter, cap_rows, x_perm, offsets, w_gate_up,
                         w_down, y_perm, gu_saved, ws, stream=None):
    lib = load_library()
    D = d.D
    dt = _act_dtype(d)
    args = (
        int(n_experts), int(inter), int(cap_rows),
        _ptr(x_perm, "x_perm", dt, min_numel=cap_rows * D),
        _ptr(offsets, "offsets", torch.int32, (n_experts + 1,)),
        _ptr(w_gate_up, "w_gate_up", dt, min_numel=n_experts * D * 2 * inter),
        _ptr(w_down, "w_down", dt, min_numel=n_experts * inter * D),
        _ptr(y_perm, "y_perm", torch.float32, min_numel=cap_rows * D),
        _ptr(gu_saved, "gu_saved", torch.float32, min_numel=cap_rows * 2 * inter),
        _ptr(ws, "ws", torch.uint8),
        ws.numel() if ws is not None else 0,
    )
    _check("moe_expert_ffn_train",
           lib.moe_expert_ffn_train(ctypes.byref(d), *args, _stream(stream)))


def moe_expert_ffn_backward(d: moe_desc, n_experts, inter, cap_rows, x_perm, offsets, w_gate_up,
                            w_down, dy_perm, dx_perm, dw_gate_up, dw_down, ws, stream=None,
                            gu_saved=None):
    lib = load_library()
    D = d.D
    bf = _act_dtype(d)
    args = (
        _ptr(x_perm, "x_perm", bf, min_numel=cap_rows * D),
        _ptr(offsets, "offsets", torch.int32, (n_experts + 1,)),
        _ptr(w_gate_up, "w_gate_up", bf, (n_experts, D, 2 * inter)),
        _ptr(w_down, "w_down", bf, (n_experts, inter, D)),
        _ptr(dy_perm, "dy_perm", bf, min_numel=cap_rows * D),
        _ptr(gu_saved, "gu_saved", torch.float32, min_numel=cap_rows * 2 * inter),
        _ptr(dx_perm, "dx_perm", torch.float32, min_numel=cap_rows * D),
        _ptr(dw_gate_up, "dw_gate_up", torch.float32, (n_experts, D, 2 * inter)),
        _ptr(dw_down, "dw_down", torch.float32, (n_experts, inter, D)),
        _ptr(ws, "ws", torch.uint8),
        ws.numel() if ws is not None else 0,
    )
    _check("moe_expert_ffn_backward",
           lib.moe_expert_ffn_backward(ctypes.byref(d), int(n_experts), int(inter),
                                       int(cap_rows), *args, _stream(stream)))


def moe_expert_gate_up_backward(d: moe_desc, n_experts, inter, cap_rows, x_perm, offsets,
                                w_gate_up, dh, dgu, h, stream=None):
    lib = load_library()
    D = d.D
    bf = _act_dtype(d)
    args = (
        _ptr(x_perm, "x_perm", bf, min_numel=cap_rows * D),
        _ptr(offsets, "offsets", torch.int32, (n_experts + 1,)),
        _ptr(w_gate_up, "w_gate_up", bf, (n_experts, D, 2 * inter)),
        _ptr(dh, "dh", torch.float32, min_numel=cap_rows * inter),
        _ptr(dgu, "dgu", bf, min_numel=cap_rows * 2 * inter),
        _ptr(h, "h", bf, min_numel=cap_rows * inter),
    )
    _check("moe_expert_gate_up_backward",
           lib.moe_expert_gate_up_backward(ctypes.byref(d), int(n_experts), int(inter),
                                           int(cap_rows), *args, _stream(stream)))


def moe_expert_weight_grad(d: moe_desc, n_experts, cap_rows, a, P, b, Q, offsets, c,
                           stream=None):
    lib = load_library()
    bf = _act_dtype(d)
    args = (
        _ptr(a, "a", bf, min_numel=cap_rows * P), int(P),
        _ptr(b, "b", bf, min_numel=cap_rows * Q), int(Q),
        _ptr(offsets, "offsets", torch.int32, (n_experts + 1,)),
        _ptr(c, "c", torch.float32, (n_experts, P, Q)),
    )
    _check("moe_expert_weight_grad",
           lib.moe_expert_weight_grad(ctypes.byref(d), int(n_experts), int(cap_rows), *args,
                                      _stream(stream)))


def moe_router_backward_workspace_size(d: moe_desc, cap_rows: int) -> int:
    return int(load_library().moe_router_backward_workspace_size(ctypes.byref(d), cap_rows))


def moe_router_backward(d: moe_desc, cap_rows, x_perm, offsets, dl_perm, dw_router, ws,
                        stream=None):
    lib = load_library()
    args = (
        _ptr(x_perm, "x_perm", _act_dtype(d), min_numel=cap_rows * d.D),
        _ptr(offsets, "offsets", torch.int32, (d.E + 1,)),
        _ptr(dl_perm, "dl_perm", torch.float32, min_numel=cap_rows),
        _ptr(dw_router, "dw_router", torch.float32, (d.E, d.D)),
        _ptr(ws, "ws", torch.uint8),
        ws.numel() if ws is not None else 0,
    )
    _check("moe_router_backward",
           lib.moe_router_backward(ctypes.byref(d), int(cap_rows), *args, _stream(stream)))


def moe_input_backward(d: moe_desc, dx_perm, pos, topk_idx, dlogit, w_router, dx_shared, dout,
                       dx, stream=None):
    lib = load_library()
    T, D, E, k = d.T, d.D, d.E, d.top_k
    args = (
        _ptr(dx_perm, "dx_perm", torch.float32),
        _ptr(pos, "pos", torch.int32, (T, k)),
        _ptr(topk_idx, "topk_idx", torch.int32, (T, k)),
        _ptr(dlogit, "dlogit", torch.float32, (T, k)),
        _ptr(w_router, "w_router", torch.float32, (E, D)),
        _ptr(dx_shared, "dx_shared", torch.float32, (T, D)),
        _ptr(dout, "dout", _act_dtype(d), (T, D)),
        _ptr(dx, "dx", _act_dtype(d), (T, D)),
    )
    if dx_perm is not None and dx_perm.numel() % D:
        raise ValueError("dx_perm: not a whole number of rows")
    _check("moe_input_backward", lib.moe_input_backward(ctypes.byref(d), *args, _stream(stream)))


def moe_backward_workspace_size(d: moe_desc) -> int:
    return int(load_library().moe_backward_workspace_size(ctypes.byref(d)))


def moe_layer_backward(d: moe_desc, x, w_router, w_gate_up, w_down, shared_gate_up, shared_down,
                       topk_idx, topk_w, offsets, pos, x_perm, y_perm, dout, dx, dw_router,
                       dw_gate_up, dw_down, dw_shared_gate_up, dw_shared_down, ws, stream=None,
                       gu_saved=None, gu_shared_saved=None):
    lib = load_library()
    T, D, E, k, I, Is = d.T, d.D, d.E, d.top_k, d.I, d.I_shared
    bf, f32 = _act_dtype(d), torch.float32
    M = T * k
    args = (
        _ptr(x, "x", bf, (T, D)),
        _ptr(w_router, "w_router", f32, (E, D)),
        _ptr(w_gate_up, "w_gate_up", bf, (E, D, 2 * I)),
        _ptr(w_down, "w_down", bf, (E, I, D)),
        _ptr(shared_gate_up, "shared_gate_up", bf, (D, 2 * Is)),
        _ptr(shared_down, "shared_down", bf, (Is, D)),
        _ptr(topk_idx, "topk_idx", torch.int32, (T, k)),
        _ptr(topk_w, "topk_w", f32, (T, k)),
        _ptr(offsets, "offsets", torch.int32, (E + 1,)),
        _ptr(pos, "pos", torch.int32, (T, k)),
        _ptr(x_perm, "x_perm", bf, min_numel=M * D),
        _ptr(y_perm, "y_perm", f32, min_numel=M * D),
        _ptr(gu_saved, "gu_saved", f32, min_numel=M * 2 * I),
        _ptr(gu_shared_saved, "gu_shared_saved", f32, (T, 2 * Is)),
        _ptr(dout, "dout", bf, (T, D)),
        _ptr(dx, "dx", bf, (T, D)),
        _ptr(dw_router, "dw_router", f32, (E, D)),
        _ptr(dw_gate_up, "dw_gate_up", f32, (E, D, 2 * I)),
        _ptr(dw_down, "dw_down", f32, (E, I, D)),
        _ptr(dw_shared_gate_up, "dw_shared_gate_up", f32, (D, 2 * Is)),
        _ptr(dw_shared_down, "dw_shared_down", f32, (Is, D)),
        _ptr(ws, "ws", torch.uint8),
        ws.numel() if ws is not None else 0,
    )
    _check("moe_layer_backward", lib.moe_layer_backward(ctypes.byref(d), *args, _stream(stream)))


# ---------------------------------------------------------------------------
# Interface variants (include/moe_variants.h).
# ---------------------------------------------------------------------------
_ROUTER_DTYPES = {"fp32": (MOE_F32, torch.float32), "bf16": (MOE_BF16, torch.bfloat16),
                  "fp16": (MOE_F16, torch.float16)}


def moe_route_typed(d: moe_desc, router_dtype: str, x, w_router, logit_bias, logits, probs,
                    topk_idx, topk_w, stream=None):
    """router_dtype 'fp32', 'bf16' or 'fp16': w_router [E, D] and logits
    [T, E] in that dtype."""
    lib = load_library()
    code, tdt = _ROUTER_DTYPES[router_dtype]
    T, D, E, k = d.T, d.D, d.E, d.top_k
    args = (
        _ptr(x, "x", _act_dtype(d), (T, D)),
        _ptr(w_router, "w_router", tdt, (E, D)),
        _ptr(logit_bias, "logit_bias", torch.float32, (E,)),
        _ptr(logits, "logits", tdt, (T, E)),
        _ptr(probs, "probs", torch.float32, (T, E)),
        _ptr(topk_idx, "topk_idx", torch.int32, (T, k)),
        _ptr(topk_w, "topk_w", torch.float32, (T, k)),
    )
    _check("moe_route_typed", lib.moe_route_typed(ctypes.byref(d), code, *args, _stream(stream)))


def pointer_array(tensors, device="cuda") -> torch.Tensor:
    """A device array of the tensors' addresses (for the *_ptrs entry points);
    the caller keeps the tensors alive while the array is in use."""
    return torch.tensor([t.data_ptr() for t in tensors], dtype=torch.int64, device=device)


def moe_expert_ffn_ptrs(d: moe_desc, n_experts, inter, cap_rows, x_perm, offsets, w_gate_up_list,
                        w_down_list, y_perm, ws, gu_ptrs=None, dn_ptrs=None, stream=None):
    """ModuleList-style experts: w_gate_up_list[j] [D, 2 inter] and
    w_down_list[j] [inter, D] (bf16), one tensor per expert. gu_ptrs / dn_ptrs
    may pass prebuilt pointer arrays (pointer_array) to skip building them."""
    lib = load_library()
    D = d.D
    bf = torch.bfloat16
    if len(w_gate_up_list) != n_experts or len(w_down_list) != n_experts:
        raise ValueError("one gate_up and one down tensor per expert")
    for j, (a, b) in enumerate(zip(w_gate_up_list, w_down_list)):
        _ptr(a, f"w_gate_up[{j}]", bf, (D, 2 * inter))
        _ptr(b, f"w_down[{j}]", _wd_dtype(d), (inter, D))
    gu = pointer_array(w_gate_up_list, x_perm.device) if gu_ptrs is None else gu_ptrs
    dn = pointer_array(w_down_list, x_perm.device) if dn_ptrs is None else dn_ptrs
    args = (
        _ptr(x_perm, "x_perm", bf, min_numel=cap_rows * D),
        _ptr(offsets, "offsets", torch.int32, (n_experts + 1,)),
        _ptr(gu, "w_gate_up_ptrs", torch.int64, (n_experts,)),
        _ptr(dn, "w_down_ptrs", torch.int64, (n_experts,)),
        _ptr(y_perm, "y_perm", _y_dtype(d), min_numel=cap_rows * D),
        _ptr(ws, "ws", torch.uint8),
        ws.numel() if ws is not None else 0,
    )
    _check("moe_expert_ffn_ptrs",
           lib.moe_expert_ffn_ptrs(ctypes.byref(d), int(n_experts), int(inter), int(cap_rows),
                                   *args, _stream(stream)))

