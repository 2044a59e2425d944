"""Device-buffer owners around the C entry points.

``LayerForward`` allocates the outputs and workspace of ``moe_layer_forward``
once and calls it: the whole layer on one GPU (every expert local). With
``packed=True`` it first packs the expert weights (moe_pack_expert_weights)
into the layout the grouped GEMMs feed to the matrix cores, once.

``LayerForwardMXFP8`` is the same layer with the MXFP8 expert FFN
(include/moe_mxfp8.h): the expert weights are packed once at construction;
a call routes (fp32 router), permutes the bf16 rows, quantizes them, runs the
MXFP8 grouped FFN and combines in fp32 into the bf16 residual.

``LayerTrain`` runs the layer forward through the step entry points, keeping
what the backward needs (routing, offsets, positions, x_perm, y_perm and, with
``save_gu`` (bf16 layers), the fp32 gate and up pre-activations of the routed
and shared experts from ``moe_expert_ffn_train``), and its backward through
``moe_layer_backward`` (include/moe_backward.h): the input gradient and the
router, expert and shared-expert weight gradients. Without ``save_gu`` the
backward recomputes G | U: the same gradients, bit for bit, for
T top_k 2I 4 bytes less memory held between the two passes.

``EPRankShareForward`` runs the share of one expert-parallel rank out of
``ep_size`` logical ranks on this GPU, as a sequence of C calls (page "Expert
Parallel (EP)", Communication Pattern; page "Worked Example", Steps 1-5):
  1. moe_route on the rank's own tokens;
  2. moe_permute of the own tokens over all experts ("send" order, with the
     split sizes each rank would receive);
  3. moe_permute over every logical rank's tokens, keeping the pairs whose
     expert is local ("receive" buffer; on a real cluster these rows arrive
     through the all-to-all);
  4. moe_expert_ffn for the local experts;
  5. moe_expert_ffn for the shared expert on the own tokens (if any); with
     ``overlap_shared=True`` (opt-in, off by default) on a second stream
     forked at the start of the step and joined before step 6 (torchtitan
     issue 5554: independent shared experts overlap the routed path and join
     before the combination), else on the step's stream after step 4;
  6. moe_unpermute_combine over every source token: each gets the weighted
     sum of its local slots (the part this rank would send back), and the own
     tokens also get the residual and the shared expert's output.
The other ranks' routing is computed once by ``setup`` (their own routers
would produce it). Torch provides only device memory, streams and events.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _binding as B


def _layer_desc(desc: B.moe_desc, packed: bool, y_fp16: bool) -> B.moe_desc:
    d = B.moe_desc.from_buffer_copy(desc)
    if packed:
        d.weight_layout = B.MOE_WEIGHTS_PACKED
    d.expert_out_dtype = B.MOE_F16 if y_fp16 else B.MOE_F32
    return d


class LayerForward:
    """packed=True: the expert weights (routed and shared) are packed once here
    (moe_pack_expert_weights) and every call reads the packed copies.
    y_fp16: the layer keeps its expert outputs (y_perm, the shared expert's
    output; workspace-internal) in fp16; default on for bf16 layers."""

    def __init__(self, desc: B.moe_desc, w_router, w_gate_up, w_down, logit_bias=None,
                 shared_gate_up=None, shared_down=None, want_logits=False, device="cuda",
                 packed=False, y_fp16=None):
        if y_fp16 is None:
            y_fp16 = desc.act_dtype == B.MOE_BF16
        desc = _layer_desc(desc, packed, y_fp16)
        if packed:
            w_gate_up, w_down = B.pack_expert_weights(desc, w_gate_up, w_down)
            if shared_gate_up is not None:
                shared_gate_up, shared_down = B.pack_expert_weights(desc, shared_gate_up,
                                                                    shared_down)
        self.d = desc
        T, D, E, k = desc.T, desc.D, desc.E, desc.top_k
        dt = torch.bfloat16 if desc.act_dtype == B.MOE_BF16 else torch.float32
        self.w = dict(w_router=w_router, logit_bias=logit_bias, w_gate_up=w_gate_up,
                      w_down=w_down, shared_gate_up=shared_gate_up, shared_down=shared_down)
        self.out = torch.empty(T, D, dtype=dt, device=device)
        self.logits = torch.empty(T, E, dtype=torch.float32, device=device) if want_logits else None
        self.topk_idx = torch.empty(T, k, dtype=torch.int32, device=device)
        self.topk_w = torch.empty(T, k, dtype=torch.float32, device=device)
        self.counts = torch.empty(E, dtype=torch.int32, device=device)
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device=device)
        self.split = torch.empty(desc.ep_size, dtype=torch.int32, device=device)
        self.perm_src = torch.empty(max(T * k, 1), dtype=torch.int32, device=device)
        self.pos = torch.empty(T, k, dtype=torch.int32, device=device)
        self.ws = B.workspace(B.moe_workspace_size(desc), device)

    def __call__(self, x, stream=None):
        w = self.w
        B.moe_layer_forward(self.d, x, w["w_router"], w["logit_bias"], w["w_gate_up"],
                            w["w_down"], w["shared_gate_up"], w["shared_down"], self.out,
                            self.logits, self.topk_idx, self.topk_w, self.counts, self.offsets,
                            self.split, self.perm_src, self.pos, self.ws, stream)
        return self.out


class LayerTrain:
    def __init__(self, desc: B.moe_desc, w_router, w_gate_up, w_down, logit_bias=None,
                 shared_gate_up=None, shared_down=None, device="cuda", save_gu=None):
        self.d = desc
        T, D, E, k, I, Is = desc.T, desc.D, desc.E, desc.top_k, desc.I, desc.I_shared
        M = T * k
        # bf: the activation dtype (bf16, or fp32 for fp32 layers)
        f32, i32 = torch.float32, torch.int32
        bf = torch.bfloat16 if desc.act_dtype == B.MOE_BF16 else torch.float32
        self.w = dict(w_router=w_router, logit_bias=logit_bias, w_gate_up=w_gate_up,
                      w_down=w_down, shared_gate_up=shared_gate_up, shared_down=shared_down)
        self.out = torch.empty(T, D, dtype=bf, device=device)
        self.topk_idx = torch.empty(T, k, dtype=i32, device=device)
        self.topk_w = torch.empty(T, k, dtype=f32, device=device)
        self.counts = torch.empty(E, dtype=i32, device=device)
        self.offsets = torch.empty(E + 1, dtype=i32, device=device)
        self.split = torch.empty(desc.ep_size, dtype=i32, device=device)
        self.perm_src = torch.empty(max(M, 1), dtype=i32, device=device)
        self.pos = torch.empty(T, k, dtype=i32, device=device)
        self.x_perm = torch.empty(M, D, dtype=bf, device=device)
        self.y_perm = torch.empty(M, D, dtype=f32, device=device)
        self.shared_out = torch.empty(T, D, dtype=f32, device=device) if Is > 0 else None
        # fp32 G | U of the forward (bf16 layers only)
        if save_gu is None:
            save_gu = desc.act_dtype == B.MOE_BF16
        if save_gu and desc.act_dtype != B.MOE_BF16:
            raise ValueError("save_gu: bf16 layers only")
        self.gu = torch.empty(M, 2 * I, dtype=f32, device=device) if save_gu else None
        self.gu_sh = (torch.empty(T, 2 * Is, dtype=f32, device=device)
                      if save_gu and Is > 0 else None)
        self.ws_route = B.workspace(B.moe_route_workspace_size(desc), device)
        self.ws_perm = B.workspace(B.moe_permute_workspace_size(desc, 0, E), device)
        self.ws_ffn = B.workspace(B.moe_ffn_workspace_size(desc, I, M), device)
        self.ws_sh = B.workspace(B.moe_ffn_workspace_size(desc, Is, T), device) if Is > 0 else None
        # gradients
        self.dx = torch.empty(T, D, dtype=bf, device=device)
        self.dw_router = torch.empty(E, D, dtype=f32, device=device)
        self.dw_gate_up = torch.empty(E, D, 2 * I, dtype=f32, device=device)
        self.dw_down = torch.empty(E, I, D, dtype=f32, device=device)
        self.dw_shared_gate_up = torch.empty(D, 2 * Is, dtype=f32, device=device) if Is else None
        self.dw_shared_down = torch.empty(Is, D, dtype=f32, device=device) if Is else None
        self.ws_bwd = B.workspace(B.moe_backward_workspace_size(desc), device)
        self.x = None

    def forward(self, x, stream=None):
        d, w = self.d, self.w
        E, I, M = d.E, d.I, d.T * d.top_k
        self.x = x
        B.moe_route(d, x, w["w_router"], w["logit_bias"], None, None, self.topk_idx, self.topk_w,
                    ws=self.ws_route, stream=stream)
        B.moe_permute(d, x, self.topk_idx, 0, E, M, self.counts, self.offsets, self.split,
                      self.perm_src, self.pos, self.x_perm, self.ws_perm, stream)
        if self.gu is not None:
            B.moe_expert_ffn_train(d, E, I, M, self.x_perm, self.offsets, w["w_gate_up"],
                                   w["w_down"], self.y_perm, self.gu, self.ws_ffn, stream)
        else:
            B.moe_expert_ffn(d, E, I, M, self.x_perm, self.offsets, w["w_gate_up"], w["w_down"],
                             self.y_perm, self.ws_ffn, stream)
        if self.shared_out is not None:
            if self.gu_sh is not None:
                B.moe_expert_ffn_train(d, 1, d.I_shared, d.T, x, None, w["shared_gate_up"],
                                       w["shared_down"], self.shared_out, self.gu_sh, self.ws_sh,
                                       stream)
            else:
                B.moe_expert_ffn(d, 1, d.I_shared, d.T, x, None, w["shared_gate_up"],
                                 w["shared_down"], self.shared_out, self.ws_sh, stream)
        B.moe_unpermute_combine(d, self.y_perm, self.pos, self.topk_w, x, self.shared_out, 0, d.T,
                                self.out, stream)
        return self.out

    def backward(self, dout, stream=None):
        w = self.w
        B.moe_layer_backward(self.d, self.x, w["w_router"], w["w_gate_up"], w["w_down"],
                             w["shared_gate_up"], w["shared_down"], self.topk_idx, self.topk_w,
                             self.offsets, self.pos, self.x_perm, self.y_perm, dout, self.dx,
                             self.dw_router, self.dw_gate_up, self.dw_down,
                             self.dw_shared_gate_up, self.dw_shared_down, self.ws_bwd, stream,
                             gu_saved=self.gu, gu_shared_saved=self.gu_sh)
        return self.dx


class EPRankShareForward:
    def __init__(self, T: int, D: int, E: int, top_k: int, I: int, ep_size: int, ep_rank: int,
                 x_src, w_router, w_gate_up_local, w_down_local, logit_bias=None,
                 shared_gate_up=None, shared_down=None, I_shared: int = 0, dtype="bf16",
                 norm_topk=True, device="cuda", overlap_shared: bool = False,
                 packed: bool = False, y_fp16=None):
        R, r = ep_size, ep_rank
        if E % R:
            raise ValueError("E must be divisible by ep_size")
        self.T, self.D, self.E, self.k, self.I, self.R, self.r = T, D, E, top_k, I, R, r
        self.E_loc = E // R
        self.e_begin, self.e_end = r * self.E_loc, (r + 1) * self.E_loc
        self.Is = I_shared
        if y_fp16 is None:
            y_fp16 = dtype == "bf16"
        kw = dict(D=D, E=E, top_k=top_k, I=I, ep_size=R, ep_rank=r, dtype=dtype,
                  norm_topk=norm_topk, I_shared=I_shared, packed=packed, y_fp16=y_fp16)
        ydt = torch.float16 if y_fp16 else torch.float32
        self.d_own = B.make_desc(T=T, **kw)
        self.d_src = B.make_desc(T=T * R, **kw)
        if packed:
            w_gate_up_local, w_down_local = B.pack_expert_weights(self.d_own, w_gate_up_local,
                                                                  w_down_local)
            if shared_gate_up is not None:
                shared_gate_up, shared_down = B.pack_expert_weights(self.d_own, shared_gate_up,
                                                                    shared_down)
        dt = torch.bfloat16 if dtype == "bf16" else torch.float32
        dev = device
        self.x_src = x_src
        self.x_own = x_src[r * T:(r + 1) * T]
        self.w = dict(w_router=w_router, logit_bias=logit_bias, w_gate_up=w_gate_up_local,
                      w_down=w_down_local, shared_gate_up=shared_gate_up, shared_down=shared_down)
        Ts = T * R
        k = top_k
        # routing of every source token; rows [r*T, (r+1)*T) are this rank's own
        self.idx_src = torch.empty(Ts, k, dtype=torch.int32, device=dev)
        self.w_src = torch.empty(Ts, k, dtype=torch.float32, device=dev)
        self.idx_own = self.idx_src[r * T:(r + 1) * T]
        self.w_own = self.w_src[r * T:(r + 1) * T]
        # send-side permute of the own tokens over all experts
        self.send_counts = torch.empty(E, dtype=torch.int32, device=dev)
        self.send_offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
        self.send_split = torch.empty(R, dtype=torch.int32, device=dev)
        self.send_cap = T * k
        self.send_perm_src = torch.empty(max(self.send_cap, 1), dtype=torch.int32, device=dev)
        self.send_pos = torch.empty(T, k, dtype=torch.int32, device=dev)
        self.x_send = torch.empty(self.send_cap, D, dtype=dt, device=dev)
        self.route_ws = B.workspace(B.moe_route_workspace_size(self.d_own), dev)
        self.send_ws = B.workspace(B.moe_permute_workspace_size(self.d_own, 0, E), dev)
        # receive side: every source pair whose expert is local
        n = self.E_loc
        self.recv_cap = Ts * min(k, n)
        self.recv_counts = torch.empty(n, dtype=torch.int32, device=dev)
        self.recv_offsets = torch.empty(n + 1, dtype=torch.int32, device=dev)
        self.recv_split = torch.empty(R, dtype=torch.int32, device=dev)
        self.recv_perm_src = torch.empty(max(self.recv_cap, 1), dtype=torch.int32, device=dev)
        self.recv_pos = torch.empty(Ts, k, dtype=torch.int32, device=dev)
        self.x_recv = torch.empty(self.recv_cap, D, dtype=dt, device=dev)
        self.recv_ws = B.workspace(
            B.moe_permute_workspace_size(self.d_src, self.e_begin, self.e_end), dev)
        self.y_recv = torch.empty(self.recv_cap, D, dtype=ydt, device=dev)
        self.ffn_ws = B.workspace(B.moe_ffn_workspace_size(self.d_src, I, self.recv_cap), dev)
        if I_shared > 0:
            self.shared_out = torch.empty(T, D, dtype=ydt, device=dev)
            self.shared_ws = B.workspace(B.moe_ffn_workspace_size(self.d_own, I_shared, T), dev)
        else:
            self.shared_out = None
        # The shared expert depends only on the own tokens: it runs on a second
        # stream (default priority), forked at the start of the step and joined
        # before the combine (the overlap of the torchtitan shared-expert
        # issue, without the lower stream priority).
        self.aux = None
        if I_shared > 0 and overlap_shared:
            self.aux = torch.cuda.Stream(device=dev)
            self.ev_fork = torch.cuda.Event()
            self.ev_join = torch.cuda.Event()
        self.out_src = torch.empty(Ts, D, dtype=dt, device=dev)

    def setup(self, stream=None):
        """Route every other logical rank's tokens (their own routers' output)."""
        w = self.w
        for q in range(self.R):
            if q == self.r:
                continue
            sl = slice(q * self.T, (q + 1) * self.T)
            B.moe_route(self.d_own, self.x_src[sl], w["w_router"], w["logit_bias"], None, None,
                        self.idx_src[sl], self.w_src[sl], ws=self.route_ws, stream=stream)

    def __call__(self, logits: Optional[torch.Tensor] = None, stream=None):
        w = self.w
        if self.aux is not None:
            main = stream if isinstance(stream, torch.cuda.Stream) else (
                torch.cuda.current_stream(self.x_own.device) if stream is None
                else torch.cuda.ExternalStream(int(stream), device=self.x_own.device))
            self.ev_fork.record(main)
            self.aux.wait_event(self.ev_fork)
            B.moe_expert_ffn(self.d_own, 1, self.Is, self.T, self.x_own, None,
                             w["shared_gate_up"], w["shared_down"], self.shared_out,
                             self.shared_ws, self.aux)
            self.ev_join.record(self.aux)
        B.moe_route(self.d_own, self.x_own, w["w_router"], w["logit_bias"], logits, None,
                    self.idx_own, self.w_own, ws=self.route_ws, stream=stream)
        B.moe_permute(self.d_own, self.x_own, self.idx_own, 0, self.E, self.send_cap,
                      self.send_counts, self.send_offsets, self.send_split, self.send_perm_src,
                      self.send_pos, self.x_send, self.send_ws, stream)
        B.moe_permute(self.d_src, self.x_src, self.idx_src, self.e_begin, self.e_end,
                      self.recv_cap, self.recv_counts, self.recv_offsets, self.recv_split,
                      self.recv_perm_src, self.recv_pos, self.x_recv, self.recv_ws, stream)
        B.moe_expert_ffn(self.d_src, self.E_loc, self.I, self.recv_cap, self.x_recv,
                         self.recv_offsets, w["w_gate_up"], w["w_down"], self.y_recv, self.ffn_ws,
                         stream)
        if self.aux is not None:
            main.wait_event(self.ev_join)
        elif self.shared_out is not None:
            B.moe_expert_ffn(self.d_own, 1, self.Is, self.T, self.x_own, None,
                             w["shared_gate_up"], w["shared_down"], self.shared_out,
                             self.shared_ws, stream)
        B.moe_unpermute_combine(self.d_src, self.y_recv, self.recv_pos, self.w_src, self.x_own,
                                self.shared_out, self.r * self.T, self.T, self.out_src, stream)
        return self.out_src


class LayerForwardMXFP8:
    def __init__(self, desc: B.moe_desc, w_router, w_gate_up, w_down, logit_bias=None,
                 want_logits=False, device="cuda"):
        if desc.act_dtype != B.MOE_BF16 or desc.I_shared != 0:
            raise ValueError("the MXFP8 layer takes a bf16 layer without a shared expert")
        self.d = desc
        T, D, E, k, I = desc.T, desc.D, desc.E, desc.top_k, desc.I
        M = T * k
        u8 = torch.uint8
        self.w_router, self.logit_bias = w_router, logit_bias
        # weights packed once (quantized per output column along K, K contiguous)
        self.guq = torch.empty(E, 2 * I, D, dtype=u8, device=device)
        self.gus = torch.empty(E, 2 * I, D // 32, dtype=u8, device=device)
        self.dq = torch.empty(E, D, I, dtype=u8, device=device)
        self.ds = torch.empty(E, D, I // 32, dtype=u8, device=device)
        B.moe_mxfp8_pack_weights(w_gate_up, self.guq, self.gus)
        B.moe_mxfp8_pack_weights(w_down, self.dq, self.ds)
        self.out = torch.empty(T, D, dtype=torch.bfloat16, device=device)
        self.logits = torch.empty(T, E, dtype=torch.float32, device=device) if want_logits else None
        self.topk_idx = torch.empty(T, k, dtype=torch.int32, device=device)
        self.topk_w = torch.empty(T, k, dtype=torch.float32, device=device)
        self.counts = torch.empty(E, dtype=torch.int32, device=device)
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device=device)
        self.split = torch.empty(desc.ep_size, dtype=torch.int32, device=device)
        self.perm_src = torch.empty(max(M, 1), dtype=torch.int32, device=device)
        self.pos = torch.empty(T, k, dtype=torch.int32, device=device)
        self.x_perm = torch.empty(M, D, dtype=torch.bfloat16, device=device)
        self.xq = torch.empty(M, D, dtype=u8, device=device)
        self.xs = torch.empty(M, D // 32, dtype=u8, device=device)
        self.y_perm = torch.empty(M, D, dtype=torch.float32, device=device)
        self.ws_route = B.workspace(B.moe_route_workspace_size(desc), device)
        self.ws_perm = B.workspace(B.moe_permute_workspace_size(desc, 0, E), device)
        self.ws_ffn = B.workspace(B.moe_ffn_mxfp8_workspace_size(desc, I, M), device)

    def __call__(self, x, stream=None):
        d = self.d
        E, I, M = d.E, d.I, d.T * d.top_k
        B.moe_route(d, x, self.w_router, self.logit_bias, self.logits, None, self.topk_idx,
                    self.topk_w, ws=self.ws_route, stream=stream)
        B.moe_permute(d, x, self.topk_idx, 0, E, M, self.counts, self.offsets, self.split,
                      self.perm_src, self.pos, self.x_perm, self.ws_perm, stream)
        B.moe_mxfp8_quantize_rows(self.x_perm, self.xq, self.xs, stream)
        B.moe_expert_ffn_mxfp8(d, E, I, M, self.xq, self.xs, self.offsets, self.guq, self.gus,
                               self.dq, self.ds, self.y_perm, self.ws_ffn, stream)
        B.moe_unpermute_combine(d, self.y_perm, self.pos, self.topk_w, x, None, 0, d.T, self.out,
                                stream)
        return self.out

