"""Seeded synthetic inputs for the MoE layer forward.

This module is shared by the HIP path's tests and benchmark and by the CPU
oracle's tests. It holds the workload table and the random draws only: none
of the layer's arithmetic (routing, permutation, expert FFN, combine) lives
here.

Recipe (the same for every workload):
  * one ``torch.Generator('cpu')`` seeded with ``seed`` (default 0);
  * draws, in this order: hidden states x ~ N(0, 1); router weight
    W_r ~ N(0, 0.02) of shape [E, D] (kept fp32); expert ``gate_up_proj``
    ~ N(0, 0.02) of shape [E_loc, D, 2I]; expert ``down_proj`` ~ N(0, 0.02)
    of shape [E_loc, I, D]; then, when the workload has a shared expert, its
    ``gate_up_proj`` [D, 2I_s] and ``down_proj`` [I_s, D]; then, when the
    workload has a Zipf routing bias, one ``randperm(E)``;
  * 0.02 is a standard deviation;
  * bf16 workloads draw in fp32 and round to bf16 with round-to-nearest-even;
    the router weight stays fp32 (the router runs in fp32).

Only the experts that this (logical) rank holds are drawn: [E_loc, ...] with
E_loc = E / ep_size for a rank-share workload, E_loc = E otherwise.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Dict, Optional

import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "scaled", "zipf_rank_bias"]


@dataclass(frozen=True)
class Workload:
    """Shape of one synthetic MoE layer workload.

    T        tokens routed by this (logical) rank
    D        hidden size
    E        routed experts (global)
    k        experts chosen per token
    I        expert intermediate size (gate_up_proj is [D, 2I])
    dtype    'f32' or 'bf16' for activations and expert weights
    ep_size  logical expert-parallel ranks (split sizes are reported over them)
    rank_share  True when this GPU runs one EP rank's share: it receives the
             pairs of all ep_size ranks' tokens whose expert is local
    ep_rank  the rank this GPU plays when rank_share is True
    I_shared intermediate size of the one shared expert (0 = none)
    zipf_s   when > 0, a per-expert routing bias zipf_s * log(1 / rank_e)
    return_logits  the router's fp32 logits are part of the output
    """

    name: str
    T: int
    D: int
    E: int
    k: int
    I: int
    dtype: str = "bf16"
    ep_size: int = 1
    rank_share: bool = False
    ep_rank: int = 0
    I_shared: int = 0
    zipf_s: float = 0.0
    return_logits: bool = False
    description: str = ""

    @property
    def E_loc(self) -> int:
        return self.E // self.ep_size if self.rank_share else self.E

    @property
    def T_src(self) -> int:
        """Tokens whose pairs can reach this GPU's experts."""
        return self.T * self.ep_size if self.rank_share else self.T

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_fp32", T=256, D=128, E=8, k=2, I=256, dtype="f32",
                 description="Tiny fp32 MoE layer, top-2 of 8 experts"),
        Workload("worked_example_geometry", T=4096, D=1024, E=16, k=2, I=2048,
                 ep_size=4,
                 description="16 experts as 4 logical ranks x 4 local experts, top-2"),
        Workload("mixtral_style", T=8192, D=4096, E=8, k=2, I=14336,
                 description="Mixtral-style layer, top-2 of 8 experts"),
        Workload("deepseek_v3_rank_share", T=4096, D=7168, E=256, k=8, I=2048,
                 ep_size=8, rank_share=True, ep_rank=0, I_shared=2048,
                 description="DeepSeek-V3-style EP rank share: 32 of 256 experts, "
                             "top-8, one shared expert"),
        Workload("skewed_fine_grained", T=16384, D=2048, E=128, k=8, I=768,
                 zipf_s=1.5, return_logits=True,
                 description="Fine-grained top-8 of 128 with a Zipf routing bias"),
    ]
}


def scaled(w: Workload, **changes) -> Workload:
    """A copy of ``w`` with some dimensions changed (for small test cases)."""
    return replace(w, **changes)


def zipf_rank_bias(E: int, s: float, g: torch.Generator) -> torch.Tensor:
    """Per-expert bias s*log(1/rank_e) over a random ranking of the experts.

    rank_e = 1 + position of expert e in one randperm(E) draw; natural log.
    """
    perm = torch.randperm(E, generator=g)
    rank = torch.empty(E, dtype=torch.float64)
    rank[perm] = torch.arange(1, E + 1, dtype=torch.float64)
    return (-s * torch.log(rank)).to(torch.float32)


def make_inputs(w: Workload, seed: int = 0) -> Dict[str, Optional[torch.Tensor]]:
    """Draw one workload's inputs on the CPU (contiguous tensors).

    Returns x [T_src, D], w_router [E, D] fp32, w_gate_up [E_loc, D, 2I],
    w_down [E_loc, I, D], shared_gate_up [D, 2I_s] | None,
    shared_down [I_s, D] | None, logit_bias [E] fp32 | None.
    For a rank-share workload, rank r's own tokens are rows [r*T, (r+1)*T).
    """
    g = torch.Generator(device="cpu").manual_seed(seed)
    dt = w.torch_dtype
    std = 0.02

    def draw(*shape, scale=1.0, keep_f32=False):
        t = torch.randn(*shape, generator=g, dtype=torch.float32)
        if scale != 1.0:
            t.mul_(scale)
        return t if keep_f32 or dt == torch.float32 else t.to(dt)

    x = draw(w.T_src, w.D)
    w_router = draw(w.E, w.D, scale=std, keep_f32=True)
    w_gate_up = draw(w.E_loc, w.D, 2 * w.I, scale=std)
    w_down = draw(w.E_loc, w.I, w.D, scale=std)
    shared_gate_up = shared_down = None
    if w.I_shared > 0:
        shared_gate_up = draw(w.D, 2 * w.I_shared, scale=std)
        shared_down = draw(w.I_shared, w.D, scale=std)
    logit_bias = zipf_rank_bias(w.E, w.zipf_s, g) if w.zipf_s > 0 else None
    return dict(x=x, w_router=w_router, w_gate_up=w_gate_up, w_down=w_down,
                shared_gate_up=shared_gate_up, shared_down=shared_down,
                logit_bias=logit_bias)


def expected_rows(w: Workload) -> int:
    """Upper bound on the (token, expert) pairs this GPU's experts receive."""
    if w.rank_share:
        return w.T_src * min(w.k, w.E_loc)
    return w.T * w.k


def ffn_flops(rows: int, D: int, I: int) -> float:
    """Multiply-add FLOPs of one SiLU-gated FFN over ``rows`` rows (2*3*D*I per row)."""
    return 6.0 * rows * D * I

