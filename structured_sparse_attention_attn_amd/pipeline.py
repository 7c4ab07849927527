"""Device-buffer plumbing around the C ABI: plan, workspace and output tensors.

Nothing here computes: it allocates torch device tensors and calls the
binding, so every step of the path runs in the library's kernels.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import (SA_MASK_LAMBDA, SA_MASK_SEGMENT, SA_MASK_SEPLLM, fwd_args, mask,
               sa_fwd_workspace_bytes, sa_plan_bytes, sa_topk_workspace_bytes,
               sparse_attn_fwd, sparse_attn_plan, topk_retrieve)

KINDS = {"sepllm": SA_MASK_SEPLLM, "lambda": SA_MASK_LAMBDA, "segment": SA_MASK_SEGMENT}


class SparseAttention:
    """One mask (one sequence), its plan buffer and a reusable workspace."""

    def __init__(self, kind: str, n_q: int, n_k: int, *, a: int = 0, w: int = 1, sep=None,
                 n_starting: int = 0, L_pretrain: int = 0, prefix_len: int = 0,
                 device: str = "cuda"):
        self.sep = sep  # keeps the device flags alive while the mask points at them
        self.mask = mask(KINDS[kind], n_q, n_k, a=a, w=w, sep=sep, n_starting=n_starting,
                         L_pretrain=L_pretrain, prefix_len=prefix_len)
        self.plan = torch.empty(sa_plan_bytes(self.mask), dtype=torch.uint8, device=device)
        self.ws: Optional[torch.Tensor] = None
        self.device = device

    def build_plan(self) -> None:
        sparse_attn_plan(self.mask, self.plan)

    def args(self, q, k, v, o, lse=None, rope_base=None, scale=None, alibi_exp=None):
        return fwd_args(q, k, v, o, lse=lse, rope_base=rope_base, scale=scale,
                        alibi_exp=alibi_exp)

    def ensure_workspace(self, args) -> None:
        need = sa_fwd_workspace_bytes(self.mask, args)
        if self.ws is None or self.ws.numel() < need:
            self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)

    def forward(self, q, k, v, o=None, lse=None, rope_base=None, scale=None, args=None,
                alibi_exp=None):
        if o is None:
            o = torch.empty_like(q)
        if args is None:
            args = self.args(q, k, v, o, lse, rope_base, scale, alibi_exp)
        self.ensure_workspace(args)
        sparse_attn_fwd(self.mask, self.plan, args, self.ws)
        return o


class TopK:
    """Workspace holder for topk_retrieve."""

    def __init__(self, n_heads: int, pool_len: int, device: str = "cuda"):
        self.ws = torch.empty(sa_topk_workspace_bytes(n_heads, pool_len), dtype=torch.uint8,
                              device=device)

    def __call__(self, q_score, pool_k, k, idx, score=None, pool_v=None, pref_k=None, pref_v=None):
        topk_retrieve(q_score, pool_k, k, idx, self.ws, score=score, pool_v=pool_v,
                      pref_k=pref_k, pref_v=pref_v)
