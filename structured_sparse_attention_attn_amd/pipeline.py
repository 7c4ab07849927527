"""Device-buffer plumbing around the C ABI: plan, workspace and output tensors.

Nothing here computes: it allocates torch device tensors and calls the
binding, so every step of the path runs in the library's kernels.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import (SA_MASK_LAMBDA, SA_MASK_SEGMENT, SA_MASK_SEPLLM, bwd_args, fwd_args, mask,
               sa_bwd_workspace_bytes, sa_decode_workspace_bytes, sa_fwd_workspace_bytes,
               sa_plan_bytes, sa_stream_layout, sa_stream_state_bytes, sa_topk_workspace_bytes,
               sa_plan_status, sparse_attn_bwd, sparse_attn_decode_step, sparse_attn_fwd, sparse_attn_plan,
               sparse_attn_segment_carry, sparse_attn_stream_reset, sparse_attn_topk_middle, stream_cfg,
               topk_retrieve)

KINDS = {"sepllm": SA_MASK_SEPLLM, "lambda": SA_MASK_LAMBDA, "segment": SA_MASK_SEGMENT}


class SparseAttention:
    """One mask (one sequence), its plan buffer and a reusable workspace."""

    def __init__(self, kind: str, n_q: int, n_k: int, *, a: int = 0, w: int = 1, sep=None,
                 n_starting: int = 0, L_pretrain: int = 0, prefix_len: int = 0,
                 sep_max: int = 0, device: str = "cuda"):
        self.sep = sep  # keeps the device flags alive while the mask points at them
        self.mask = mask(KINDS[kind], n_q, n_k, a=a, w=w, sep=sep, n_starting=n_starting,
                         L_pretrain=L_pretrain, prefix_len=prefix_len, sep_max=sep_max)
        self.plan = torch.empty(sa_plan_bytes(self.mask), dtype=torch.uint8, device=device)
        self.ws: Optional[torch.Tensor] = None
        self.bws: Optional[torch.Tensor] = None
        self.device = device

    def build_plan(self, check: bool = False) -> None:
        """Enqueue the plan; with `check`, wait for it and raise if the mask broke sep_max."""
        sparse_attn_plan(self.mask, self.plan)
        if check:
            sa_plan_status(self.plan)

    def args(self, q, k, v, o, lse=None, rope_base=None, scale=None, alibi_exp=None):
        return fwd_args(q, k, v, o, lse=lse, rope_base=rope_base, scale=scale,
                        alibi_exp=alibi_exp, mask=self.mask)

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

    def topk_middle(self, q, k, v, o, lse, k_mid, rope_base=None, scale=None):
        """Adds each query's k_mid largest-logit middle tokens (LAMBDA masks) to the
        forward's o and lse in place; returns the chosen indices and their base-2 logits."""
        B, h_q, n_q, _ = q.shape
        sel = torch.empty((B, h_q, n_q, k_mid), dtype=torch.int32, device=self.device)
        score = torch.empty((B, h_q, n_q, k_mid), dtype=torch.float32, device=self.device)
        sparse_attn_topk_middle(self.mask, self.args(q, k, v, o, lse, rope_base, scale), k_mid, sel, score)
        return sel, score

    def backward(self, q, k, v, o, lse, dout, rope_base=None, scale=None, alibi_exp=None,
                 dq=None, dk=None, dv=None):
        """Gradients (dq, dk, dv) of the forward that wrote o and lse."""
        dq = torch.empty_like(q) if dq is None else dq
        dk = torch.empty_like(k) if dk is None else dk
        dv = torch.empty_like(v) if dv is None else dv
        args = self.args(q, k, v, o, lse, rope_base, scale, alibi_exp)
        need = sa_bwd_workspace_bytes(self.mask, args)
        if self.bws is None or self.bws.numel() < need:
            self.bws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
        sparse_attn_bwd(self.mask, self.plan, args, bwd_args(dout, dq, dk, dv, q=q, k=k), self.bws)
        return dq, dk, dv


class TopK:
    """Workspace holder for topk_retrieve."""

    def __init__(self, n_heads: int, pool_len: int, device: str = "cuda"):
        self.ws = torch.empty(sa_topk_workspace_bytes(n_heads, pool_len), dtype=torch.uint8,
                              device=device)

    def __call__(self, q_score, pool_k, k, idx, score=None, pool_v=None, pref_k=None, pref_v=None):
        topk_retrieve(q_score, pool_k, k, idx, self.ws, score=score, pool_v=pool_v,
                      pref_k=pref_k, pref_v=pref_v)


class SegmentRunner:
    """Several segments of one layer end to end: (C_i, o_i) = F(x_i, C_{i-1}, R_{i-1})
    (segmented-execution page, overall framework and key designs 2-3).

    Heads 0..n_local-1 attend to [tail | segment], the tail being their latest
    M raw keys/values; the other heads attend to [prefix | segment], the prefix
    being the top-M rows of a detached pool of their earlier segments, scored
    by the previous segment's last raw query.  The first segment has no prefix.
    K/V live in two alternating buffers [1, H, M+S, d]: the caller writes the
    segment's raw K/V into the views seg_kv() returns (rows M..M+S-1), the
    prefix occupies rows M-P..M-1, and after the forward the carry and the
    retrieval fill the other buffer's prefix rows for the next segment.
    """

    def __init__(self, n_heads: int, n_local: int, d: int, seg_len: int, tail_len: int,
                 pool_cap: int, *, rope_base=None, scale=None, dtype=torch.bfloat16,
                 device: str = "cuda"):
        self.H, self.nl, self.d, self.S, self.M = n_heads, n_local, d, seg_len, tail_len
        self.n_long = n_heads - n_local
        self.rope_base, self.scale = rope_base, scale
        shape = (1, n_heads, tail_len + seg_len, d)
        self.bufs = [(torch.empty(shape, dtype=dtype, device=device),
                      torch.empty(shape, dtype=dtype, device=device)) for _ in range(2)]
        self.cur = 0
        self.P = 0
        self.pool_len = 0
        self.pool_k = self.pool_v = None
        self.topk = None
        if self.n_long:
            self.pool_k = torch.empty((self.n_long, pool_cap, d), dtype=dtype, device=device)
            self.pool_v = torch.empty_like(self.pool_k)
            self.topk = TopK(self.n_long, pool_cap, device=device)
        self.idx = None  # pool rows of the prefix the next segment's long heads read
        self._attn = {}
        self.device = device

    def reset(self) -> None:
        """Start a new sequence: no tail, empty pool (plans and buffers are kept)."""
        self.cur = 0
        self.P = 0
        self.pool_len = 0
        self.idx = None

    def seg_kv(self):
        """Views [1, H, S, d] of the current buffer receiving the segment's raw K and V."""
        k, v = self.bufs[self.cur]
        return k[:, :, self.M:], v[:, :, self.M:]

    def attention(self, P: int) -> SparseAttention:
        if P not in self._attn:
            sa = SparseAttention("segment", self.S, P + self.S, prefix_len=P, device=self.device)
            sa.build_plan()
            self._attn[P] = sa
        return self._attn[P]

    def step(self, q, o=None, lse=None):
        """Forward of one segment (q [1, H, S, d] raw), then the carry and the retrieval."""
        M, S, P, nl = self.M, self.S, self.P, self.nl
        k, v = self.bufs[self.cur]
        kc, vc = k[:, :, M - P:], v[:, :, M - P:]
        o = self.attention(P).forward(q, kc, vc, o=o, lse=lse, rope_base=self.rope_base,
                                      scale=self.scale)
        nk, nv = self.bufs[1 - self.cur]
        keep = min(M, P + S)
        sparse_attn_segment_carry(kc[0], vc[0], nl, P, S, M,
                                  nk[0, :nl, M - keep:M] if nl else None,
                                  nv[0, :nl, M - keep:M] if nl else None,
                                  self.pool_k, self.pool_v, self.pool_len)
        nxt = keep
        if self.n_long:
            self.pool_len += S
            ksel = min(M, self.pool_len)
            self.idx = torch.empty((self.n_long, ksel), dtype=torch.int32, device=self.device)
            self.topk(q[0, nl:, S - 1, :], self.pool_k[:, :self.pool_len], ksel, self.idx,
                      pool_v=self.pool_v[:, :self.pool_len], pref_k=nk[0, nl:, M - ksel:M],
                      pref_v=nv[0, nl:, M - ksel:M])
            assert nl == 0 or ksel == keep
            nxt = ksel
        self.cur ^= 1
        self.P = nxt
        return o


class StreamDecoder:
    """Streaming decode for a batch of sequences: one state buffer and one workspace, both
    device memory.  kind "sepllm": the generation-time cache (Initial, Separator, Local,
    Past) with (a, s, w, c); kind "lambda": LM-Infinite's starting span a = n_starting
    and window L_pretrain + 1 (s, w, c unused)."""

    def __init__(self, batch, h_q, h_kv, d, a, s=1, w=1, c=0, *, rope_base=None, scale=None,
                 kind: str = "sepllm", L_pretrain: int = 0, device: str = "cuda"):
        self.lam = kind == "lambda"
        self.cfg = stream_cfg(batch, h_q, h_kv, d, a, s, w, c, rope_base=rope_base, scale=scale,
                              kind=KINDS[kind], L_pretrain=L_pretrain)
        self.state = torch.empty(sa_stream_state_bytes(self.cfg), dtype=torch.uint8, device=device)
        self.ws = torch.empty(sa_decode_workspace_bytes(self.cfg), dtype=torch.uint8, device=device)
        self.layout = sa_stream_layout(self.cfg)
        self.reset()

    def reset(self) -> None:
        sparse_attn_stream_reset(self.cfg, self.state)

    def step(self, q, k, v, is_sep=None, o=None, lse=None):
        o = torch.empty_like(q) if o is None else o
        sparse_attn_decode_step(self.cfg, self.state, q, k, v, is_sep, o, self.ws, lse=lse)
        return o

    def held(self, b: int):
        """Token indices sequence b's cache holds (reads the state back; for inspection)."""
        c, a, s_, w = self.cfg.c, self.cfg.a, self.cfg.s, self.cfg.w
        if self.lam:
            s_, w = 0, self.cfg.L_pretrain + 1
            c = a + w
        P = c - a - s_ - w
        st = self.state.cpu()
        ctrl = st[self.layout[4]:self.layout[4] + self.cfg.batch * 32].view(torch.int32).view(-1, 8)[b]
        pos = st[self.layout[2]:self.layout[2] + self.cfg.batch * c * 4].view(torch.int32).view(-1, c)[b]
        n_init, n_sep, n_past, n_local = (int(ctrl[i]) for i in (1, 2, 4, 5))
        slots = (list(range(n_init)) + list(range(a, a + n_sep)) + list(range(a + s_, a + s_ + n_past))
                 + list(range(a + s_ + P, a + s_ + P + n_local)))
        return sorted(int(pos[x]) for x in slots)

