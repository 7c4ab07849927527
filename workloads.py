"""Seeded synthetic inputs shared by the tests, the benchmark and the CPU baseline.

This module only draws random tensors and describes the workloads (shapes,
mask parameters, seeds).  It holds none of the method's arithmetic: no key sets,
no positions, no rotations, no attention.  Both the HIP path and the fp64 oracle
consume what it returns; neither is imported here.

Recipe (every workload): values come from ``torch.Generator('cpu')`` seeded
with ``1000*c`` for workload ``c`` and are drawn as fp32 ``torch.randn`` in the
order listed by each workload, then rounded to bf16 (round-to-nearest-even) for
the bf16 workloads.  Separator flags are i.i.d. Bernoulli(p) per position:
``torch.rand(m, generator=seed 1000*c+7) < p`` stored as uint8.  The pages
measure on tokenised text (LongBench, GSM8K-CoT, PG19 on Llama-2/3); these
seeded tensors take the same shapes and stand in for it.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import torch

SEPLLM, LAMBDA, SEGMENT = "sepllm", "lambda", "segment"


@dataclasses.dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    mode: str
    dtype: str          # "f32" | "bf16"
    batch: int
    h_q: int
    h_kv: int
    d: int
    n_q: int
    n_k: int
    a: int = 0          # SepLLM initial tokens
    w: int = 1          # SepLLM neighbour tokens
    p_sep: float = 0.0  # SepLLM separator density
    n_s: int = 0        # LM-Infinite starting span
    L: int = 0          # LM-Infinite pre-training length (distance cap)
    P: int = 0          # segment prefix length
    rope_base: Optional[float] = None
    alibi_exp: Optional[float] = None  # ALiBi slope exponent E (instead of RoPE)
    # segment workload extras
    n_local: int = 0    # heads 0..n_local-1 see the carried tail
    pool_len: int = 0   # detached retrieval pool length
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / (self.d ** 0.5)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


WORKLOADS: Dict[int, Workload] = {
    1: Workload(1, "sepllm_tiny_f32", SEPLLM, "f32", 1, 2, 2, 64, 512, 512,
                a=4, w=64, p_sep=0.1, rope_base=None, seed=1000),
    2: Workload(2, "sepllm_llama2_4k", SEPLLM, "bf16", 1, 32, 32, 128, 4096, 4096,
                a=4, w=256, p_sep=0.08, rope_base=10000.0, seed=2000),
    3: Workload(3, "lminfinite_lambda_32k", LAMBDA, "bf16", 1, 32, 32, 128, 32768, 32768,
                n_s=10, L=4096, rope_base=10000.0, seed=3000),
    4: Workload(4, "segment_s4096_p1024", SEGMENT, "bf16", 1, 32, 32, 128, 4096, 5120,
                P=1024, rope_base=10000.0, n_local=24, pool_len=32768, seed=4000),
    5: Workload(5, "sepllm_llama3_gqa_128k", SEPLLM, "bf16", 1, 32, 8, 128, 131072, 131072,
                a=4, w=1024, p_sep=0.06, rope_base=500000.0, seed=5000),
    # an ALiBi model (MPT-7B shape: 32 heads, head_dim 128, pre-trained on 2K tokens) under the
    # Lambda mask with its bias clipped at L_pretrain
    6: Workload(6, "lminfinite_alibi_lambda_32k", LAMBDA, "bf16", 1, 32, 32, 128, 32768, 32768,
                n_s=10, L=2048, alibi_exp=8.0, seed=6000),
    # a Pythia-160M-shaped layer (12 heads, head_dim 64) under the SepLLM training mask with
    # n = 64 neighbours, a batch of 8 sequences of 4096 tokens; RoPE over every dimension
    7: Workload(7, "sepllm_pythia_4k_d64", SEPLLM, "bf16", 8, 12, 12, 64, 4096, 4096,
                a=4, w=64, p_sep=0.08, rope_base=10000.0, seed=7000),
}


def _randn(shape, g) -> torch.Tensor:
    return torch.randn(*shape, generator=g, dtype=torch.float32)


def sep_flags(m: int, p: float, seed: int) -> torch.Tensor:
    """i.i.d. Bernoulli(p) separator flags, uint8 [m]."""
    g = torch.Generator("cpu").manual_seed(seed)
    return (torch.rand(m, generator=g) < p).to(torch.uint8)


def make_inputs(wl: Workload) -> Dict[str, torch.Tensor]:
    """CPU tensors for one workload, in its dtype.

    SepLLM / Lambda: q [B,h_q,m,d], k and v [B,h_kv,m,d] (+ sep [m] for SepLLM).
    Segment: q, k_seg, v_seg [B,h,S,d]; k_tail, v_tail [B,n_local,P,d];
    k_pool, v_pool [B,h-n_local,pool_len,d] (that draw order).
    """
    g = torch.Generator("cpu").manual_seed(wl.seed)
    dt = wl.torch_dtype
    B, d = wl.batch, wl.d
    out: Dict[str, torch.Tensor] = {}
    if wl.mode == SEGMENT:
        n_long = wl.h_q - wl.n_local
        shapes = [("q", (B, wl.h_q, wl.n_q, d)), ("k_seg", (B, wl.h_q, wl.n_q, d)),
                  ("v_seg", (B, wl.h_q, wl.n_q, d)), ("k_tail", (B, wl.n_local, wl.P, d)),
                  ("v_tail", (B, wl.n_local, wl.P, d)), ("k_pool", (B, n_long, wl.pool_len, d)),
                  ("v_pool", (B, n_long, wl.pool_len, d))]
        for name, shp in shapes:
            out[name] = _randn(shp, g).to(dt)
        return out
    out["q"] = _randn((B, wl.h_q, wl.n_q, d), g).to(dt)
    out["k"] = _randn((B, wl.h_kv, wl.n_k, d), g).to(dt)
    out["v"] = _randn((B, wl.h_kv, wl.n_k, d), g).to(dt)
    if wl.mode == SEPLLM:
        out["sep"] = sep_flags(wl.n_k, wl.p_sep, wl.seed + 7)
    return out


def small(mode: str, *, seed: int, dtype: str = "bf16", batch: int = 1, h_q: int = 2,
          h_kv: int = 2, d: int = 128, m: int = 300, a: int = 4, w: int = 64,
          p_sep: float = 0.1, n_s: int = 10, L: int = 100, P: int = 0,
          rope_base: Optional[float] = 10000.0, alibi_exp: Optional[float] = None) -> Workload:
    """A small workload for parity tests (several tiles plus a ragged tail)."""
    n_q = m
    n_k = m + P if mode == SEGMENT else m
    return Workload(0, f"small_{mode}_{seed}", mode, dtype, batch, h_q, h_kv, d, n_q, n_k,
                    a=a, w=w, p_sep=p_sep, n_s=n_s, L=L, P=P, rope_base=rope_base,
                    alibi_exp=alibi_exp, seed=seed)


def make_small_inputs(wl: Workload) -> Dict[str, torch.Tensor]:
    """q [B,h_q,n_q,d], k and v [B,h_kv,n_k,d] (+ sep [n_k] for SepLLM) for a small workload."""
    g = torch.Generator("cpu").manual_seed(wl.seed)
    dt = wl.torch_dtype
    out = {"q": _randn((wl.batch, wl.h_q, wl.n_q, wl.d), g).to(dt),
           "k": _randn((wl.batch, wl.h_kv, wl.n_k, wl.d), g).to(dt),
           "v": _randn((wl.batch, wl.h_kv, wl.n_k, wl.d), g).to(dt)}
    if wl.mode == SEPLLM:
        out["sep"] = sep_flags(wl.n_k, wl.p_sep, wl.seed + 7)
    return out


def make_grad(shape, seed: int, dtype=torch.bfloat16) -> torch.Tensor:
    """An upstream gradient dO: fp32 torch.randn from its own seed, rounded to dtype."""
    g = torch.Generator("cpu").manual_seed(seed)
    return _randn(shape, g).to(dtype)


def make_segment_stream(n_heads: int, seg_len: int, d: int, n_segments: int, seed: int,
                        dtype=torch.bfloat16):
    """Raw q, k, v [1, n_heads, seg_len, d] for each of n_segments segments (drawn in that order)."""
    g = torch.Generator("cpu").manual_seed(seed)
    out = []
    for _ in range(n_segments):
        out.append(tuple(_randn((1, n_heads, seg_len, d), g).to(dtype) for _ in range(3)))
    return out


def make_decode_stream(batch: int, h_q: int, h_kv: int, d: int, n_steps: int, seed: int,
                       p_sep: float, dtype=torch.bfloat16):
    """Per-step raw q [n, B, h_q, d], k, v [n, B, h_kv, d] (fp32 randn in that order, rounded to
    dtype) and i.i.d. Bernoulli(p_sep) separator flags uint8 [n, B] from seed + 7."""
    g = torch.Generator("cpu").manual_seed(seed)
    q = _randn((n_steps, batch, h_q, d), g).to(dtype)
    k = _randn((n_steps, batch, h_kv, d), g).to(dtype)
    v = _randn((n_steps, batch, h_kv, d), g).to(dtype)
    gf = torch.Generator("cpu").manual_seed(seed + 7)
    flags = (torch.rand((n_steps, batch), generator=gf) < p_sep).to(torch.uint8)
    return q, k, v, flags


def make_pool_inputs(n_heads: int, pool_len: int, d: int, seed: int, dtype=torch.bfloat16):
    """Scoring queries [n_heads,d] and pool keys/values [n_heads,pool_len,d] for top-k tests."""
    g = torch.Generator("cpu").manual_seed(seed)
    q = _randn((n_heads, d), g).to(dtype)
    k = _randn((n_heads, pool_len, d), g).to(dtype)
    v = _randn((n_heads, pool_len, d), g).to(dtype)
    return q, k, v
