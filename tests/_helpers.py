"""Shared test plumbing: workloads -> oracle specs and device tensors."""
import math

import numpy as np
import torch

import oracle as O
import workloads as W


def spec_of(wl, sep_np=None):
    return O.MaskSpec(wl.mode, wl.n_q, wl.n_k, a=wl.a, w=wl.w, sep=sep_np, n_s=wl.n_s, L=wl.L,
                      P=wl.P)


def device_mask(wl, sep=None):
    from structured_sparse_attention_attn_amd.pipeline import SparseAttention
    return SparseAttention(wl.mode, wl.n_q, wl.n_k, a=wl.a, w=wl.w, sep=sep, n_starting=wl.n_s,
                           L_pretrain=wl.L, prefix_len=wl.P)


def sample_rows(n_q, n_random, seed):
    """Every row of the first two and last two tiles plus n_random random rows."""
    r = np.random.default_rng(seed)
    edge = set(range(min(n_q, 256))) | set(range(max(0, n_q - 256), n_q))
    rnd = set(r.choice(n_q, size=min(n_random, n_q), replace=False).tolist())
    return np.array(sorted(edge | rnd))


def oracle_rows(Q, K, V, spec, rope_base, scale, heads, rows, kv_of=None):
    """Fast-mode oracle for the given heads and rows (rows grouped by tile)."""
    rows = np.asarray(rows)
    groups = {}
    for i in rows.tolist():
        groups.setdefault(i // 128, []).append(i)
    h_q, h_kv = Q.shape[0], K.shape[0]
    Os, Ls = [], []
    for h in heads:
        g = kv_of(h) if kv_of else h // (h_q // h_kv)
        o, l = O.attention_fast(Q[h], K[g], V[g], spec, rope_base, scale,
                                [np.array(v) for _, v in sorted(groups.items())])
        Os.append(o)
        Ls.append(l)
    return np.stack(Os), np.stack(Ls)


def compare(o_gpu, o_ref, lse_gpu, lse_ref, dtype):
    """Max-abs / mean-abs bars: bf16 1e-2 / 1e-3 on O; fp32 1e-5 on O.

    LSE bars (not stated by the target; derived): the logits see the bf16
    rounding of the rotated q and k (relative 2^-9 each) and of nothing else,
    so |d logit| <~ 2 * 2^-9 * scale * sum|q_c k_c|, a few 1e-3 for N(0,1)
    inputs; 2e-2 leaves margin.  fp32 keeps 1e-5.
    """
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    err = np.abs(o_gpu - o_ref)
    lerr = np.abs(np.asarray(lse_gpu, dtype=np.float64) - lse_ref)
    if dtype == "bf16":
        assert err.max() <= 1e-2, f"max-abs {err.max()}"
        assert err.mean() <= 1e-3, f"mean-abs {err.mean()}"
        assert lerr.max() <= 2e-2, f"lse max-abs {lerr.max()}"
    else:
        assert err.max() <= 1e-5, f"max-abs {err.max()}"
        assert lerr.max() <= 1e-5, f"lse max-abs {lerr.max()}"
    return float(err.max()), float(err.mean()), float(lerr.max())


def to64(t):
    return t.detach().to("cpu").double().numpy()


def log(msg):
    print(msg, flush=True)
