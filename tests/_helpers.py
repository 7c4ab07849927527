"""Shared test plumbing: workloads -> oracle specs and device tensors."""
import math

import numpy as np
import torch

import oracle as O
import workloads as W


def spec_of(wl, sep_np=None):
    return O.MaskSpec(wl.mode, wl.n_q, wl.n_k, a=wl.a, w=wl.w, sep=sep_np, n_s=wl.n_s, L=wl.L,
                      P=wl.P)


def device_mask(wl, sep=None, sep_max=0):
    from structured_sparse_attention_attn_amd.pipeline import SparseAttention
    return SparseAttention(wl.mode, wl.n_q, wl.n_k, a=wl.a, w=wl.w, sep=sep, n_starting=wl.n_s,
                           L_pretrain=wl.L, prefix_len=wl.P, sep_max=sep_max)


def sample_rows(n_q, n_random, seed):
    """Every row of the first two and last two tiles plus n_random random rows."""
    r = np.random.default_rng(seed)
    edge = set(range(min(n_q, 256))) | set(range(max(0, n_q - 256), n_q))
    rnd = set(r.choice(n_q, size=min(n_random, n_q), replace=False).tolist())
    return np.array(sorted(edge | rnd))


def oracle_rows(Q, K, V, spec, rope_base, scale, heads, rows, kv_of=None, slope_of=None):
    """Fast-mode oracle for the given heads and rows (rows grouped by tile).

    slope_of(h): the ALiBi slope of head h (None: no bias)."""
    rows = np.asarray(rows)
    groups = {}
    for i in rows.tolist():
        groups.setdefault(i // 128, []).append(i)
    h_q, h_kv = Q.shape[0], K.shape[0]
    Os, Ls = [], []
    for h in heads:
        g = kv_of(h) if kv_of else h // (h_q // h_kv)
        o, l = O.attention_fast(Q[h], K[g], V[g], spec, rope_base, scale,
                                [np.array(v) for _, v in sorted(groups.items())],
                                alibi=slope_of(h) if slope_of else None)
        Os.append(o)
        Ls.append(l)
    return np.stack(Os), np.stack(Ls)


def effective_keys(lse, lse2):
    """Participation ratio 1 / sum_j p_ij^2 of each row's softmax weights, from the oracle's
    LSE of the logits (lse) and of the doubled logits (lse2): sum_j p_j^2 = e^{lse2 - 2 lse}.
    Equals |A_i| for uniform weights."""
    return np.exp(2.0 * np.asarray(lse) - np.asarray(lse2))


def row_counts(spec, rows):
    """|A_i| for the listed rows (from the oracle's predicates)."""
    rows = np.asarray(rows)
    out = np.zeros(len(rows), dtype=np.int64)
    for s in range(0, len(rows), 128):
        out[s:s + 128] = O.mask_rows(spec, rows[s:s + 128]).sum(axis=1)
    return out


def bf16_half_ulp(x):
    """Half the spacing of bf16 numbers at |x| (8 significant bits): 2^(floor(log2|x|) - 8);
    the quantum of rounding a result to bf16."""
    ax = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return np.ldexp(1.0, (np.floor(np.log2(ax)) - 8).astype(np.int64))


def logit_bound(Q, K, spec, scale, rows, kv_of=None):
    """B_i = scale * |q_i| * max_{j in A_i} |k_j| per (head, row): bounds every logit of the row
    (rotations keep norms), so the bf16 rounding of the rotated q and k (relative 2^-9 each)
    moves a logit, and the LSE, by at most about 2^-8 * B_i.  Q [h_q, n_q, d], K [h_kv, n_k, d]."""
    rows = np.asarray(rows)
    h_q, h_kv = Q.shape[0], K.shape[0]
    M = np.zeros((h_q, len(rows)))
    for s in range(0, len(rows), 128):
        vis = O.mask_rows(spec, rows[s:s + 128])
        for h in range(h_q):
            g = kv_of(h) if kv_of else h // (h_q // h_kv)
            kn = np.linalg.norm(K[g], axis=1)
            M[h, s:s + 128] = np.where(vis, kn[None, :], 0.0).max(axis=1)
    return scale * np.linalg.norm(Q[:, rows], axis=2) * M


def compare(o_gpu, o_ref, lse_gpu, lse_ref, dtype, lse_tol=None):
    """Parity bars.

    fp32: max-abs 1e-5 on O and on the LSE (the stated bar).
    bf16: every element |o_gpu - o_ref| <= 1e-2 + half a bf16 ulp of |o_ref|, and
    mean-abs <= 1e-3 + the mean over elements of a quarter bf16 ulp of |o_ref|
    (the stated bar, max-abs 1e-2 and mean-abs 1e-3, read for a result that is
    itself delivered in bf16: rounding the exact value to bf16 alone moves an
    element by up to half an ulp, 0.0078 at |O| in [2, 4), and by a quarter ulp
    on average; on a 3-key decode cache that rounding alone is a mean-abs of 9e-4).
    LSE (no stated bar): the logits see only the bf16 rounding of the rotated q
    and k, a few 1e-3 for N(0,1) inputs; 2e-2, or the per-row ``lse_tol``
    (e.g. 2e-2 + 2^-8 * logit_bound) for inputs with a wider logit range.
    """
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    err = np.abs(o_gpu - o_ref)
    lerr = np.abs(np.asarray(lse_gpu, dtype=np.float64) - lse_ref)
    if dtype == "bf16":
        bar = 1e-2 + bf16_half_ulp(o_ref)
        worst = float((err - bar).max()) if err.size else 0.0
        assert worst <= 0.0, f"max-abs {err.max()} exceeds 1e-2 + half-ulp by {worst}"
        mean_bar = 1e-3 + 0.5 * float(bf16_half_ulp(o_ref).mean()) if err.size else 1e-3
        assert err.mean() <= mean_bar, f"mean-abs {err.mean()} > {mean_bar}"
        tol = 2e-2 if lse_tol is None else np.asarray(lse_tol)
        assert np.all(lerr <= tol), f"lse max-abs {lerr.max()}"
    else:
        assert err.max() <= 1e-5, f"max-abs {err.max()}"
        assert lerr.max() <= 1e-5, f"lse max-abs {lerr.max()}"
    return float(err.max()), float(err.mean()), float(lerr.max())


def to64(t):
    return t.detach().to("cpu").double().numpy()


def log(msg):
    print(msg, flush=True)
