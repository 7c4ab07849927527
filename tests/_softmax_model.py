"""A float32 model of the bf16 forward kernel's online softmax (test support).

The kernel keeps, per query row, a reference m_ref (base-2) that is raised
only when needed: while some row of a 32-row wave has no finite reference,
every unit takes the exact row maximum; afterwards a unit's weights are
p = 2^(s - m_ref) straight from the matrix product, and only when some row's
weight sum of the unit passes 2^10 is the reference raised.  A unit whose
weights reach 2^64 (or overflow) is computed again and taken with its exact
row maximum.

This module replays that state machine on the CPU for the rows of one tile,
in the kernel's unit order (gathered separator chunks, the plan's blocks --
last to first under the ALiBi bias -- then LM-Infinite's capped passes), from
logits computed in fp64 from the pages' definitions (oracle primitives).  It
reports which branches the inputs reach and the LSE the update rule yields.
With ``old_rule=True`` it applies the earlier rule (no recomputation: the
rescale divides by the unit's largest weight whatever its size), which turns
a weight of +inf into NaN.  It models decisions and ranges, not the kernel's
bf16 rounding.
"""
from __future__ import annotations

import math

import numpy as np

import oracle as O

LOG2E = 1.0 / math.log(2.0)


def tile_units(spec: O.MaskSpec, plan, t: int, *, use_cap: bool, reverse: bool):
    """Units of tile t in the kernel's order: lists of (key index array, kind).

    kind is "sep" (gathered separators: visible to every row of the tile),
    "block" (the key-set predicate; with use_cap the capped pairs excluded) or
    "cap" (capped pairs only)."""
    it0, it1 = int(plan["tile_ptr"][t]), int(plan["tile_ptr"][t + 1])
    items = [int(x) for x in plan["items"][it0:it1]]
    units = []
    if spec.mode == O.SEPLLM and spec.sep is not None:
        nsep = int(plan["sep_count"][t])
        sep = plan["sep_idx"][:nsep]
        for c0 in range(0, nsep, O.BK):
            units.append((np.asarray(sep[c0:c0 + O.BK], dtype=np.int64), "sep"))
    capped = [x for x in items if use_cap and (x >> 24) & O.FLAG_CAPPED]
    ordinary = []
    for x in items:
        blk = x & 0xFFFFFF
        if use_cap and (x >> 24) & O.FLAG_CAPPED and blk * O.BK + O.BK - 1 < t * O.TQ - spec.L:
            continue  # every visible pair of this block is a capped one
        ordinary.append(blk)
    if reverse:
        ordinary = ordinary[::-1]
    for blk in ordinary:
        units.append((np.arange(blk * O.BK, min(spec.n_k, blk * O.BK + O.BK)), "block"))
    for x in capped:
        blk = x & 0xFFFFFF
        units.append((np.arange(blk * O.BK, min(spec.n_k, blk * O.BK + O.BK)), "cap"))
    return units


def unit_logits(q, k, spec, rows, keys, kind, rope_base, scale, slope, use_cap):
    """Base-2 logits [len(rows), len(keys)] of one unit (-inf where not visible)."""
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.int64)
    vis = O.visible(spec, rows[:, None], keys[None, :])
    if spec.mode == O.LAMBDA and use_cap:
        cap = O.capped(spec, rows[:, None], keys[None, :])
        vis = vis & (cap if kind == "cap" else ~cap)
    delta = (O.pos_q(spec, rows)[:, None] - O.pos_k(spec, keys)[None, :]).astype(np.float64)
    if spec.mode == O.LAMBDA:
        delta = np.minimum(delta, spec.L)
    if rope_base:
        th = O.rope_theta(q.shape[1], rope_base)
        S = np.empty((len(rows), len(keys)))
        for r, i in enumerate(rows.tolist()):
            qr = O.rotate(np.broadcast_to(q[i], (len(keys), q.shape[1])), delta[r][:, None] * th[None, :])
            S[r] = np.einsum("jd,jd->j", qr, k[keys])
    else:
        S = q[rows] @ k[keys].T
    S = S * scale
    if slope is not None:
        S = S - slope * delta
    return np.where(vis, S * LOG2E, -np.inf)


def replay_wave(unit_S, *, old_rule=False):
    """Replays one wave (rows of unit_S[u], 32 or fewer) through the update rule.

    unit_S: list over units of base-2 logits [rows, keys].  Returns a dict with
    the flags 'rescale' (the 2^10 branch ran), 'recompute' (the 2^64 branch ran),
    'overflow' (some weight was +inf) and the base-2 LSE per row (m_ref + log2 l)."""
    f32 = np.float32
    n = unit_S[0].shape[0]
    has_ref = np.zeros(n, dtype=bool)
    m_ref = np.zeros(n, dtype=f32)
    l_run = np.zeros(n, dtype=f32)
    flags = dict(rescale=False, recompute=False, overflow=False)
    with np.errstate(over="ignore", invalid="ignore"):
        for S in unit_S:
            s = (S - m_ref[:, None].astype(np.float64)).astype(f32)  # the product starts from -m_ref
            if not has_ref.all():
                mx = s.max(axis=1)
                delta = np.where(np.isneginf(mx), f32(0), np.where(has_ref, np.maximum(mx, f32(0)), mx))
                alpha = np.exp2(-delta)
                p = np.exp2(s - delta[:, None])
                l_run = l_run * alpha + p.sum(axis=1, dtype=f32)
                m_ref = m_ref + delta
                has_ref = has_ref | ~np.isneginf(mx)
                continue
            p = np.exp2(s)
            flags["overflow"] |= bool(np.isinf(p).any())
            psum = p.sum(axis=1, dtype=f32)
            if (psum > 1024).any():
                flags["rescale"] = True
                pm = p.max(axis=1)
                if not old_rule and not (pm < f32(2.0 ** 64)).all():
                    flags["recompute"] = True
                    mx = np.maximum(s.max(axis=1), f32(0))
                    alpha = np.exp2(-mx)
                    p = np.exp2(s - mx[:, None])
                    l_run = l_run * alpha
                    m_ref = m_ref + mx
                else:
                    up = pm > 1
                    f = np.where(up, f32(1) / pm, f32(1))
                    p = p * f[:, None]
                    l_run = l_run * f
                    m_ref = np.where(up, m_ref + np.log2(pm), m_ref)
                psum = p.sum(axis=1, dtype=f32)
            l_run = l_run + psum
    return dict(flags, lse2=m_ref.astype(np.float64) + np.log2(l_run.astype(np.float64)))


def replay(q, k, spec, rope_base, scale, *, slope=None, old_rule=False, tiles=None):
    """Replays every full 32-row wave of the listed tiles (default: all).

    q [n_q, d], k [n_k, d] fp64 (one head).  Returns (flags over all waves,
    {row: base-2 LSE})."""
    plan = O.plan(spec)
    use_cap = spec.mode == O.LAMBDA and bool(rope_base) and spec.n_s > 0
    reverse = slope is not None
    tiles = range(plan["n_tiles"]) if tiles is None else tiles
    flags = dict(rescale=False, recompute=False, overflow=False)
    lse = {}
    for t in tiles:
        units = tile_units(spec, plan, t, use_cap=use_cap, reverse=reverse)
        for w0 in range(t * O.TQ, min(spec.n_q, t * O.TQ + O.TQ), 32):
            rows = np.arange(w0, w0 + 32)
            if rows[-1] >= spec.n_q:
                continue  # a wave with rows past the end also holds rows the model does not follow
            S = [unit_logits(q, k, spec, rows, keys, kind, rope_base, scale, slope, use_cap)
                 for keys, kind in units]
            r = replay_wave(S, old_rule=old_rule)
            for key in flags:
                flags[key] |= r[key]
            for i, v in zip(rows.tolist(), r["lse2"].tolist()):
                lse[i] = v
    return flags, lse


# ----------------------------------------------------------------------------
# Inputs that reach the rare branches
# ----------------------------------------------------------------------------

def spike_queries(q, k, spec, rows, target, scale, *, rope_base=None, slope=None, h_q=1, h_kv=1):
    """q [B, h_q, n_q, d] with rows ``rows`` of every head replaced by a large
    query aimed at one visible key, so that this pair's logit is ``target``
    (natural units) while the row's other logits stay ordinary:

    * SepLLM / segment: the diagonal key (distance 0, no rotation);
    * LM-Infinite with RoPE: the first starting key seen at the capped
      distance (q = c R(-L) k_0, the logit being scale <R(L) q, k_0>);
    * LM-Infinite with the ALiBi bias: the first key (logit scale <q, k_0> - m L).

    q, k fp64 numpy; returns a new fp64 array."""
    q = np.array(q, dtype=np.float64, copy=True)
    group = h_q // h_kv
    for b in range(q.shape[0]):
        for h in range(h_q):
            kk = k[b, h // group]
            for i in rows:
                if spec.mode == O.LAMBDA:
                    kj = kk[0]
                    if rope_base:
                        th = O.rope_theta(kk.shape[1], rope_base)
                        dirn = O.rotate(kj, -float(spec.L) * th)
                        want = target
                    else:
                        dirn = kj
                        want = target + (slope(h) if slope else 0.0) * min(i, spec.L)
                else:
                    dirn = kk[O.pos_q(spec, i)]
                    want = target
                q[b, h, i] = dirn * (want / (scale * float(kj @ kj) if spec.mode == O.LAMBDA
                                             else scale * float(dirn @ dirn)))
    return q
