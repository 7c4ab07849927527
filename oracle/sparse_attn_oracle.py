"""fp64 reference for structured sparse causal attention (test infrastructure only).

Sources, cited by page title and section:

* SepLLM page ("SepLLM: Accelerate Large Language Models by Compressing One
  Segment into One Separator"), part 五 item 2: the mask M keeps, for query i,
  the initial ``a`` tokens, the separators before i and the ``n`` neighbouring
  tokens; every other entry is set to -inf before the softmax.  Part 六 6.1:
  ``O = Softmax(Q K^T / sqrt(d_k), masked by M) V``.
* LM-Infinite page (NAACL 2024, hyper.ai summary), section 方法: the
  Lambda-shaped set ``A_i = {j<=i : j<n_starting} U {j<=i : i-j<=L_pretrain}``;
  the distance cap ``d'_ij = min(i-j, L_pretrain)`` inside the logit
  ``w(q_i, k_j, d'_ij)``; and its RoPE realisation (window keys rotated as
  usual; starting-span keys outside the window unrotated with the query
  rotated to the fixed distance L_pretrain); for ALiBi-style models, the
  linear distance bias clipped to the same cap, then the Lambda mask.
* Segmented-execution page ("Training-Inference Consistent Segmented Execution
  for Long-Context LLMs"), 方法详解 / 整体框架 and 关键设计: a segment attends
  causally to [prefix | segment]; prefix positions are re-indexed to 0..P-1 and
  the segment is shifted by P; the long-range heads' prefix is the top-k of a
  detached pool scored by the segment-end query (forward only).

Readings taken where the pages are silent or garbled:
rotate-half RoPE with ``theta_c = base**(-2c/d)``; SepLLM neighbours are
``0 <= i-j < w`` (the query itself included); "separator before i" includes
j = i; masked means -inf (the printed elementwise product with M is not taken
literally); the Lambda window keeps ``i-j <= L`` literally; softmax scale
``1/sqrt(d)`` everywhere; GQA head h reads kv head ``h // (h_q/h_kv)``; the
top-k score is the fp64 chain ``((0 + q0 k0) + q1 k1) + ...`` with ties to the
lower index, and the retrieved rows keep ascending pool order; the ALiBi
variant adds ``-m_h * d'_ij`` to the scaled logit (no rotation), with the
geometric head slopes ``m_h = 2**(-E (h+1) / h_q)`` (E = 8 is the usual
choice; the page names no slopes).

Everything is plain numpy in fp64; the only library primitives are matrix
products, sorting and elementwise transcendental functions.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np

SEPLLM, LAMBDA, SEGMENT = "sepllm", "lambda", "segment"
TQ = 128          # queries per plan tile
BK = 64           # keys per plan block
FLAG_FULL = 1     # every (i, j) of tile x block is visible
FLAG_CAPPED = 2   # some visible (i, j) of tile x block has i - j > L_pretrain

__all__ = [
    "SEPLLM", "LAMBDA", "SEGMENT", "TQ", "BK", "FLAG_FULL", "FLAG_CAPPED", "MaskSpec",
    "visible", "capped", "key_set", "pos_q", "pos_k", "mask_rows", "rope_theta", "rotate",
    "attention_rows", "attention_fast", "attention", "plan", "plan_items_of_tile",
    "topk_scores", "topk_select", "pair_counts", "pair_count_total", "q0_closed_form",
    "alibi_slope", "q0_alibi_closed_form", "segmented_run", "attention_grad_rows",
    "attention_backward", "attention_grad_keys_fast", "StreamCache", "stream_cache_tokens", "decode_attention",
    "middle_scores", "attention_topk_middle",
]


@dataclasses.dataclass
class MaskSpec:
    """The pages' mask parameters for one sequence (shared by all heads)."""
    mode: str
    n_q: int
    n_k: int
    a: int = 0                       # SepLLM: initial tokens
    w: int = 1                       # SepLLM: neighbouring tokens (0 <= i-j < w)
    sep: Optional[np.ndarray] = None  # SepLLM: uint8 flags [n_k]; None = no separators
    n_s: int = 0                     # LM-Infinite: n_starting
    L: int = 0                       # LM-Infinite: L_pretrain
    P: int = 0                       # segment: prefix length (n_k = P + n_q)

    def sep_flags(self) -> np.ndarray:
        if self.sep is None:
            return np.zeros(self.n_k, dtype=np.uint8)
        return np.asarray(self.sep, dtype=np.uint8)


# ----------------------------------------------------------------------------
# Key sets and positions
# ----------------------------------------------------------------------------

def visible(spec: MaskSpec, i, j) -> np.ndarray:
    """Element-wise membership ``j in A_i`` (arrays broadcast).

    SepLLM (part 五 item 2): ``j <= i and (j < a or i-j < w or sep[j])``.
    LM-Infinite (方法, Lambda mask): ``j <= i and (j < n_starting or i-j <= L)``.
    Segment (整体框架): the prefix is fully visible and the segment causal,
    i.e. ``j <= P + i`` over keys ``[prefix | segment]``.
    """
    i = np.asarray(i, dtype=np.int64)
    j = np.asarray(j, dtype=np.int64)
    inside = (i >= 0) & (i < spec.n_q) & (j >= 0) & (j < spec.n_k)
    if spec.mode == SEPLLM:
        flags = spec.sep_flags()
        sep_j = flags[np.clip(j, 0, spec.n_k - 1)] == 1
        return inside & (j <= i) & ((j < spec.a) | (i - j < spec.w) | sep_j)
    if spec.mode == LAMBDA:
        return inside & (j <= i) & ((j < spec.n_s) | (i - j <= spec.L))
    if spec.mode == SEGMENT:
        return inside & (j <= spec.P + i)
    raise ValueError(spec.mode)


def capped(spec: MaskSpec, i, j) -> np.ndarray:
    """Visible pairs whose distance is capped: ``i - j > L`` (LM-Infinite only)."""
    if spec.mode != LAMBDA:
        return np.zeros(np.broadcast(np.asarray(i), np.asarray(j)).shape, dtype=bool)
    i = np.asarray(i, dtype=np.int64)
    j = np.asarray(j, dtype=np.int64)
    return visible(spec, i, j) & (i - j > spec.L)


def key_set(spec: MaskSpec, i: int) -> np.ndarray:
    """Ascending key indices of ``A_i``, evaluated element by element."""
    return np.flatnonzero(visible(spec, i, np.arange(spec.n_k)))


def pos_q(spec: MaskSpec, i):
    """RoPE position of query i: i, or P + i for a segment (segment shifted by P)."""
    return np.asarray(i, dtype=np.int64) + (spec.P if spec.mode == SEGMENT else 0)


def pos_k(spec: MaskSpec, j):
    """RoPE position of key j: its index (prefix re-indexed to 0..P-1 in segment mode)."""
    return np.asarray(j, dtype=np.int64)


def mask_rows(spec: MaskSpec, rows: Sequence[int]) -> np.ndarray:
    """bool [len(rows), n_k]: the visible keys of each listed query."""
    rows = np.asarray(rows, dtype=np.int64)
    return visible(spec, rows[:, None], np.arange(spec.n_k)[None, :])


# ----------------------------------------------------------------------------
# Rotary position embedding (rotate-half pairing, fp64)
# ----------------------------------------------------------------------------

def rope_theta(d: int, base: float) -> np.ndarray:
    """Frequencies ``theta_c = base ** (-2c/d)`` for c = 0 .. d/2-1 (fp64)."""
    c = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * c / d)


def rotate(x: np.ndarray, angle: np.ndarray) -> np.ndarray:
    """Rotate each pair (x[c], x[c+d/2]) by ``angle[..., c]`` (counter-clockwise)."""
    h = x.shape[-1] // 2
    x1, x2 = x[..., :h], x[..., h:]
    cs, sn = np.cos(angle), np.sin(angle)
    return np.concatenate([x1 * cs - x2 * sn, x2 * cs + x1 * sn], axis=-1)


# ----------------------------------------------------------------------------
# Attention, definition mode: one query row at a time, relative rotation per pair
# ----------------------------------------------------------------------------

def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, rows: Sequence[int],
                   spec: MaskSpec, rope_base: Optional[float], scale: float,
                   alibi: Optional[float] = None):
    """Masked softmax attention for the listed query rows of one head.

    q [n_q, d], k and v [n_k, d] (fp64).  For every key j in A_i the logit is
    ``scale * <Rot(delta) q_i, k_j>`` with ``delta = pos_q(i) - pos_k(j)``
    (LM-Infinite: ``delta' = min(delta, L)``), i.e. the page's
    ``w(q_i, k_j, d'_ij)`` for RoPE.  With ``alibi`` = m (and no RoPE) the
    logit is ``scale * <q_i, k_j> - m * delta'`` instead: the ALiBi bias with
    its distance clipped to the same cap.  Masked keys take no part (-inf
    logit).  Returns O [len(rows), d] and the natural-log LSE [len(rows)].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d = q.shape[1]
    theta = rope_theta(d, rope_base) if rope_base else None
    O = np.zeros((len(rows), v.shape[1]))
    lse = np.zeros(len(rows))
    for r, i in enumerate(rows):
        A = key_set(spec, int(i))
        if theta is None:
            s = k[A] @ q[i]
        else:
            delta = pos_q(spec, int(i)) - pos_k(spec, A)
            if spec.mode == LAMBDA:
                delta = np.minimum(delta, spec.L)
            ang = delta.astype(np.float64)[:, None] * theta[None, :]
            qr = rotate(np.broadcast_to(q[i], (len(A), d)), ang)
            s = np.einsum("jd,jd->j", qr, k[A])
        s = s * scale
        if alibi is not None:
            dist = pos_q(spec, int(i)) - pos_k(spec, A)
            if spec.mode == LAMBDA:
                dist = np.minimum(dist, spec.L)
            s = s - alibi * dist.astype(np.float64)
        mu = s.max()
        e = np.exp(s - mu)
        z = e.sum()
        O[r] = (e @ v[A]) / z
        lse[r] = mu + math.log(z)
    return O, lse


# ----------------------------------------------------------------------------
# Attention, fast mode: absolute rotations, one query tile at a time
# ----------------------------------------------------------------------------

def attention_fast(q: np.ndarray, k: np.ndarray, v: np.ndarray, spec: MaskSpec,
                   rope_base: Optional[float], scale: float,
                   row_blocks: Optional[Sequence[Sequence[int]]] = None,
                   alibi: Optional[float] = None):
    """Same result as :func:`attention_rows`, computed tile-wise for speed.

    q and k are rotated once at their absolute positions, using
    ``<R(a) q, R(b) k> = <R(a-b) q, k>``; capped LM-Infinite pairs use the
    page's realisation ``<R(L) q_i, k_j>`` with the raw key.  Each block of
    query rows takes the union of its visible keys, a dense product, the mask
    (-inf), then the softmax.  ``row_blocks`` defaults to consecutive groups
    of 128 rows.  ``alibi`` adds the clipped distance bias as in
    :func:`attention_rows`.  Returns (O, LSE) for the rows covered, in order.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n_q, d = q.shape
    if row_blocks is None:
        row_blocks = [np.arange(s, min(n_q, s + TQ)) for s in range(0, n_q, TQ)]
    if rope_base:
        theta = rope_theta(d, rope_base)
        kr = rotate(k, pos_k(spec, np.arange(spec.n_k)).astype(np.float64)[:, None] * theta[None, :])
    outs, lses = [], []
    for rows in row_blocks:
        rows = np.asarray(rows, dtype=np.int64)
        M = mask_rows(spec, rows)
        U = np.flatnonzero(M.any(axis=0))
        Mu = M[:, U]
        if rope_base:
            qr = rotate(q[rows], pos_q(spec, rows).astype(np.float64)[:, None] * theta[None, :])
            S = qr @ kr[U].T
            if spec.mode == LAMBDA:
                C = capped(spec, rows[:, None], U[None, :])
                if C.any():
                    qcap = rotate(q[rows], float(spec.L) * theta[None, :])
                    S = np.where(C, qcap @ k[U].T, S)
        else:
            S = q[rows] @ k[U].T
        S = S * scale
        if alibi is not None:
            dist = pos_q(spec, rows)[:, None] - pos_k(spec, U)[None, :]
            if spec.mode == LAMBDA:
                dist = np.minimum(dist, spec.L)
            S = S - alibi * dist.astype(np.float64)
        S = np.where(Mu, S, -np.inf)
        mu = S.max(axis=1)
        E = np.exp(S - mu[:, None])
        z = E.sum(axis=1)
        outs.append((E @ v[U]) / z[:, None])
        lses.append(mu + np.log(z))
    return np.concatenate(outs, axis=0), np.concatenate(lses, axis=0)


def attention(Q, K, V, spec: MaskSpec, rope_base: Optional[float], scale: float,
              heads: Optional[Sequence[int]] = None, rows: Optional[Sequence[int]] = None,
              mode: str = "fast", alibi_exp: Optional[float] = None):
    """Multi-head wrapper: Q [h_q, n_q, d], K and V [h_kv, n_k, d] (batch squeezed).

    Query head h reads kv head ``h // (h_q // h_kv)``.  ``rows`` restricts the
    query rows (definition mode evaluates them one by one; fast mode groups
    them 128 at a time).  ``alibi_exp`` = E selects the ALiBi bias with slope
    ``alibi_slope(h, h_q, E)`` for head h (``rope_base`` must then be None).
    Returns O [len(heads), len(rows), d], LSE [..].
    """
    h_q, h_kv = Q.shape[0], K.shape[0]
    group = h_q // h_kv
    if alibi_exp is not None and rope_base:
        raise ValueError("the ALiBi bias replaces RoPE: pass rope_base=None")
    heads = list(range(h_q)) if heads is None else list(heads)
    rows = np.arange(Q.shape[1]) if rows is None else np.asarray(rows)
    Os, Ls = [], []
    for h in heads:
        g = h // group
        m = None if alibi_exp is None else alibi_slope(h, h_q, alibi_exp)
        if mode == "definition":
            o, l = attention_rows(Q[h], K[g], V[g], rows, spec, rope_base, scale, m)
        else:
            blocks = [rows[s:s + TQ] for s in range(0, len(rows), TQ)]
            o, l = attention_fast(Q[h], K[g], V[g], spec, rope_base, scale, blocks, m)
        Os.append(o)
        Ls.append(l)
    return np.stack(Os), np.stack(Ls)


# ----------------------------------------------------------------------------
# Plan: per 128-query tile, the 64-key blocks to visit and the separators to gather
# ----------------------------------------------------------------------------

def plan_items_of_tile(spec: MaskSpec, t: int) -> List[int]:
    """Encoded items ``block | flags << 24`` of tile t, from the predicates.

    Candidate blocks hold a key ``j <= q1`` (``j <= P + q1`` for a segment).
    SepLLM only visits the sink blocks ``b < ceil(a/64)`` and the blocks from
    ``floor(win_lo/64)`` on, where ``win_lo = max(0, q0-w+1)``: keys in between
    are reached through the gathered separator list.  A candidate is kept
    when some (i, j) of tile x block is visible; FULL when all are (and the
    block has 64 keys); CAPPED when some visible pair has i - j > L.
    """
    n_q, n_k = spec.n_q, spec.n_k
    q0 = TQ * t
    q1 = min(n_q, q0 + TQ) - 1
    rows = np.arange(q0, q1 + 1, dtype=np.int64)
    last_key = min(n_k - 1, q1 + (spec.P if spec.mode == SEGMENT else 0))
    last_blk = last_key // BK
    if spec.mode == SEPLLM:
        nsb = -(-spec.a // BK)
        win_lo = max(0, q0 - spec.w + 1)
        cands = sorted(set(range(min(nsb, last_blk + 1))) | set(range(win_lo // BK, last_blk + 1)))
    else:
        cands = list(range(last_blk + 1))
    cands = np.array(cands, dtype=np.int64)
    # all candidate keys at once: [rows, candidates, 64]
    j = cands[:, None] * BK + np.arange(BK)[None, :]
    vis = visible(spec, rows[:, None, None], j[None, :, :])
    live = vis.any(axis=(0, 2))
    full = vis.all(axis=(0, 2)) & (cands * BK + BK <= n_k)
    if spec.mode == LAMBDA:
        cap = (vis & (rows[:, None, None] - j[None, :, :] > spec.L)).any(axis=(0, 2))
    else:
        cap = np.zeros(len(cands), dtype=bool)
    out = []
    for b, lv, fl, cp in zip(cands.tolist(), live, full, cap):
        if lv:
            out.append(b | ((FLAG_FULL if fl else 0) | (FLAG_CAPPED if cp else 0)) << 24)
    return out


def plan(spec: MaskSpec) -> Dict[str, np.ndarray]:
    """The plan the GPU must reproduce bit for bit.

    Returns tile_ptr int32 [n_tiles+1] (CSR into items), items int32,
    sep_count int32 [n_tiles], sep_idx int32 [n_sep] (ascending separator
    positions j >= g0 = 64*ceil(a/64)), sep_bits uint64 [n_blocks] (bit r of
    word b is sep[64b+r]).  ``sep_count[t]`` counts the separators in
    ``[g0, gh)`` with ``gh = 64*floor(win_lo/64)``; every such key precedes
    and lies outside the window of every query of the tile, so it is visible
    to all of them exactly when it is a separator.
    """
    n_q, n_k = spec.n_q, spec.n_k
    n_tiles = -(-n_q // TQ)
    n_blocks = -(-n_k // BK)
    tile_ptr = [0]
    items: List[int] = []
    sep_count = np.zeros(n_tiles, dtype=np.int32)
    sep_bits = np.zeros(n_blocks, dtype=np.uint64)
    sep_idx = np.zeros(0, dtype=np.int32)
    if spec.mode == SEPLLM:
        flags = spec.sep_flags()
        g0 = BK * (-(-spec.a // BK))
        sep_idx = np.array([j for j in range(g0, n_k) if flags[j] == 1], dtype=np.int32)
        for b in range(n_blocks):
            word = 0
            for r in range(BK):
                if BK * b + r < n_k and flags[BK * b + r] == 1:
                    word |= 1 << r
            sep_bits[b] = np.uint64(word)
    for t in range(n_tiles):
        it = plan_items_of_tile(spec, t)
        items.extend(it)
        tile_ptr.append(len(items))
        if spec.mode == SEPLLM:
            q0 = TQ * t
            win_lo = max(0, q0 - spec.w + 1)
            gh = BK * (win_lo // BK)
            g0 = BK * (-(-spec.a // BK))
            sep_count[t] = int(np.count_nonzero(sep_idx < gh)) if gh > g0 else 0
    return {
        "n_tiles": n_tiles, "n_blocks": n_blocks,
        "tile_ptr": np.array(tile_ptr, dtype=np.int32),
        "items": np.array(items, dtype=np.int32),
        "sep_count": sep_count,
        "sep_idx": sep_idx,
        "sep_bits": sep_bits,
    }


# ----------------------------------------------------------------------------
# Top-k retrieval of the prefix (segmented execution, long-range heads)
# ----------------------------------------------------------------------------

def topk_scores(q: np.ndarray, pool_k: np.ndarray) -> np.ndarray:
    """fp64 scores ``s_j = ((0 + q_0 k_j0) + q_1 k_j1) + ... + q_{d-1} k_j,d-1``.

    Inputs are bf16 or fp32 values upcast to fp64, so every product is exact
    and each step is one round-to-nearest addition (the same as an fma).
    """
    q = np.asarray(q, dtype=np.float64)
    pool_k = np.asarray(pool_k, dtype=np.float64)
    s = np.zeros(pool_k.shape[0], dtype=np.float64)
    for c in range(q.shape[0]):
        s = s + q[c] * pool_k[:, c]
    return s


def topk_select(scores: np.ndarray, k: int) -> np.ndarray:
    """The k largest scores, ties to the lower index, returned in ascending index order."""
    n = scores.shape[0]
    order = np.lexsort((np.arange(n), -scores))
    return np.sort(order[:k]).astype(np.int32)


# ----------------------------------------------------------------------------
# Counts and closed forms used by the measurement and the pins
# ----------------------------------------------------------------------------

def pair_counts(spec: MaskSpec) -> np.ndarray:
    """|A_i| for every query i (int64), from the predicates."""
    out = np.zeros(spec.n_q, dtype=np.int64)
    for s in range(0, spec.n_q, TQ):
        rows = np.arange(s, min(spec.n_q, s + TQ))
        out[rows] = mask_rows(spec, rows).sum(axis=1)
    return out


def pair_count_total(spec: MaskSpec) -> int:
    return int(pair_counts(spec).sum())


def q0_closed_form(v: np.ndarray, spec: MaskSpec, rows: Sequence[int]):
    """With Q = 0 every visible logit is 0: O_i = mean of v_j over A_i, LSE_i = ln |A_i|."""
    v = np.asarray(v, dtype=np.float64)
    O = np.zeros((len(rows), v.shape[1]))
    lse = np.zeros(len(rows))
    for r, i in enumerate(rows):
        A = key_set(spec, int(i))
        O[r] = v[A].mean(axis=0)
        lse[r] = math.log(len(A))
    return O, lse


# ----------------------------------------------------------------------------
# ALiBi-style bias (LM-Infinite page, section 方法: distance clipped to L_pretrain)
# ----------------------------------------------------------------------------

def alibi_slope(h: int, h_q: int, exp: float) -> float:
    """Slope of query head h: ``2 ** (-exp * (h + 1) / h_q)``, a geometric sequence."""
    return 2.0 ** (-float(exp) * (h + 1) / h_q)


def q0_alibi_closed_form(v: np.ndarray, spec: MaskSpec, rows: Sequence[int], m: float):
    """Lambda mask with Q = 0: key j's logit is ``-m * min(i-j, L)``.

    The partition function is summed in closed form, not over A_i: the window
    keys ``i-j = 0..min(i, L)`` make the geometric series
    ``(1 - e^{-m (W+1)}) / (1 - e^{-m})`` and each of the
    ``min(n_s, max(0, i-L))`` starting-span keys outside the window adds
    ``e^{-m L}``.  O_i is the bias-weighted mean of v over A_i."""
    v = np.asarray(v, dtype=np.float64)
    O = np.zeros((len(rows), v.shape[1]))
    lse = np.zeros(len(rows))
    for r, i in enumerate(rows):
        i = int(i)
        W = min(i, spec.L)
        n_far = min(spec.n_s, max(0, i - spec.L))
        win = -math.expm1(-m * (W + 1)) / -math.expm1(-m) if m > 0 else float(W + 1)
        lse[r] = math.log(win + n_far * math.exp(-m * spec.L))
        A = key_set(spec, i)
        wgt = np.exp(-m * np.minimum(i - A, spec.L))
        O[r] = (wgt @ v[A]) / wgt.sum()
    return O, lse


# ----------------------------------------------------------------------------
# Several segments end to end (segmented-execution page, 方法详解 / 整体框架 and
# 关键设计: (C_i, o_i) = F(x_i, C_{i-1}, R_{i-1}))
# ----------------------------------------------------------------------------

def segmented_run(Q_segs, K_segs, V_segs, n_local: int, M: int, R: int,
                  rope_base: Optional[float], scale: float):
    """Runs N segments through the segment recurrence, one head set per call.

    Q_segs[i], K_segs[i], V_segs[i]: [H, S, d] raw projections of segment i.
    Heads 0..n_local-1 are local: they attend to [C_{i-1} | segment], C being
    the latest M raw keys/values they have seen (the tail carried across
    segments).  Heads n_local..H-1 are long-range: they attend to
    [R_{i-1} | segment], R_{i-1} being the top-R rows of a read-only pool that
    holds every earlier segment's raw keys/values of those heads, scored by
    the segment-end raw query and kept in pool order.  Segment 1 has no
    prefix.  The prefix takes positions 0..P-1 and the segment P..P+S-1
    (attention in SEGMENT mode); the carried tail and the retrieved prefix
    have the same length, so M == R is required.

    Order after segment i: the tail becomes the last M rows of
    [C_{i-1} | segment]; the segment's long-head rows are appended to the
    pool; the next prefix is retrieved from the updated pool with the last
    query of segment i.

    Returns a list of per-segment dicts {"O", "LSE", "P", "idx"} (idx: the
    retrieved pool rows the segment's long heads read, or None) and the final
    state {"tail_k", "tail_v", "pool_k", "pool_v"}.
    """
    if M != R:
        raise ValueError("the carried tail and the retrieved prefix must have one length")
    H, S, d = np.asarray(Q_segs[0]).shape
    n_long = H - n_local
    tail_k = np.zeros((n_local, 0, d))
    tail_v = np.zeros((n_local, 0, d))
    pool_k = np.zeros((n_long, 0, d))
    pool_v = np.zeros((n_long, 0, d))
    pref_k = np.zeros((n_long, 0, d))
    pref_v = np.zeros((n_long, 0, d))
    idx = None
    out = []
    for Qi, Ki, Vi in zip(Q_segs, K_segs, V_segs):
        Qi = np.asarray(Qi, dtype=np.float64)
        Ki = np.asarray(Ki, dtype=np.float64)
        Vi = np.asarray(Vi, dtype=np.float64)
        P = tail_k.shape[1]
        assert pref_k.shape[1] == P
        Kc = np.concatenate([np.concatenate([tail_k, pref_k], axis=0), Ki], axis=1)
        Vc = np.concatenate([np.concatenate([tail_v, pref_v], axis=0), Vi], axis=1)
        spec = MaskSpec(SEGMENT, S, P + S, P=P)
        O, L = attention(Qi, Kc, Vc, spec, rope_base, scale)
        out.append({"O": O, "LSE": L, "P": P, "idx": idx})
        # carry: the latest M keys/values of the local heads
        keep = min(M, P + S)
        tail_k = Kc[:n_local, P + S - keep:]
        tail_v = Vc[:n_local, P + S - keep:]
        # the detached pool gains this segment's long-head rows
        pool_k = np.concatenate([pool_k, Ki[n_local:]], axis=1)
        pool_v = np.concatenate([pool_v, Vi[n_local:]], axis=1)
        # the next prefix: top-R pool rows scored by this segment's last query
        k_sel = min(R, pool_k.shape[1])
        idx = np.stack([topk_select(topk_scores(Qi[n_local + j, S - 1], pool_k[j]), k_sel)
                        for j in range(n_long)]) if n_long else np.zeros((0, k_sel), dtype=np.int64)
        pref_k = np.stack([pool_k[j, idx[j]] for j in range(n_long)]) if n_long else np.zeros((0, k_sel, d))
        pref_v = np.stack([pool_v[j, idx[j]] for j in range(n_long)]) if n_long else np.zeros((0, k_sel, d))
    return out, {"tail_k": tail_k, "tail_v": tail_v, "pool_k": pool_k, "pool_v": pool_v}


# ----------------------------------------------------------------------------
# Backward of the masked attention (gradients of O with respect to q, k, v)
# ----------------------------------------------------------------------------

def attention_grad_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, dO: np.ndarray,
                        rows: Sequence[int], spec: MaskSpec, rope_base: Optional[float],
                        scale: float, alibi: Optional[float] = None):
    """Gradients of the listed rows' outputs, one head, definition mode.

    For query i with key set A_i, logits s_j as in :func:`attention_rows`
    (``s_j = scale <R(delta'_ij) q_i, k_j>``, plus ``-m delta'`` with ALiBi),
    p = softmax(s), o_i = sum_j p_j v_j.  With the upstream gradient dO_i:
    dp_j = <dO_i, v_j>, D_i = <dO_i, o_i>, ds_j = p_j (dp_j - D_i), and
      dq_i  = sum_j ds_j * scale * R(-delta'_ij) k_j,
      dk_j += ds_j * scale * R(delta'_ij) q_i,
      dv_j += p_j * dO_i
    (the rotation is orthogonal, so the transpose of R(delta) is R(-delta)).
    Returns dq [len(rows), d] and the contributions of these rows to dk, dv
    [n_k, d]; summed over every query row they are the full dk, dv.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    d = q.shape[1]
    theta = rope_theta(d, rope_base) if rope_base else None
    dq = np.zeros((len(rows), d))
    dk = np.zeros((k.shape[0], d))
    dv = np.zeros((v.shape[0], v.shape[1]))
    for r, i in enumerate(rows):
        i = int(i)
        A = key_set(spec, i)
        delta = pos_q(spec, i) - pos_k(spec, A)
        if spec.mode == LAMBDA:
            delta = np.minimum(delta, spec.L)
        if theta is None:
            qr = np.broadcast_to(q[i], (len(A), d))
            kr = k[A]
        else:
            ang = delta.astype(np.float64)[:, None] * theta[None, :]
            qr = rotate(np.broadcast_to(q[i], (len(A), d)), ang)   # R(delta) q_i per key
            kr = rotate(k[A], -ang)                                 # R(-delta) k_j per key
        s = scale * np.einsum("jd,jd->j", qr, k[A])
        if alibi is not None:
            s = s - alibi * delta.astype(np.float64)
        p = np.exp(s - s.max())
        p = p / p.sum()
        o = p @ v[A]
        dp = v[A] @ dO[i]
        ds = p * (dp - dO[i] @ o)
        dq[r] = scale * (ds @ kr)
        np.add.at(dk, A, scale * ds[:, None] * qr)
        np.add.at(dv, A, p[:, None] * dO[i][None, :])
    return dq, dk, dv


def attention_grad_keys_fast(q: np.ndarray, k: np.ndarray, v: np.ndarray, dO: np.ndarray,
                             spec: MaskSpec, rope_base: Optional[float], scale: float,
                             keys: Sequence[int], rows: Sequence[int],
                             alibi: Optional[float] = None):
    """dk, dv of the listed keys summed over the listed query rows, one head: the same
    gradients as :func:`attention_grad_rows`, computed tile-wise like
    :func:`attention_fast` (absolute rotations, one dense masked product per block of
    up to 128 rows).

    With qr_i = R(pos_q(i)) q_i and kr_j = R(pos_k(j)) k_j the logit is
    s_ij = scale <qr_i, kr_j>, so ds/dk_j = scale R(-pos_k(j)) qr_i; a capped
    LM-Infinite pair has s_ij = scale <R(L) q_i, k_j> and ds/dk_j = scale R(L) q_i;
    with the ALiBi bias (no rotation) ds/dk_j = scale q_i.  Per row: p = softmax(s),
    o = p V, D = <dO_i, o>, ds_j = p_j (<dO_i, v_j> - D); dk_j += ds_j ds/dk_j and
    dv_j += p_j dO_i.  Returns dk, dv [len(keys), d].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    d = q.shape[1]
    theta = rope_theta(d, rope_base) if rope_base else None
    dk = np.zeros((len(keys), d))
    dv = np.zeros((len(keys), v.shape[1]))
    for s0 in range(0, len(rows), TQ):
        R = rows[s0:s0 + TQ]
        M = mask_rows(spec, R)
        U = np.flatnonzero(M.any(axis=0))
        Mu = M[:, U]
        C = np.zeros(Mu.shape, dtype=bool)
        if theta is not None:
            qr = rotate(q[R], pos_q(spec, R).astype(np.float64)[:, None] * theta[None, :])
            kr = rotate(k[U], pos_k(spec, U).astype(np.float64)[:, None] * theta[None, :])
            S = qr @ kr.T
            if spec.mode == LAMBDA:
                C = capped(spec, R[:, None], U[None, :])
                qcap = rotate(q[R], float(spec.L) * theta[None, :])
                S = np.where(C, qcap @ k[U].T, S)
        else:
            qr = q[R]
            S = qr @ k[U].T
        S = S * scale
        if alibi is not None:
            dist = pos_q(spec, R)[:, None] - pos_k(spec, U)[None, :]
            if spec.mode == LAMBDA:
                dist = np.minimum(dist, spec.L)
            S = S - alibi * dist.astype(np.float64)
        S = np.where(Mu, S, -np.inf)
        P = np.exp(S - S.max(axis=1, keepdims=True))
        P = P / P.sum(axis=1, keepdims=True)
        Oo = P @ v[U]
        D = np.einsum("rd,rd->r", dO[R], Oo)
        dS = P * (dO[R] @ v[U].T - D[:, None])
        pos_in_u = np.searchsorted(U, keys)
        present = (pos_in_u < len(U)) & (U[np.minimum(pos_in_u, len(U) - 1)] == keys)
        kk = np.flatnonzero(present)
        cols = pos_in_u[kk]
        dv[kk] += P[:, cols].T @ dO[R]
        dsn = np.where(C[:, cols], 0.0, dS[:, cols])
        dsc = np.where(C[:, cols], dS[:, cols], 0.0)
        g = scale * (dsn.T @ qr)  # sum_i ds_ij qr_i, in the rotated frame of key j
        if theta is not None:
            g = rotate(g, -pos_k(spec, keys[kk]).astype(np.float64)[:, None] * theta[None, :])
            if C.any():
                g = g + scale * (dsc.T @ rotate(q[R], float(spec.L) * theta[None, :]))
        dk[kk] += g
    return dk, dv


def attention_backward(Q, K, V, dO, spec: MaskSpec, rope_base: Optional[float], scale: float,
                       alibi_exp: Optional[float] = None, rows: Optional[Sequence[int]] = None):
    """Multi-head gradients: Q, dO [h_q, n_q, d]; K, V [h_kv, n_k, d] (batch squeezed).

    dK and dV of kv head g sum the contributions of its query heads
    h in [g*G, (g+1)*G), G = h_q / h_kv.  ``rows`` restricts the query rows
    (dQ is returned for those rows; dK, dV then hold only their contributions).
    """
    h_q, h_kv = Q.shape[0], K.shape[0]
    group = h_q // h_kv
    rows = np.arange(Q.shape[1]) if rows is None else np.asarray(rows)
    dQ = np.zeros((h_q, len(rows), Q.shape[2]))
    dK = np.zeros(K.shape, dtype=np.float64)
    dV = np.zeros(V.shape, dtype=np.float64)
    for h in range(h_q):
        g = h // group
        m = None if alibi_exp is None else alibi_slope(h, h_q, alibi_exp)
        dq, dk, dv = attention_grad_rows(Q[h], K[g], V[g], dO[h], rows, spec, rope_base, scale, m)
        dQ[h] = dq
        dK[g] += dk
        dV[g] += dv
    return dQ, dK, dV


# ----------------------------------------------------------------------------
# Streaming decode with the four-part cache (SepLLM page, part 6.2, generation)
# ----------------------------------------------------------------------------

class StreamCache:
    """Which tokens the generation-time cache holds, one token at a time.

    Parts: Initial (the first ``a`` tokens), Separator (at most ``s``
    separators, the most recent kept), Local window (the last ``w`` tokens,
    the newest one included) and Past (tokens that left the local window
    since the last compression).  The run size ``a + s + w + |Past|`` may
    not exceed ``c``: when a token entering Past brings it to ``c``, the
    separators of Past move to the Separator part (the oldest separators
    beyond ``s`` are dropped) and the rest of Past is discarded.  Positions
    are the tokens' original indices.  Holds token indices only.
    """

    def __init__(self, a: int, s: int, w: int, c: int):
        if not (a >= 0 and s >= 1 and w >= 1 and c > a + s + w):
            raise ValueError("need a >= 0, s >= 1, w >= 1 and c > a + s + w")
        self.a, self.s, self.w, self.c = a, s, w, c
        self.initial: List[int] = []
        self.sep: List[int] = []
        self.local: List[int] = []
        self.past: List[int] = []
        self.flags: List[int] = []
        self.t = 0

    @property
    def run_size(self) -> int:
        return self.a + self.s + self.w + len(self.past)

    def append(self, is_sep: bool) -> int:
        """Adds token ``t`` (the next index) and applies the policy; returns t."""
        t = self.t
        self.flags.append(1 if is_sep else 0)
        if t < self.a:
            self.initial.append(t)
        else:
            self.local.append(t)
            if len(self.local) > self.w:
                self.past.append(self.local.pop(0))
                if self.run_size >= self.c:
                    moved = [j for j in self.past if self.flags[j]]
                    self.sep = (self.sep + moved)[-self.s:]
                    self.past = []
        self.t = t + 1
        return t

    def tokens(self) -> np.ndarray:
        return np.array(sorted(self.initial + self.sep + self.past + self.local), dtype=np.int64)


def stream_cache_tokens(t: int, flags: np.ndarray, a: int, s: int, w: int, c: int) -> np.ndarray:
    """The same set in closed form, after token t has been added.

    Tokens a, a+1, ... leave the local window in order: after token t,
    e = max(0, t + 1 - a - w) of them have.  Every P = c - a - s - w of them
    a compression empties Past, so Past holds the last e mod P of them and
    the first P * floor(e / P) were compressed; the Separator part holds the
    last s separators among the compressed tokens.
    """
    P = c - a - s - w
    e = max(0, t + 1 - a - w)
    comp = P * (e // P)
    init = np.arange(0, min(a, t + 1))
    local = np.arange(max(a, t - w + 1), t + 1) if t >= a else np.arange(0)
    past = np.arange(a + comp, a + e)
    compressed = np.arange(a, a + comp)
    seps = compressed[np.asarray(flags)[compressed] == 1][-s:] if comp > 0 else np.arange(0)
    return np.array(sorted(set(init.tolist()) | set(seps.tolist()) | set(past.tolist())
                           | set(local.tolist())), dtype=np.int64)


def decode_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, t: int, tokens: np.ndarray,
                     rope_base: Optional[float], scale: float):
    """One decode step of one head: query t over the cached tokens (SepLLM page,
    part 6.1 restricted to the held keys), RoPE at the original positions.
    q [d] raw; k, v [n, d] raw rows of every token so far.  Returns o [d], lse."""
    q = np.asarray(q, dtype=np.float64)
    kk = np.asarray(k, dtype=np.float64)[tokens]
    vv = np.asarray(v, dtype=np.float64)[tokens]
    if rope_base:
        d = q.shape[0]
        theta = rope_theta(d, rope_base)
        ang = (float(t) - tokens.astype(np.float64))[:, None] * theta[None, :]
        s_ = scale * np.einsum("jd,jd->j", rotate(np.broadcast_to(q, kk.shape), ang), kk)
    else:
        s_ = scale * (kk @ q)
    mu = s_.max()
    e = np.exp(s_ - mu)
    return (e @ vv) / e.sum(), mu + math.log(e.sum())


# ----------------------------------------------------------------------------
# LM-Infinite's optional top-k middle tokens (LM-Infinite page, section 方法)
# ----------------------------------------------------------------------------

def middle_scores(q: np.ndarray, k: np.ndarray, spec: MaskSpec, i: int, rope_base: Optional[float],
                  scale: float):
    """The middle tokens of query i, ``n_starting <= j < i - L`` (outside both
    spans of the Lambda mask), and their logits at the capped distance L:
    ``scale <R(L) q_i, k_j>`` (or ``scale <q_i, k_j>`` without RoPE).
    Returns (j ascending, logits)."""
    assert spec.mode == LAMBDA
    j = np.arange(spec.n_s, max(spec.n_s, i - spec.L))
    q = np.asarray(q, dtype=np.float64)
    qi = q[i]
    if rope_base:
        qi = rotate(qi, float(spec.L) * rope_theta(q.shape[1], rope_base))
    return j, scale * (np.asarray(k, dtype=np.float64)[j] @ qi)


def attention_topk_middle(q: np.ndarray, k: np.ndarray, v: np.ndarray, rows: Sequence[int],
                          spec: MaskSpec, rope_base: Optional[float], scale: float, k_mid: int):
    """Lambda-mask attention with the k largest-logit middle tokens of each query
    added to its key set (ties to the lower index); every key beyond the
    window, selected middle tokens included, takes the capped distance L.
    Returns O [len(rows), d], LSE and the selected indices [len(rows), <= k_mid]
    (ascending)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d = q.shape[1]
    theta = rope_theta(d, rope_base) if rope_base else None
    O = np.zeros((len(rows), v.shape[1]))
    lse = np.zeros(len(rows))
    sels = []
    for r, i in enumerate(rows):
        i = int(i)
        jm, sm = middle_scores(q, k, spec, i, rope_base, scale)
        sel = jm[topk_select(sm, min(k_mid, len(jm)))] if len(jm) else jm
        sels.append(sel)
        A = np.union1d(key_set(spec, i), sel)
        delta = np.minimum(pos_q(spec, i) - pos_k(spec, A), spec.L)
        if theta is None:
            s_ = k[A] @ q[i]
        else:
            ang = delta.astype(np.float64)[:, None] * theta[None, :]
            s_ = np.einsum("jd,jd->j", rotate(np.broadcast_to(q[i], (len(A), d)), ang), k[A])
        s_ = s_ * scale
        mu = s_.max()
        e = np.exp(s_ - mu)
        O[r] = (e @ v[A]) / e.sum()
        lse[r] = mu + math.log(e.sum())
    return O, lse, sels

