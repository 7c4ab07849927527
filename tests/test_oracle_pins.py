"""Pins for the fp64 oracle: it is checked against things other than itself.

Pins, by oracle function:
  visible / key_set     hand-written key sets (tests/golden/key_sets_hand.json);
                        counting closed forms; degenerate cases against masks
                        built by torch.tril/triu.
  rope_theta / rotate   hand-evaluated d=4 example; the complex-exponential
                        form; R(0)=I; norm preservation; relative-position
                        identity <R(a)q,R(b)k> = <R(a-b)q,k>.
  attention_rows/_fast  torch scaled_dot_product_attention (fp64, CPU) on the
                        degenerate cases named by the pages (full causal,
                        pure window, segment causal); Q=0 closed form;
                        definition mode == fast mode (incl. the capped RoPE
                        realisation); LSE against torch.logsumexp.
  plan                  coverage identity (every visible pair covered exactly
                        once); numpy packbits for sep_bits; flatnonzero for
                        the separator list.
  topk_scores/_select   pure-Python float chain; exact rational error bound;
                        heapq.nlargest; k=N and k=1 special cases.
  pair counts           closed forms for LM-Infinite, segment and SepLLM; the
                        segmented page's effective context S + aM + b(1-a)R.
  ALiBi (Lambda)        the textbook geometric slopes (h_q = 8: 1/2 .. 1/256);
                        torch SDPA with an additive bias built by torch where
                        no distance reaches the cap; Q = 0 closed forms (the
                        geometric-series partition function and the weight at
                        distance 0, at the cap and beyond it); a steep slope
                        that leaves only the diagonal.
  segmented_run         the whole history of raw projections: the final tail
                        is the latest M history rows, the pool every long-head
                        row; each retrieved prefix is heapq's top-M of the
                        history under a pure-Python score chain; every
                        segment's output equals torch SDPA on explicitly
                        rotated [prefix | segment] rows.
  attention_grad_rows / attention_backward
                        torch.autograd (fp64) through forwards built here from
                        torch primitives (SepLLM, segment, capped Lambda via
                        the RoPE realisation, capped ALiBi, GQA); central
                        finite differences through the definition-mode forward.
  StreamCache / stream_cache_tokens / decode_attention
                        a ten-step hand trace of the generation-time cache
                        (tests/golden/stream_cache_hand.json); the state
                        machine against the independently written closed form
                        on long random streams; the run size never above c and
                        its mean over whole periods under the page's bound
                        (w+c+a+s)/2; decode output against torch SDPA on
                        explicitly rotated rows with a mask over the held set.
  middle_scores / attention_topk_middle
                        k at least the middle size: the capped realisation over
                        the whole causal mask built in torch; the selection
                        against heapq over pure-Python scores (exact ties);
                        k = 0 equals the Lambda attention.
"""
import heapq
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(12345)


# ---------------------------------------------------------------------------
# helpers written independently of the oracle
# ---------------------------------------------------------------------------

def complex_rope(x: torch.Tensor, pos: torch.Tensor, base: float) -> torch.Tensor:
    """RoPE as a complex product: (x_c + i x_{c+d/2}) * exp(i pos base^(-2c/d))."""
    d = x.shape[-1]
    inv = 1.0 / (base ** (torch.arange(0, d, 2, dtype=torch.float64) / d))
    ang = pos.to(torch.float64)[:, None] * inv[None, :]
    z = torch.complex(x[..., : d // 2], x[..., d // 2:]) * torch.polar(torch.ones_like(ang), ang)
    return torch.cat([z.real, z.imag], dim=-1)


def sdpa(q, k, v, mask, scale):
    return torch.nn.functional.scaled_dot_product_attention(
        q[None, None], k[None, None], v[None, None], attn_mask=mask[None, None], scale=scale)[0, 0]


def rand(*shape):
    return RNG.standard_normal(shape)


# ---------------------------------------------------------------------------
# key sets
# ---------------------------------------------------------------------------

def test_key_sets_hand_written():
    g = json.load(open(os.path.join(GOLDEN, "key_sets_hand.json")))
    s = g["sepllm"]
    flags = np.zeros(s["m"], np.uint8)
    flags[s["sep"]] = 1
    spec = O.MaskSpec(O.SEPLLM, s["m"], s["m"], a=s["a"], w=s["w"], sep=flags)
    assert [O.key_set(spec, i).tolist() for i in range(s["m"])] == s["A"]
    lam = g["lambda"]
    spec = O.MaskSpec(O.LAMBDA, lam["m"], lam["m"], n_s=lam["n_s"], L=lam["L"])
    assert [O.key_set(spec, i).tolist() for i in range(lam["m"])] == lam["A"]
    capped = [np.flatnonzero(O.capped(spec, i, np.arange(lam["m"]))).tolist() for i in range(lam["m"])]
    assert capped == lam["capped"]
    seg = g["segment"]
    spec = O.MaskSpec(O.SEGMENT, seg["S"], seg["S"] + seg["P"], P=seg["P"])
    assert [O.key_set(spec, i).tolist() for i in range(seg["S"])] == seg["A"]


def _sepllm_count_closed_form(m, a, w, flags):
    """|A_i| = min(i+1, w) + #{j < a : j <= i-w} + #{separators j >= a : j <= i-w}."""
    sep_not_sink = np.where(np.arange(m) >= a, flags, 0).astype(np.int64)
    cs = np.concatenate([[0], np.cumsum(sep_not_sink)])
    out = []
    for i in range(m):
        far = i - w  # keys j <= far are outside the window
        n = min(i + 1, w)
        if far >= 0:
            n += min(a, far + 1) + cs[far + 1]
        out.append(n)
    return np.array(out)


@pytest.mark.parametrize("m,a,w,p", [(200, 4, 16, 0.1), (333, 70, 5, 0.3), (150, 0, 1, 0.5),
                                     (129, 3, 200, 0.2)])
def test_sepllm_counts_closed_form(m, a, w, p):
    flags = (RNG.random(m) < p).astype(np.uint8)
    spec = O.MaskSpec(O.SEPLLM, m, m, a=a, w=w, sep=flags)
    np.testing.assert_array_equal(O.pair_counts(spec), _sepllm_count_closed_form(m, a, w, flags))


def test_lambda_count_closed_form():
    # per-row |A_i| = min(i, L) + 1 + min(n_s, max(0, i - L))
    for m, n_s, L in [(700, 10, 100), (300, 0, 64), (257, 64, 7), (100, 3, 200)]:
        spec = O.MaskSpec(O.LAMBDA, m, m, n_s=n_s, L=L)
        expect = [min(i, L) + 1 + min(n_s, max(0, i - L)) for i in range(m)]
        np.testing.assert_array_equal(O.pair_counts(spec), expect)


def test_lambda_32k_pair_count_closed_form():
    # the 32K LM-Infinite workload (n_s=10, L=4096): closed form only (the predicate
    # version of the same count is checked at smaller sizes above)
    m, n_s, L = 32768, 10, 4096
    total = sum(min(i, L) + 1 + min(n_s, max(0, i - L)) for i in range(m))
    capped = sum(min(n_s, max(0, i - L)) for i in range(m))
    assert total == 126_146_505 and capped == 286_665


def test_segment_count_and_effective_context():
    S, P = 96, 40
    spec = O.MaskSpec(O.SEGMENT, S, S + P, P=P)
    assert O.pair_count_total(spec) == S * P + S * (S + 1) // 2
    # effective context per token (segmented page, key design 3): S + alpha*M + beta*(1-alpha)*R
    # for the last query of a long-range layer (beta = 1): local heads see M + S keys, long
    # heads R + S; with M = R = P the head average is S + alpha*P + (1-alpha)*P.
    h_local, h_long = 24, 8
    alpha = h_local / (h_local + h_long)
    per_head = [len(O.key_set(spec, S - 1))] * (h_local + h_long)
    assert np.mean(per_head) == pytest.approx(S + alpha * P + 1.0 * (1 - alpha) * P)
    assert O.pair_count_total(O.MaskSpec(O.SEGMENT, 4096, 5120, P=1024)) == 12_584_960


def test_degenerate_masks_against_torch_construction():
    m = 150
    causal = torch.ones(m, m, dtype=torch.bool).tril()
    # SepLLM a=0, w>=m, no separators -> full causal
    spec = O.MaskSpec(O.SEPLLM, m, m, a=0, w=m, sep=None)
    np.testing.assert_array_equal(O.mask_rows(spec, range(m)), causal.numpy())
    # SepLLM with every token a separator -> full causal
    spec = O.MaskSpec(O.SEPLLM, m, m, a=3, w=5, sep=np.ones(m, np.uint8))
    np.testing.assert_array_equal(O.mask_rows(spec, range(m)), causal.numpy())
    # SepLLM a=0 no separators -> band of width w
    spec = O.MaskSpec(O.SEPLLM, m, m, a=0, w=7, sep=None)
    np.testing.assert_array_equal(O.mask_rows(spec, range(m)), causal.triu(-6).numpy())
    # SepLLM general = band | sink columns | separator columns, within causal
    flags = (RNG.random(m) < 0.2).astype(np.uint8)
    spec = O.MaskSpec(O.SEPLLM, m, m, a=5, w=9, sep=flags)
    cols = torch.zeros(m, dtype=torch.bool)
    cols[:5] = True
    cols |= torch.from_numpy(flags).bool()
    expect = causal & (causal.triu(-8) | cols[None, :])
    np.testing.assert_array_equal(O.mask_rows(spec, range(m)), expect.numpy())
    # Lambda n_s = 0 degenerates to the recent window i - j <= L (LM-Infinite, method)
    spec = O.MaskSpec(O.LAMBDA, m, m, n_s=0, L=20)
    np.testing.assert_array_equal(O.mask_rows(spec, range(m)), causal.triu(-20).numpy())
    # Lambda L >= m-1 -> full causal
    spec = O.MaskSpec(O.LAMBDA, m, m, n_s=4, L=m - 1)
    np.testing.assert_array_equal(O.mask_rows(spec, range(m)), causal.numpy())
    # Segment: prefix fully visible, segment causal
    S, P = 70, 30
    spec = O.MaskSpec(O.SEGMENT, S, S + P, P=P)
    np.testing.assert_array_equal(O.mask_rows(spec, range(S)),
                                  torch.ones(S, S + P, dtype=torch.bool).tril(P).numpy())


# ---------------------------------------------------------------------------
# rotary embedding
# ---------------------------------------------------------------------------

def test_rope_hand_example():
    # d = 4, base = 100: theta = (1, 0.1); pairs are (x0, x2) and (x1, x3)
    np.testing.assert_allclose(O.rope_theta(4, 100.0), [1.0, 0.1], rtol=0, atol=1e-15)
    x = np.array([1.0, 2.0, 3.0, 4.0])
    c1, s1, c2, s2 = math.cos(1.0), math.sin(1.0), math.cos(0.1), math.sin(0.1)
    expect = [1 * c1 - 3 * s1, 2 * c2 - 4 * s2, 3 * c1 + 1 * s1, 4 * c2 + 2 * s2]
    got = O.rotate(x, 1.0 * O.rope_theta(4, 100.0))
    np.testing.assert_allclose(got, expect, rtol=0, atol=1e-15)


@pytest.mark.parametrize("base", [10000.0, 500000.0])
def test_rope_matches_complex_form_and_identities(base):
    d, n = 128, 64
    x = rand(n, d)
    pos = RNG.integers(0, 131072, size=n)
    theta = O.rope_theta(d, base)
    got = O.rotate(x, pos[:, None] * theta[None, :])
    ref = complex_rope(torch.from_numpy(x), torch.from_numpy(pos), base).numpy()
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-10)
    np.testing.assert_allclose(O.rotate(x, 0 * theta[None, :]), x, rtol=0, atol=0)
    np.testing.assert_allclose(np.linalg.norm(got, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    q, k = rand(d), rand(d)
    for a_, b_ in [(5, 3), (100000, 99000), (4096, 0), (17, 17)]:
        lhs = O.rotate(q, a_ * theta) @ O.rotate(k, b_ * theta)
        rhs = O.rotate(q, (a_ - b_) * theta) @ k
        assert abs(lhs - rhs) < 1e-10


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def _pre_rotated(q, k, pq, pk, base):
    if base is None:
        return torch.from_numpy(q), torch.from_numpy(k)
    return (complex_rope(torch.from_numpy(q), torch.from_numpy(pq), base),
            complex_rope(torch.from_numpy(k), torch.from_numpy(pk), base))


@pytest.mark.parametrize("base", [None, 10000.0])
def test_attention_degenerate_cases_vs_sdpa(base):
    d, m = 64, 200
    scale = 1.0 / math.sqrt(d)
    q, k, v = rand(m, d), rand(m, d), rand(m, d)
    pos = np.arange(m)
    qr, kr = _pre_rotated(q, k, pos, pos, base)
    causal = torch.ones(m, m, dtype=torch.bool).tril()
    cases = [
        (O.MaskSpec(O.SEPLLM, m, m, a=0, w=m), causal),                      # full causal
        (O.MaskSpec(O.LAMBDA, m, m, n_s=0, L=31), causal.triu(-31)),          # pure window
        (O.MaskSpec(O.LAMBDA, m, m, n_s=5, L=m - 1), causal),                 # no capping
        (O.MaskSpec(O.SEPLLM, m, m, a=0, w=16), causal.triu(-15)),           # band, no sinks
    ]
    for spec, mask in cases:
        ref = sdpa(qr, kr, torch.from_numpy(v), mask, scale).numpy()
        o_fast, _ = O.attention_fast(q, k, v, spec, base, scale)
        o_def, _ = O.attention_rows(q, k, v, range(m), spec, base, scale)
        np.testing.assert_allclose(o_fast, ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(o_def, ref, rtol=0, atol=1e-12)
    # segment: prefix 0..P-1, queries at P + i
    S, P = 150, 50
    q, k, v = rand(S, d), rand(S + P, d), rand(S + P, d)
    qr, kr = _pre_rotated(q, k, np.arange(P, P + S), np.arange(S + P), base)
    mask = torch.ones(S, S + P, dtype=torch.bool).tril(P)
    ref = sdpa(qr, kr, torch.from_numpy(v), mask, scale).numpy()
    spec = O.MaskSpec(O.SEGMENT, S, S + P, P=P)
    o_fast, _ = O.attention_fast(q, k, v, spec, base, scale)
    o_def, _ = O.attention_rows(q, k, v, range(S), spec, base, scale)
    np.testing.assert_allclose(o_fast, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(o_def, ref, rtol=0, atol=1e-12)


def test_attention_general_sepllm_vs_sdpa_and_lse():
    d, m = 128, 300
    scale = 1.0 / math.sqrt(d)
    q, k, v = rand(m, d), rand(m, d), rand(m, d)
    flags = (RNG.random(m) < 0.1).astype(np.uint8)
    spec = O.MaskSpec(O.SEPLLM, m, m, a=4, w=40, sep=flags)
    qr, kr = _pre_rotated(q, k, np.arange(m), np.arange(m), 10000.0)
    causal = torch.ones(m, m, dtype=torch.bool).tril()
    cols = torch.zeros(m, dtype=torch.bool)
    cols[:4] = True
    cols |= torch.from_numpy(flags).bool()
    mask = causal & (causal.triu(-39) | cols[None, :])
    ref = sdpa(qr, kr, torch.from_numpy(v), mask, scale).numpy()
    logits = (qr @ kr.T) * scale
    ref_lse = torch.logsumexp(logits.masked_fill(~mask, -math.inf), dim=1).numpy()
    o, lse = O.attention_fast(q, k, v, spec, 10000.0, scale)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)
    o2, lse2 = O.attention_rows(q, k, v, range(m), spec, 10000.0, scale)
    np.testing.assert_allclose(o2, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2, ref_lse, rtol=0, atol=1e-12)


def test_lambda_capped_definition_equals_realisation():
    # LM-Infinite, method: distance cap d' = min(i-j, L) (definition mode rotates q by d'
    # per pair) versus the page's RoPE realisation (fast mode: raw key, query rotated by L)
    d, m = 128, 400
    scale = 1.0 / math.sqrt(d)
    q, k, v = rand(m, d), rand(m, d), rand(m, d)
    spec = O.MaskSpec(O.LAMBDA, m, m, n_s=10, L=64)
    o_def, l_def = O.attention_rows(q, k, v, range(m), spec, 10000.0, scale)
    o_fast, l_fast = O.attention_fast(q, k, v, spec, 10000.0, scale)
    np.testing.assert_allclose(o_fast, o_def, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l_fast, l_def, rtol=0, atol=1e-12)
    # the cap changes the result: uncapped RoPE over the same key set differs
    o_unc, _ = O.attention_rows(q, k, v, range(m), O.MaskSpec(O.SEPLLM, m, m, a=10, w=65),
                                10000.0, scale)
    assert np.abs(o_unc[200:] - o_def[200:]).max() > 1e-3
    # with the same key set (a = n_s, w = L+1) the two masks coincide; rows i <= L never cap
    np.testing.assert_allclose(o_unc[:65], o_def[:65], rtol=0, atol=1e-12)
    # at i - j == L both branches of the realisation agree
    theta = O.rope_theta(d, 10000.0)
    i, j = 300, 300 - 64
    a_ = O.rotate(q[i], i * theta) @ O.rotate(k[j], j * theta)
    b_ = O.rotate(q[i], 64 * theta) @ k[j]
    assert abs(a_ - b_) < 1e-10


@pytest.mark.parametrize("mode", [O.SEPLLM, O.LAMBDA, O.SEGMENT])
def test_q_zero_closed_form(mode):
    d, m, P = 64, 260, 37
    v = rand(m + P, d)
    if mode == O.SEPLLM:
        spec = O.MaskSpec(mode, m, m, a=3, w=20, sep=(RNG.random(m) < 0.2).astype(np.uint8))
    elif mode == O.LAMBDA:
        spec = O.MaskSpec(mode, m, m, n_s=5, L=30)
    else:
        spec = O.MaskSpec(mode, m, m + P, P=P)
    vv = v[: spec.n_k]
    q = np.zeros((m, d))
    k = rand(spec.n_k, d)
    o, lse = O.attention_fast(q, k, vv, spec, 10000.0, 0.125)
    cnt = O.pair_counts(spec)
    np.testing.assert_allclose(lse, np.log(cnt), rtol=0, atol=1e-13)
    # O_i is the plain mean of the visible values; checked with a cumulative sum for the
    # contiguous masks and by direct means otherwise
    mask = O.mask_rows(spec, range(m))
    ref = (mask.astype(np.float64) @ vv) / cnt[:, None]
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    o2, lse2 = O.q0_closed_form(vv, spec, range(m))
    np.testing.assert_allclose(o2, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2, np.log(cnt), rtol=0, atol=1e-13)


def test_gqa_mapping():
    d, m = 32, 64
    Q, K, V = rand(4, m, d), rand(2, m, d), rand(2, m, d)
    spec = O.MaskSpec(O.LAMBDA, m, m, n_s=2, L=10)
    o, _ = O.attention(Q, K, V, spec, 10000.0, 0.2)
    for h in range(4):
        ref, _ = O.attention_fast(Q[h], K[h // 2], V[h // 2], spec, 10000.0, 0.2)
        np.testing.assert_array_equal(o[h], ref)


# ---------------------------------------------------------------------------
# plan
# ---------------------------------------------------------------------------

def _check_plan(spec):
    pl = O.plan(spec)
    n_tiles, n_blocks = pl["n_tiles"], pl["n_blocks"]
    assert n_tiles == -(-spec.n_q // 128) and n_blocks == -(-spec.n_k // 64)
    tp, items = pl["tile_ptr"], pl["items"]
    assert tp[0] == 0 and tp[-1] == len(items) and np.all(np.diff(tp) >= 0)
    flags = spec.sep_flags()
    if spec.mode == O.SEPLLM:
        g0 = 64 * (-(-spec.a // 64))
        np.testing.assert_array_equal(pl["sep_idx"], np.flatnonzero(flags[g0:]) + g0)
        padded = np.zeros(n_blocks * 64, np.uint8)
        padded[: spec.n_k] = flags
        words = np.packbits(padded.reshape(n_blocks, 64), axis=1, bitorder="little")
        np.testing.assert_array_equal(pl["sep_bits"], words.view("<u8").reshape(n_blocks))
    for t in range(n_tiles):
        q0, q1 = 128 * t, min(spec.n_q, 128 * t + 128) - 1
        rows = np.arange(q0, q1 + 1)
        blocks = items[tp[t]:tp[t + 1]] & 0xFFFFFF
        fl = items[tp[t]:tp[t + 1]] >> 24
        assert np.all(np.diff(blocks) > 0)
        covered = np.zeros((len(rows), spec.n_k), np.int64)
        seps = pl["sep_idx"][: pl["sep_count"][t]]
        covered[:, seps] += 1
        vis = O.mask_rows(spec, rows)
        # gathered separators are visible to every query of the tile
        assert vis[:, seps].all()
        for b, f in zip(blocks, fl):
            j = np.arange(64 * b, min(spec.n_k, 64 * b + 64))
            covered[:, j] += vis[:, j]
            assert bool(f & O.FLAG_FULL) == (64 * b + 64 <= spec.n_k and bool(vis[:, j].all()))
            cap = (vis[:, j] & (rows[:, None] - j[None, :] > spec.L)) if spec.mode == O.LAMBDA \
                else np.zeros((1, 1), bool)
            assert bool(f & O.FLAG_CAPPED) == bool(cap.any())
            assert vis[:, j].any()
        # coverage identity: each visible pair exactly once, no invisible pair
        np.testing.assert_array_equal(covered, vis.astype(np.int64))
    return pl


@pytest.mark.parametrize("seed", range(6))
def test_plan_coverage_random(seed):
    r = np.random.default_rng(seed)
    m = int(r.integers(1, 700))
    for mode in (O.SEPLLM, O.LAMBDA, O.SEGMENT):
        if mode == O.SEPLLM:
            flags = (r.random(m) < r.choice([0.0, 0.05, 0.3, 1.0])).astype(np.uint8)
            spec = O.MaskSpec(mode, m, m, a=int(r.integers(0, 150)), w=int(r.integers(1, 400)),
                              sep=flags)
        elif mode == O.LAMBDA:
            spec = O.MaskSpec(mode, m, m, n_s=int(r.integers(0, 150)), L=int(r.integers(0, 400)))
        else:
            P = int(r.integers(0, 300))
            spec = O.MaskSpec(mode, m, m + P, P=P)
        _check_plan(spec)


def test_plan_small_configs_shape():
    # workload-1 shape (m=512, a=4, w=64): 4 tiles, 8 blocks
    flags = (RNG.random(512) < 0.1).astype(np.uint8)
    pl = _check_plan(O.MaskSpec(O.SEPLLM, 512, 512, a=4, w=64, sep=flags))
    assert pl["n_tiles"] == 4 and pl["n_blocks"] == 8
    # segment with S=256, P=64: tile t visits blocks 0 .. floor((P + q1)/64)
    pl = _check_plan(O.MaskSpec(O.SEGMENT, 256, 320, P=64))
    assert (np.diff(pl["tile_ptr"]) == [3, 5]).all()


# ---------------------------------------------------------------------------
# top-k retrieval
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_topk_scores_chain_and_error_bound(dt):
    # with bf16 inputs the fp64 chain is usually exact; fp32 inputs make the order visible
    d, n = 128, 50
    q = torch.randn(d).to(dt).double().numpy()
    k = torch.randn(n, d).to(dt).double().numpy()
    s = O.topk_scores(q, k)
    for j in range(n):
        acc = 0.0
        for c in range(d):
            acc = acc + float(q[c]) * float(k[j, c])
        assert acc == s[j]
        exact = sum(Fraction(float(q[c])) * Fraction(float(k[j, c])) for c in range(d))
        bound = d * 2.0 ** -53 * float(sum(abs(Fraction(float(q[c])) * Fraction(float(k[j, c])))
                                           for c in range(d)))
        assert abs(float(exact - Fraction(s[j]))) <= bound


def test_topk_select_rules():
    n = 1000
    s = RNG.standard_normal(n)
    s[::7] = 0.5  # many ties
    for k in (1, 10, 300, n):
        idx = O.topk_select(s, k)
        ref = sorted(j for _, j in heapq.nlargest(k, ((v, -j) for j, v in enumerate(s))))
        ref = sorted(-j for j in ref)
        assert idx.tolist() == ref
    assert O.topk_select(s, n).tolist() == list(range(n))
    assert O.topk_select(s, 1)[0] == int(np.argmax(s))
    # ties: all equal -> the lowest indices
    assert O.topk_select(np.zeros(50), 5).tolist() == [0, 1, 2, 3, 4]
    assert O.topk_select(np.array([0.0, -0.0, 0.0, -1.0]), 2).tolist() == [0, 1]


# ---------------------------------------------------------------------------
# ALiBi bias clipped at L (LM-Infinite page, section 方法)
# ---------------------------------------------------------------------------

def test_alibi_slopes_textbook():
    # the geometric ALiBi slopes: for 8 heads 1/2, 1/4, ..., 1/256
    assert [O.alibi_slope(h, 8, 8.0) for h in range(8)] == [2.0 ** -(h + 1) for h in range(8)]
    s16 = [O.alibi_slope(h, 16, 8.0) for h in range(16)]
    assert s16[-1] == 2.0 ** -8
    np.testing.assert_allclose(np.array(s16[1:]) / np.array(s16[:-1]), 2.0 ** -0.5, rtol=1e-15)


@pytest.mark.parametrize("n_s,L", [(5, 199), (0, 31)])
def test_alibi_without_cap_vs_sdpa(n_s, L):
    # no visible pair has i - j > L (full causal, or a pure window), so the bias is the
    # textbook ALiBi -m (i - j), built here by torch as an additive SDPA mask
    d, m, slope = 64, 200, 0.0625
    scale = 1.0 / math.sqrt(d)
    q, k, v = rand(m, d), rand(m, d), rand(m, d)
    ar = torch.arange(m)
    dist = (ar[:, None] - ar[None, :]).to(torch.float64)
    keep = (dist >= 0) & (dist <= L)
    bias = torch.where(keep, -slope * dist, torch.tensor(-math.inf, dtype=torch.float64))
    tq, tk = torch.from_numpy(q), torch.from_numpy(k)
    ref = sdpa(tq, tk, torch.from_numpy(v), bias, scale).numpy()
    ref_lse = torch.logsumexp(tq @ tk.T * scale + bias, dim=1).numpy()
    spec = O.MaskSpec(O.LAMBDA, m, m, n_s=n_s, L=L)
    o, lse = O.attention_fast(q, k, v, spec, None, scale, alibi=slope)
    o2, lse2 = O.attention_rows(q, k, v, range(m), spec, None, scale, slope)
    for a, b in ((o, ref), (o2, ref), (lse, ref_lse), (lse2, ref_lse)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n_s,L,slope", [(5, 30, 0.05), (12, 7, 0.3), (3, 64, 2.0 ** -8)])
def test_alibi_q_zero_closed_form(n_s, L, slope):
    # Q = 0: logit of key j is -m min(i-j, L).  Partition function: the window keys at
    # distances 0..W give a geometric series, each starting-span key beyond the window
    # gives e^{-mL}.  Value columns that mark one distance class read that class's weight.
    d, m = 16, 260
    spec = O.MaskSpec(O.LAMBDA, m, m, n_s=n_s, L=L)
    q, k = np.zeros((m, d)), rand(m, d)
    v = rand(m, d)
    i = np.arange(m)
    W = np.minimum(i, L)
    n_far = np.minimum(n_s, np.maximum(0, i - L))
    Z = np.array([sum(math.exp(-slope * t) for t in range(w + 1)) for w in W]) \
        + n_far * math.exp(-slope * L)
    # column 0: keys beyond the window (all in the starting span); column 1: j == i;
    # column 2: the key at distance exactly L
    vf = v.copy()
    v[:, :3] = 0.0
    o_parts = []
    for r in range(m):
        vr = v.copy()
        vr[: max(0, r - L), 0] = 1.0
        vr[r, 1] = 1.0
        if r >= L:
            vr[r - L, 2] = 1.0
        o_r, l_r = O.attention_rows(q, k, vr, [r], spec, None, 0.1, slope)
        o_parts.append((o_r[0], l_r[0]))
    o = np.array([p[0] for p in o_parts])
    lse = np.array([p[1] for p in o_parts])
    np.testing.assert_allclose(lse, np.log(Z), rtol=0, atol=1e-13)
    np.testing.assert_allclose(o[:, 0], n_far * math.exp(-slope * L) / Z, rtol=0, atol=1e-15)
    np.testing.assert_allclose(o[:, 1], 1.0 / Z, rtol=0, atol=1e-15)
    np.testing.assert_allclose(o[:, 2], np.where(i >= L, math.exp(-slope * L), 0.0) / Z,
                               rtol=0, atol=1e-15)
    # the helper's closed form and the fast mode agree with the definition
    o_cf, l_cf = O.q0_alibi_closed_form(vf, spec, range(m), slope)
    o_f, l_f = O.attention_fast(q, k, vf, spec, None, 0.1, alibi=slope)
    o_d, l_d = O.attention_rows(q, k, vf, range(m), spec, None, 0.1, slope)
    np.testing.assert_allclose(l_cf, np.log(Z), rtol=0, atol=1e-13)
    for a, b in ((o_f, o_d), (o_cf, o_d), (l_f, l_d)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_alibi_steep_slope_keeps_the_diagonal():
    # with m = 60 every key but j = i is suppressed by e^{-60} or less
    d, m = 32, 150
    q, k, v = rand(m, d), rand(m, d), rand(m, d)
    spec = O.MaskSpec(O.LAMBDA, m, m, n_s=4, L=20)
    o, lse = O.attention_fast(q, k, v, spec, None, 0.05, alibi=60.0)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, 0.05 * np.einsum("id,id->i", q, k), rtol=0, atol=1e-14)


def test_alibi_heads_use_their_slopes():
    d, m = 32, 140
    Q, K, V = rand(8, m, d), rand(2, m, d), rand(2, m, d)
    spec = O.MaskSpec(O.LAMBDA, m, m, n_s=3, L=40)
    o, lse = O.attention(Q, K, V, spec, None, 0.2, alibi_exp=8.0)
    for h in (0, 5, 7):
        o_h, l_h = O.attention_rows(Q[h], K[h // 4], V[h // 4], range(m), spec, None, 0.2,
                                    2.0 ** -(h + 1))
        np.testing.assert_allclose(o[h], o_h, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[h], l_h, rtol=0, atol=1e-12)
    with pytest.raises(ValueError):
        O.attention(Q, K, V, spec, 10000.0, 0.2, alibi_exp=8.0)


# ---------------------------------------------------------------------------
# several segments end to end (segmented-execution page, method / overall framework)
# ---------------------------------------------------------------------------

def _py_chain(q, k):
    acc = 0.0
    for c in range(len(q)):
        acc = acc + float(q[c]) * float(k[c])
    return acc


@pytest.mark.parametrize("S,M", [(150, 100), (60, 100)])
def test_segmented_run_against_history(S, M):
    # Everything a segment reads is stated here in terms of the whole history of raw
    # projections: local heads see the latest M history rows, long heads the top-M history
    # rows by the previous segment's last query, both at positions 0..P-1 before the
    # segment at P..P+S-1 (causal), checked with torch SDPA on explicitly rotated inputs.
    H, nl, d, N, base = 4, 2, 32, 3, 10000.0
    scale = 1.0 / math.sqrt(d)
    Qs = [torch.randn(H, S, d, dtype=torch.float64).to(torch.bfloat16).double().numpy() for _ in range(N)]
    Ks = [torch.randn(H, S, d, dtype=torch.float64).to(torch.bfloat16).double().numpy() for _ in range(N)]
    Vs = [torch.randn(H, S, d, dtype=torch.float64).numpy() for _ in range(N)]
    out, state = O.segmented_run(Qs, Ks, Vs, nl, M, M, base, scale)
    K_all = np.concatenate(Ks, axis=1)
    V_all = np.concatenate(Vs, axis=1)
    # final state: the last M rows of the local heads' history; the whole long-head history
    keep = min(M, N * S)
    np.testing.assert_array_equal(state["tail_k"], K_all[:nl, N * S - keep:])
    np.testing.assert_array_equal(state["tail_v"], V_all[:nl, N * S - keep:])
    np.testing.assert_array_equal(state["pool_k"], K_all[nl:])
    np.testing.assert_array_equal(state["pool_v"], V_all[nl:])
    for i in range(N):
        seg = out[i]
        hist = i * S
        P = min(M, hist)
        assert seg["P"] == P
        if i == 0:
            assert seg["idx"] is None
        for h in range(H):
            if h < nl or i == 0:
                pk, pv = K_all[h, hist - P:hist], V_all[h, hist - P:hist]
            else:
                j = h - nl
                scores = [_py_chain(Qs[i - 1][h, S - 1], K_all[h, r]) for r in range(hist)]
                top = heapq.nlargest(P, range(hist), key=lambda r: (scores[r], -r))
                assert seg["idx"][j].tolist() == sorted(top)
                pk, pv = K_all[h, sorted(top)], V_all[h, sorted(top)]
            kc = np.concatenate([pk, Ks[i][h]])
            vc = np.concatenate([pv, Vs[i][h]])
            qr = complex_rope(torch.from_numpy(Qs[i][h]), torch.arange(P, P + S), base)
            kr = complex_rope(torch.from_numpy(kc), torch.arange(P + S), base)
            mask = torch.ones(S, P + S, dtype=torch.bool).tril(P)
            ref = sdpa(qr, kr, torch.from_numpy(vc), mask, scale).numpy()
            np.testing.assert_allclose(seg["O"][h], ref, rtol=0, atol=1e-12)
    with pytest.raises(ValueError):
        O.segmented_run(Qs, Ks, Vs, nl, M, M + 1, base, scale)


# ---------------------------------------------------------------------------
# backward (gradients of O)
# ---------------------------------------------------------------------------

def _torch_rot_angles(pos, d, base):
    inv = 1.0 / (base ** (torch.arange(0, d, 2, dtype=torch.float64) / d))
    return pos.to(torch.float64)[:, None] * inv[None, :]


def _torch_rotate(x, ang):
    """rotate-half RoPE applied with per-row angles ang [n, d/2] (autograd-friendly)."""
    h = x.shape[-1] // 2
    c, s = torch.cos(ang), torch.sin(ang)
    return torch.cat([x[..., :h] * c - x[..., h:] * s, x[..., h:] * c + x[..., :h] * s], dim=-1)


def _torch_masked_attention(q, k, v, logits_fn, mask):
    s = logits_fn(q, k).masked_fill(~mask, -math.inf)
    return torch.softmax(s, dim=-1) @ v


@pytest.mark.parametrize("case", ["sepllm", "segment", "lambda_capped", "alibi_capped", "gqa"])
def test_backward_vs_torch_autograd(case):
    # the forward is built here from torch primitives (rotations, a boolean mask, softmax) and
    # differentiated by torch.autograd in fp64; the oracle's gradient formulas must agree
    d, m, base = 16, 150, 500.0
    scale = 1.0 / math.sqrt(d)
    h_q, h_kv = (4, 2) if case == "gqa" else (1, 1)
    P = 40 if case == "segment" else 0
    n_k = m + P
    Q = torch.randn(h_q, m, d, dtype=torch.float64)
    K = torch.randn(h_kv, n_k, d, dtype=torch.float64)
    V = torch.randn(h_kv, n_k, d, dtype=torch.float64)
    dO = torch.randn(h_q, m, d, dtype=torch.float64)
    i = torch.arange(m)[:, None] + P
    j = torch.arange(n_k)[None, :]
    rope, slope_exp = base, None
    if case in ("sepllm", "gqa"):
        flags = (RNG.random(n_k) < 0.15).astype(np.uint8)
        spec = O.MaskSpec(O.SEPLLM, m, n_k, a=3, w=20, sep=flags)
        mask = (j <= i) & ((j < 3) | (i - j < 20) | torch.from_numpy(flags).bool()[None, :])
    elif case == "segment":
        spec = O.MaskSpec(O.SEGMENT, m, n_k, P=P)
        mask = j <= i
    else:
        spec = O.MaskSpec(O.LAMBDA, m, n_k, n_s=6, L=25)
        mask = (j <= i) & ((j < 6) | (i - j <= 25))
        if case == "alibi_capped":
            rope, slope_exp = None, 2.0
    capped = mask & (i - j > 25) if case in ("lambda_capped", "alibi_capped") else torch.zeros_like(mask)
    Qg, Kg, Vg = (t.clone().requires_grad_(True) for t in (Q, K, V))
    outs = []
    for h in range(h_q):
        g = h // (h_q // h_kv)
        qh, kh, vh = Qg[h], Kg[g], Vg[g]
        if rope:
            qr = _torch_rotate(qh, _torch_rot_angles(torch.arange(P, P + m), d, base))
            kr = _torch_rotate(kh, _torch_rot_angles(torch.arange(n_k), d, base))
            qcap = _torch_rotate(qh, _torch_rot_angles(torch.full((m,), 25), d, base))
            fn = lambda a, b: torch.where(capped, scale * (qcap @ kh.T), scale * (qr @ kr.T))  # noqa: E731
        else:
            slope = 2.0 ** (-slope_exp * (h + 1) / h_q) if slope_exp else 0.0
            dist = torch.clamp(i - j, max=25).to(torch.float64) if slope_exp else 0.0
            fn = lambda a, b, s_=slope, d_=dist: scale * (a @ b.T) - s_ * d_  # noqa: E731
        outs.append(_torch_masked_attention(qh, kh, vh, fn, mask))
    (torch.stack(outs) * dO).sum().backward()
    dq, dk, dv = O.attention_backward(Q.numpy(), K.numpy(), V.numpy(), dO.numpy(), spec, rope, scale,
                                      alibi_exp=slope_exp)
    np.testing.assert_allclose(dq, Qg.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, Kg.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, Vg.grad.numpy(), rtol=0, atol=1e-11)


def test_backward_capped_finite_differences():
    # central differences of <dO, O> through the oracle's (pinned) definition-mode forward
    d, m = 8, 60
    spec = O.MaskSpec(O.LAMBDA, m, m, n_s=4, L=10)
    q, k, v, do = (RNG.standard_normal((m, d)) for _ in range(4))
    dq, dk, dv = O.attention_grad_rows(q, k, v, do, range(m), spec, 100.0, 0.3)

    def f(q_, k_, v_):
        o, _ = O.attention_rows(q_, k_, v_, range(m), spec, 100.0, 0.3)
        return float((o * do).sum())
    eps = 1e-6
    for name, g in (("q", dq), ("k", dk), ("v", dv)):
        for a, b in [(3, 1), (17, 5), (40, 0), (59, 7), (0, 2)]:
            args = {"q_": q.copy(), "k_": k.copy(), "v_": v.copy()}
            args[name + "_"][a, b] += eps
            fp = f(**args)
            args[name + "_"][a, b] -= 2 * eps
            fm = f(**args)
            assert abs((fp - fm) / (2 * eps) - g[a, b]) < 1e-7, (name, a, b)


# ---------------------------------------------------------------------------
# streaming decode with the four-part cache (SepLLM page, part 6.2, generation)
# ---------------------------------------------------------------------------

def test_stream_cache_hand_trace():
    g = json.load(open(os.path.join(GOLDEN, "stream_cache_hand.json")))
    sc = O.StreamCache(g["a"], g["s"], g["w"], g["c"])
    for t, f in enumerate(g["flags"]):
        sc.append(bool(f))
        assert sc.tokens().tolist() == g["tokens_after_step"][t], t
        assert sc.run_size == g["run_size_after_step"][t], t
        assert O.stream_cache_tokens(t, np.array(g["flags"]), g["a"], g["s"], g["w"], g["c"]).tolist() \
            == g["tokens_after_step"][t]


@pytest.mark.parametrize("a,s,w,c,p", [(4, 64, 128, 324, 0.1), (4, 8, 16, 40, 0.6), (0, 1, 1, 3, 0.5),
                                       (2, 3, 5, 20, 0.0), (3, 4, 6, 30, 1.0)])
def test_stream_cache_closed_form_and_occupancy(a, s, w, c, p):
    n = 2500
    flags = (RNG.random(n) < p).astype(np.uint8)
    sc = O.StreamCache(a, s, w, c)
    P = c - a - s - w
    sizes = []
    for t in range(n):
        sc.append(bool(flags[t]))
        np.testing.assert_array_equal(sc.tokens(), O.stream_cache_tokens(t, flags, a, s, w, c))
        assert sc.run_size <= c
        sizes.append(sc.run_size)
    # after the warm-up the run size cycles a+s+w .. c-1: its mean over whole periods is
    # a+s+w+(P-1)/2, under the page's bound (w+c+a+s)/2
    t0 = a + w + P  # first compression
    m = (n - t0) // P * P
    mean = float(np.mean(sizes[t0:t0 + m]))
    assert mean == pytest.approx(a + s + w + (P - 1) / 2) and mean < (w + c + a + s) / 2


def test_decode_attention_vs_sdpa():
    d, n, base = 32, 400, 10000.0
    a, s, w, c = 4, 8, 16, 60
    flags = (RNG.random(n) < 0.3).astype(np.uint8)
    q, k, v = rand(n, d), rand(n, d), rand(n, d)
    scale = d ** -0.5
    for t in (0, 3, 20, 57, 150, 399):
        toks = O.stream_cache_tokens(t, flags, a, s, w, c)
        o, lse = O.decode_attention(q[t], k[:t + 1], v[:t + 1], t, toks, base, scale)
        qr = complex_rope(torch.from_numpy(q[t:t + 1]), torch.tensor([t]), base)
        kr = complex_rope(torch.from_numpy(k[:t + 1]), torch.arange(t + 1), base)
        mask = torch.zeros(1, t + 1, dtype=torch.bool)
        mask[0, torch.from_numpy(toks)] = True
        ref = sdpa(qr, kr, torch.from_numpy(v[:t + 1]), mask, scale).numpy()[0]
        np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
        ref_l = torch.logsumexp((qr @ kr.T * scale).masked_fill(~mask, -math.inf), dim=1).item()
        assert abs(lse - ref_l) < 1e-12


# ---------------------------------------------------------------------------
# LM-Infinite top-k middle tokens (LM-Infinite page, section 方法)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("base", [None, 10000.0])
def test_topk_middle_all_selected_is_capped_causal(base):
    # with k at least the middle size every j <= i is attended, each at min(i-j, L): the
    # page's capped realisation over the whole causal mask, built here in torch
    d, m, n_s, L = 32, 160, 5, 20
    scale = d ** -0.5
    q, k, v = rand(m, d), rand(m, d), rand(m, d)
    spec = O.MaskSpec(O.LAMBDA, m, m, n_s=n_s, L=L)
    o, lse, _ = O.attention_topk_middle(q, k, v, range(m), spec, base, scale, k_mid=m)
    tq, tk = torch.from_numpy(q), torch.from_numpy(k)
    i = torch.arange(m)[:, None]
    j = torch.arange(m)[None, :]
    if base:
        qr = complex_rope(tq, torch.arange(m), base)
        kr = complex_rope(tk, torch.arange(m), base)
        qL = complex_rope(tq, torch.full((m,), L), base)
        logits = torch.where(i - j > L, scale * (qL @ tk.T), scale * (qr @ kr.T))
    else:
        logits = scale * (tq @ tk.T)
    logits = logits.masked_fill(j > i, -math.inf)
    ref = torch.softmax(logits, dim=1) @ torch.from_numpy(v)
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, torch.logsumexp(logits, dim=1).numpy(), rtol=0, atol=1e-12)


def test_topk_middle_selection_brute_force():
    # the selected set is heapq's k largest of a pure-Python score list (lower index on ties),
    # k = 0 leaves the Lambda attention unchanged
    d, m, n_s, L, kk = 8, 90, 3, 10, 4
    q = np.round(rand(m, d) * 4) / 4  # coarse values: exact ties occur
    k = np.round(rand(m, d) * 4) / 4
    v = rand(m, d)
    spec = O.MaskSpec(O.LAMBDA, m, m, n_s=n_s, L=L)
    _, _, sels = O.attention_topk_middle(q, k, v, range(m), spec, None, 1.0, kk)
    for i in range(m):
        cand = list(range(n_s, max(n_s, i - L)))
        sc = {j: sum(float(q[i, c]) * float(k[j, c]) for c in range(d)) for j in cand}
        best = sorted(heapq.nlargest(kk, cand, key=lambda j: (sc[j], -j)))
        assert sels[i].tolist() == best, i
    o0, l0, _ = O.attention_topk_middle(q, k, v, range(m), spec, 10000.0, 0.3, 0)
    o1, l1 = O.attention_rows(q, k, v, range(m), spec, 10000.0, 0.3)
    np.testing.assert_allclose(o0, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l0, l1, rtol=0, atol=1e-12)


@pytest.mark.parametrize("case", ["sepllm", "lambda_capped", "alibi_capped", "segment", "sepllm_norope"])
def test_grad_keys_fast_equals_definition_mode(case):
    # the tile-wise gradient of chosen keys (absolute rotations, capped pairs through the
    # page's realisation <R(L) q, k>) against the per-row definition mode, itself pinned by
    # torch.autograd and central differences above; every key and its rows, and a subset of
    # keys over a subset of rows that spans several tiles
    d, m, base = 16, 300, 500.0
    scale = 1.0 / math.sqrt(d)
    P = 40 if case == "segment" else 0
    n_k = m + P
    rope, slope = base, None
    if case.startswith("sepllm"):
        flags = (RNG.random(n_k) < 0.15).astype(np.uint8)
        spec = O.MaskSpec(O.SEPLLM, m, n_k, a=3, w=20, sep=flags)
        if case == "sepllm_norope":
            rope = None
    elif case == "segment":
        spec = O.MaskSpec(O.SEGMENT, m, n_k, P=P)
    else:
        spec = O.MaskSpec(O.LAMBDA, m, n_k, n_s=6, L=25)
        if case == "alibi_capped":
            rope, slope = None, 0.2
    q, do = (RNG.standard_normal((m, d)) for _ in range(2))
    k, v = (RNG.standard_normal((n_k, d)) for _ in range(2))
    _, rk, rv = O.attention_grad_rows(q, k, v, do, range(m), spec, rope, scale, slope)
    fk, fv = O.attention_grad_keys_fast(q, k, v, do, spec, rope, scale, np.arange(n_k), np.arange(m), slope)
    np.testing.assert_allclose(fk, rk, rtol=0, atol=1e-12 * max(1.0, np.abs(rk).max()))
    np.testing.assert_allclose(fv, rv, rtol=0, atol=1e-12 * max(1.0, np.abs(rv).max()))
    keys = np.array([0, 2, 5, 64, 65, 130, n_k - 1])
    rows = np.arange(100, m)
    _, rk2, rv2 = O.attention_grad_rows(q, k, v, do, rows, spec, rope, scale, slope)
    fk2, fv2 = O.attention_grad_keys_fast(q, k, v, do, spec, rope, scale, keys, rows, slope)
    np.testing.assert_allclose(fk2, rk2[keys], rtol=0, atol=1e-12 * max(1.0, np.abs(rk2).max()))
    np.testing.assert_allclose(fv2, rv2[keys], rtol=0, atol=1e-12 * max(1.0, np.abs(rv2).max()))
