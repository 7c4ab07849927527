"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Plans and index lists must match bit for bit.  Outputs must be within
max-abs 1e-2 / mean-abs 1e-3 for bf16 inputs and max-abs 1e-5 for fp32.
Small cases are compared in full; the five workloads at their real sizes are
compared on every row of the first and last two tiles plus random rows.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from _helpers import (compare, device_mask, log, logit_bound, oracle_rows, sample_rows, spec_of,
                      to64)
from _softmax_model import replay, spike_queries

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import structured_sparse_attention_attn_amd as m
    return m


def _plan_compare(sa, wl, sep_cpu):
    sa_obj = device_mask(wl, None if sep_cpu is None else sep_cpu.cuda())
    sa_obj.build_plan()
    torch.cuda.synchronize()
    got = sa.plan_to_host(sa_obj.mask, sa_obj.plan)
    ref = O.plan(spec_of(wl, None if sep_cpu is None else sep_cpu.numpy()))
    hdr = got["header"]
    assert hdr.magic == 0x31504153 and hdr.n_items == len(ref["items"])
    assert hdr.n_sep == len(ref["sep_idx"])
    for key in ("tile_ptr", "items", "sep_count", "sep_idx", "sep_bits"):
        np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
    return sa_obj, got


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_plan_bitexact_workloads(sa, cid):
    wl = W.WORKLOADS[cid]
    log(f"plan workload {cid}")
    sep = W.sep_flags(wl.n_k, wl.p_sep, wl.seed + 7) if wl.mode == W.SEPLLM else None
    _plan_compare(sa, wl, sep)


def _random_masks():
    r = np.random.default_rng(7)
    out = []
    for m in [1, 2, 63, 64, 65, 127, 128, 129, 700, 1000]:
        for kind in (W.SEPLLM, W.LAMBDA, W.SEGMENT):
            if kind == W.SEPLLM:
                a = int(r.choice([0, 1, 4, 63, 64, 65, 200]))
                w = int(r.choice([1, 2, 63, 64, 100, 5000]))
                p = float(r.choice([0.0, 0.05, 0.5, 1.0]))
                out.append((W.small(kind, seed=int(r.integers(1 << 30)), m=m, a=a, w=w, p_sep=p), p))
            elif kind == W.LAMBDA:
                out.append((W.small(kind, seed=1, m=m, n_s=int(r.choice([0, 1, 10, 64, 100])),
                                    L=int(r.choice([0, 1, 63, 64, 300, 5000]))), None))
            else:
                out.append((W.small(kind, seed=1, m=m, P=int(r.choice([0, 1, 64, 200]))), None))
    return out


def test_plan_bitexact_random(sa):
    for wl, p in _random_masks():
        sep = W.sep_flags(wl.n_k, p, wl.seed + 7) if wl.mode == W.SEPLLM else None
        _plan_compare(sa, wl, sep)


def _run_small(sa, wl, *, strided=False, q_zero=False, check_canary=False, qmul=1.0, vmul=1.0,
               spike=None, expect=()):
    """Runs one small case through the C ABI and compares it with the oracle in full.

    qmul / vmul scale q and v (powers of 2: exact in bf16); spike lists rows whose query is
    replaced by one aimed at a single visible key with a logit of 150 natural units
    (spike_queries).  expect names flags of the CPU replay of the kernel's softmax update
    rule that these inputs must raise (e.g. "rescale", "recompute"), so the test is known to
    reach those branches.  With qmul or spike the LSE bar widens with the logit magnitude:
    2e-2 + 2^-8 * logit_bound (the bf16 rounding of the rotated q and k)."""
    inp = W.make_small_inputs(wl)
    q, k, v = inp["q"], inp["k"], inp["v"]
    if q_zero:
        q = torch.zeros_like(q)
    sep = inp.get("sep")
    if qmul != 1.0:
        q = (q.float() * qmul).to(q.dtype)
    if vmul != 1.0:
        v = (v.float() * vmul).to(v.dtype)
    slope_of = (lambda h: O.alibi_slope(h, wl.h_q, wl.alibi_exp)) if wl.alibi_exp else None
    if spike is not None:
        spec0 = spec_of(wl, None if sep is None else sep.numpy())
        q = torch.from_numpy(spike_queries(to64(q), to64(k), spec0, spike, 150.0, wl.scale,
                                           rope_base=wl.rope_base, slope=slope_of, h_q=wl.h_q,
                                           h_kv=wl.h_kv)).to(q.dtype)
    if expect:
        spec0 = spec_of(wl, None if sep is None else sep.numpy())
        flags, _ = replay(to64(q[0, 0]), to64(k[0, 0]), spec0, wl.rope_base, wl.scale,
                          slope=slope_of(0) if slope_of else None)
        for f in expect:
            assert flags[f], f"the inputs do not reach the '{f}' branch"
    dev = "cuda"
    if strided:
        # [B,T,H,d] storage viewed as [B,H,T,d]
        qd = q.permute(0, 2, 1, 3).contiguous().to(dev).permute(0, 2, 1, 3)
        kd = k.permute(0, 2, 1, 3).contiguous().to(dev).permute(0, 2, 1, 3)
        vd = v.permute(0, 2, 1, 3).contiguous().to(dev).permute(0, 2, 1, 3)
    else:
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    sa_obj = device_mask(wl, None if sep is None else sep.to(dev))
    sa_obj.build_plan()
    guard = 4096
    o_store = torch.full((guard * 2 + q.numel(),), 7.0, dtype=q.dtype, device=dev)
    o = o_store[guard:guard + q.numel()].view(q.shape)
    lse = torch.full((wl.batch, wl.h_q, wl.n_q), 7.0, dtype=torch.float32, device=dev)
    sa_obj.forward(qd, kd, vd, o=o, lse=lse, rope_base=wl.rope_base, scale=wl.scale,
                   alibi_exp=wl.alibi_exp)
    torch.cuda.synchronize()
    if check_canary:
        assert torch.all(o_store[:guard] == 7.0) and torch.all(o_store[-guard:] == 7.0)
    spec = spec_of(wl, None if sep is None else sep.numpy())
    cnt = O.pair_counts(spec)
    for b in range(wl.batch):
        Q, K, V = to64(q[b]), to64(k[b]), to64(v[b])
        ref_o, ref_l = O.attention(Q, K, V, spec, wl.rope_base, wl.scale, alibi_exp=wl.alibi_exp)
        lse_tol = None
        if qmul != 1.0 or spike is not None:
            lse_tol = 2e-2 + 2.0 ** -8 * logit_bound(Q, K, spec, wl.scale, np.arange(wl.n_q))
        assert np.isfinite(to64(o[b])).all() and np.isfinite(to64(lse[b])).all()
        compare(to64(o[b]), ref_o, to64(lse[b]), ref_l, wl.dtype, lse_tol=lse_tol)
        if q_zero and wl.alibi_exp is None:
            np.testing.assert_allclose(to64(lse[b]), np.broadcast_to(np.log(cnt), ref_l.shape),
                                       rtol=0, atol=2e-6)
        elif q_zero:
            # the closed-form partition function of the clipped bias (geometric series).
            # fp32: the bias carries a relative error of ~2^-24.  bf16: the sum is taken over
            # the bf16-rounded weights (relative error <= 2^-9 each), so
            # |d LSE| <= -ln(1 - 2^-9) < 2e-3.
            tol = 2e-3 if wl.dtype == "bf16" else 2e-5
            for h in range(wl.h_q):
                _, l_cf = O.q0_alibi_closed_form(V[h // (wl.h_q // wl.h_kv)], spec,
                                                 range(wl.n_q), O.alibi_slope(h, wl.h_q, wl.alibi_exp))
                np.testing.assert_allclose(to64(lse[b, h]), l_cf, rtol=0, atol=tol)
    return o, lse


SMALL = [
    # (mode, kwargs)
    (W.SEPLLM, dict(m=700, a=4, w=64, p_sep=0.1)),
    (W.SEPLLM, dict(m=700, a=70, w=100, p_sep=0.2, h_q=4, h_kv=2)),
    (W.SEPLLM, dict(m=333, a=0, w=1, p_sep=0.3)),
    (W.SEPLLM, dict(m=257, a=4, w=5000, p_sep=0.0)),
    (W.SEPLLM, dict(m=500, a=200, w=17, p_sep=1.0, batch=2)),
    (W.SEPLLM, dict(m=1, a=4, w=64, p_sep=0.5)),
    (W.LAMBDA, dict(m=900, n_s=10, L=300)),
    (W.LAMBDA, dict(m=700, n_s=0, L=100, h_q=4, h_kv=1)),
    (W.LAMBDA, dict(m=600, n_s=100, L=64)),
    (W.LAMBDA, dict(m=300, n_s=10, L=0)),
    (W.LAMBDA, dict(m=300, n_s=5, L=5000)),
    (W.SEGMENT, dict(m=600, P=200)),
    (W.SEGMENT, dict(m=300, P=0)),
    (W.SEGMENT, dict(m=129, P=1, h_q=4, h_kv=2, batch=2)),
    (W.SEGMENT, dict(m=200, P=33000)),  # > 512 blocks per tile: items read from the plan directly
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", range(len(SMALL)))
def test_fwd_small(sa, case, dtype):
    mode, kw = SMALL[case]
    for rope in (10000.0, None):
        d = 128 if dtype == "bf16" else 64
        wl = W.small(mode, seed=100 + case, dtype=dtype, d=d, rope_base=rope, **kw)
        log(f"small {case} {dtype} rope={rope}")
        _run_small(sa, wl, check_canary=True)


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_fwd_small_bf16_d64(sa, case):
    """bf16 with 64-element heads (the Pythia-class shape): the same cases as above."""
    mode, kw = SMALL[case]
    for rope in (10000.0, None):
        wl = W.small(mode, seed=700 + case, dtype="bf16", d=64, rope_base=rope, **kw)
        log(f"small d64 {case} rope={rope}")
        _run_small(sa, wl, check_canary=True)


def test_fwd_bf16_d64_strided_and_alibi(sa):
    wl = W.small(W.SEPLLM, seed=730, d=64, m=700, a=70, w=100, p_sep=0.2, h_q=4, h_kv=2)
    _run_small(sa, wl, strided=True)
    for i, kw in enumerate(ALIBI_SMALL):
        wl = W.small(W.LAMBDA, seed=740 + i, d=64, rope_base=None, **kw)
        log(f"alibi d64 {i}")
        _run_small(sa, wl, check_canary=True)
    wl = W.small(W.LAMBDA, seed=760, d=64, m=640, n_s=10, L=100, rope_base=None, alibi_exp=8.0)
    _run_small(sa, wl, q_zero=True)


def test_fwd_f32_d128_and_strided(sa):
    wl = W.small(W.SEPLLM, seed=5, dtype="f32", d=128, m=300, a=4, w=50, p_sep=0.1)
    _run_small(sa, wl)
    wl = W.small(W.LAMBDA, seed=6, dtype="bf16", m=500, n_s=10, L=100, h_q=4, h_kv=2)
    _run_small(sa, wl, strided=True)


@pytest.mark.parametrize("mode", [W.SEPLLM, W.LAMBDA, W.SEGMENT])
def test_q_zero_counts(sa, mode):
    # Q = 0: every visible logit is 0, so LSE_i = ln |A_i| and O_i = mean of v over A_i
    kw = dict(m=640, a=4, w=64, p_sep=0.1) if mode == W.SEPLLM else (
        dict(m=640, n_s=10, L=100) if mode == W.LAMBDA else dict(m=640, P=100))
    wl = W.small(mode, seed=9, **kw)
    _run_small(sa, wl, q_zero=True)


def _ulp_bf16(x):
    """One bf16 ulp at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return np.ldexp(1.0, (np.floor(np.log2(ax)) - 7).astype(np.int64))


def _check_rotated(got, x, angle, factor, what):
    """got (bf16 rows) against the fp64 rotation of x by angle, times factor: within one bf16
    ulp of the exact value (the one rounding to bf16 takes half), plus 2^-18 of the pair's
    magnitude for the fp32 rotation and the hardware sine/cosine when the result cancels."""
    ref = O.rotate(x, angle) * factor
    h = x.shape[-1] // 2
    mag = (np.abs(x[..., :h]) + np.abs(x[..., h:])) * abs(factor)
    mag = np.concatenate([mag, mag], axis=-1)
    err = np.abs(got - ref)
    bound = _ulp_bf16(ref) + 2.0 ** -18 * mag
    bad = err > bound
    assert not bad.any(), (what, int(bad.sum()), float(err[bad].max()))


ROPE_CASES = [
    # (mode, kwargs, rope_base): positions up to 131071 with base 500000 (workload 5's keys,
    # one kv head), the 32K Lambda capped keys, a segment with a 1024-row prefix
    (W.SEPLLM, dict(m=131072, a=4, w=1024, p_sep=0.06, h_q=4, h_kv=1), 500000.0),
    (W.LAMBDA, dict(m=32768, n_s=10, L=4096, h_q=1, h_kv=1), 10000.0),
    (W.SEGMENT, dict(m=4096, P=1024, h_q=2, h_kv=2), 10000.0),
]


@pytest.mark.parametrize("case", range(len(ROPE_CASES)))
def test_rope_stage_direct(sa, case):
    """The RoPE stage alone (sparse_attn_rope), read back from the workspace sections the C
    ABI reports: rotated keys R(pos_k(j)) k_j (LM-Infinite page, section "method", and the
    segmented-execution page: positions 0..P-1 for the prefix), the capped keys
    R(-L) k_j * scale * log2(e) for j < n_starting, and the gathered separator rows, byte
    for byte the rotated key rows and raw value rows at SEP[r] (SepLLM page, part 6.2)."""
    mode, kw, base = ROPE_CASES[case]
    wl = W.small(mode, seed=600 + case, rope_base=base, **kw)
    log(f"rope stage {case}: n_k={wl.n_k}")
    inp = W.make_small_inputs(wl)
    sep = inp.get("sep")
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    sa_obj = device_mask(wl, None if sep is None else sep.cuda())
    sa_obj.build_plan()
    o = torch.empty_like(q)
    args = sa_obj.args(q, k, v, o, rope_base=base, scale=wl.scale)
    sa_obj.ensure_workspace(args)
    sa.sparse_attn_rope(sa_obj.mask, sa_obj.plan, args, sa_obj.ws)
    torch.cuda.synchronize()
    lay = sa.sa_fwd_workspace_layout(sa_obj.mask, args)
    ws = sa_obj.ws
    B, hkv, nk, d = wl.batch, wl.h_kv, wl.n_k, wl.d

    def section(off, rows):
        n = B * hkv * rows * d * 2
        return ws[off:off + n].view(torch.bfloat16).view(B, hkv, rows, d)

    spec = spec_of(wl, None if sep is None else sep.numpy())
    theta = O.rope_theta(d, base)
    krot = section(lay.krot, nk)
    pos = O.pos_k(spec, np.arange(nk)).astype(np.float64)
    for g in range(hkv):
        _check_rotated(to64(krot[0, g]), to64(k[0, g]), pos[:, None] * theta[None, :], 1.0, "krot")
    if mode == W.LAMBDA:
        assert lay.kcap >= 0 and lay.cap_rows >= wl.n_s
        kcap = section(lay.kcap, lay.cap_rows)
        fac = wl.scale / math.log(2.0)
        for g in range(hkv):
            _check_rotated(to64(kcap[0, g, :wl.n_s]), to64(k[0, g, :wl.n_s]),
                           np.full((wl.n_s, d // 2), -float(wl.L)) * theta[None, :], fac, "kcap")
    if mode == W.SEPLLM:
        pl = O.plan(spec)
        n_used = int(pl["sep_count"].max())
        assert n_used > 1000
        rows = torch.from_numpy(pl["sep_idx"][:n_used].astype(np.int64)).cuda()
        ksep = section(lay.ksep, lay.sep_rows)
        vsep = section(lay.vsep, lay.sep_rows)
        for g in range(hkv):
            assert torch.equal(ksep[0, g, :n_used], krot[0, g][rows])
            assert torch.equal(vsep[0, g, :n_used], v[0, g][rows])


# Inputs with a wide logit range (the bf16 forward's online softmax against a stale
# per-row reference; SepLLM page part 6.1, LM-Infinite page section "method").
WIDE = [
    (W.SEPLLM, dict(m=700, a=4, w=64, p_sep=0.1, h_q=4, h_kv=2), 10000.0, None),
    (W.LAMBDA, dict(m=900, n_s=10, L=100), 10000.0, None),
    (W.SEGMENT, dict(m=600, P=200), 10000.0, None),
    (W.LAMBDA, dict(m=900, n_s=10, L=300, h_q=4, h_kv=2), None, 8.0),
]


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("case", range(len(WIDE)))
def test_fwd_wide_logits(sa, case, d):
    """Queries scaled by 4 (logit std about 4 natural units) and values by 1/4: rows whose
    later units exceed their reference by more than 2^10 in weight take the rescale."""
    mode, kw, rope, alibi = WIDE[case]
    wl = W.small(mode, seed=520 + case, rope_base=rope, alibi_exp=alibi, d=d, **kw)
    log(f"wide logits {case}")
    _run_small(sa, wl, check_canary=True, qmul=4.0, vmul=0.25, expect=("rescale",))


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("case", range(len(WIDE)))
def test_fwd_logit_spike(sa, case, d):
    """Every 7th row of the second half aims its query at one key with a logit of 150 natural
    units, visited after the keys that set the row's reference: the capped starting key
    (Lambda with RoPE, visited last), the diagonal key after the gathered separators (SepLLM)
    or the prefix (segment), the first key under the clipped ALiBi bias (visited last).  The
    weight against the stale reference would overflow (2^(s - m_ref) with s - m_ref >= 128):
    the kernel computes that unit again with its exact row maximum."""
    mode, kw, rope, alibi = WIDE[case]
    wl = W.small(mode, seed=540 + case, rope_base=rope, alibi_exp=alibi, d=d, **kw)
    log(f"logit spike {case}")
    _run_small(sa, wl, check_canary=True, spike=list(range(wl.n_q // 2, wl.n_q, 7)),
               expect=("recompute", "overflow"))


def test_determinism(sa):
    wl = W.small(W.SEPLLM, seed=11, m=1000, a=4, w=128, p_sep=0.1, h_q=4, h_kv=2)
    o1, l1 = _run_small(sa, wl)
    o2, l2 = _run_small(sa, wl)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def _workload_parity(sa, cid, heads, n_random):
    wl = W.WORKLOADS[cid]
    log(f"workload {cid}: inputs")
    inp = W.make_inputs(wl)
    sep = inp.get("sep")
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    sa_obj = device_mask(wl, None if sep is None else sep.cuda())
    sa_obj.build_plan()
    lse = torch.empty((wl.batch, wl.h_q, wl.n_q), dtype=torch.float32, device="cuda")
    o = sa_obj.forward(q, k, v, lse=lse, rope_base=wl.rope_base, scale=wl.scale,
                       alibi_exp=wl.alibi_exp)
    torch.cuda.synchronize()
    log(f"workload {cid}: oracle")
    spec = spec_of(wl, None if sep is None else sep.numpy())
    rows = np.arange(wl.n_q) if n_random is None else sample_rows(wl.n_q, n_random, cid)
    group = wl.h_q // wl.h_kv
    kv_heads = sorted(set(h // group for h in heads))
    K = {g: to64(inp["k"][0, g]) for g in kv_heads}
    V = {g: to64(inp["v"][0, g]) for g in kv_heads}
    for h in heads:
        g = h // group
        Qh = to64(inp["q"][0, h])
        slope = None if wl.alibi_exp is None else O.alibi_slope(h, wl.h_q, wl.alibi_exp)
        ref_o, ref_l = oracle_rows(Qh[None], K[g][None], V[g][None], spec, wl.rope_base, wl.scale,
                                   [0], rows, slope_of=lambda _h: slope)
        got_o = to64(o[0, h][torch.from_numpy(rows).cuda()])
        got_l = to64(lse[0, h][torch.from_numpy(rows).cuda()])
        stats = compare(got_o, ref_o[0], got_l, ref_l[0], wl.dtype)
        log(f"workload {cid} head {h}: max-abs {stats[0]:.2e} mean-abs {stats[1]:.2e} lse {stats[2]:.2e}")


def test_workload1_full(sa):
    _workload_parity(sa, 1, heads=[0, 1], n_random=None)


def test_workload7_sampled(sa):
    """The Pythia-class 4K SepLLM layer (12 heads of 64, batch 8): batch row 0, three heads."""
    _workload_parity(sa, 7, heads=[0, 5, 11], n_random=300)


def test_workload2_full_rows(sa):
    _workload_parity(sa, 2, heads=[0, 13, 31], n_random=None)


def test_workload3_sampled(sa):
    _workload_parity(sa, 3, heads=[0, 31], n_random=192)


def test_workload5_sampled(sa):
    _workload_parity(sa, 5, heads=[0, 5, 31], n_random=96)


def test_workload6_alibi_sampled(sa):
    _workload_parity(sa, 6, heads=[0, 17, 31], n_random=192)


# The ALiBi bias clipped at L_pretrain under the Lambda mask (LM-Infinite page, section
# "method").  Slopes 2^(-E (h+1) / h_q): E = 8 with 2 heads gives 1/16 and 1/256 (starting-span
# keys beyond the cap keep real weight); E = 0.5 gives slopes near 1, where the bias spans
# hundreds of base-2 units across a row.
ALIBI_SMALL = [
    dict(m=900, n_s=10, L=300, h_q=8, h_kv=2, alibi_exp=8.0),
    dict(m=700, n_s=0, L=100, alibi_exp=8.0),
    dict(m=600, n_s=100, L=64, alibi_exp=8.0),
    dict(m=300, n_s=10, L=0, alibi_exp=8.0),
    dict(m=300, n_s=5, L=5000, alibi_exp=8.0),
    dict(m=1, n_s=10, L=100, alibi_exp=8.0),
    dict(m=129, n_s=3, L=40, alibi_exp=2.0, batch=2),
    dict(m=900, n_s=10, L=300, alibi_exp=0.5),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", range(len(ALIBI_SMALL)))
def test_fwd_alibi_small(sa, case, dtype):
    d = 128 if dtype == "bf16" else 64
    wl = W.small(W.LAMBDA, seed=300 + case, dtype=dtype, d=d, rope_base=None, **ALIBI_SMALL[case])
    log(f"alibi small {case} {dtype}")
    _run_small(sa, wl, check_canary=True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_alibi_q_zero_closed_form(sa, dtype):
    wl = W.small(W.LAMBDA, seed=19, dtype=dtype, d=128 if dtype == "bf16" else 64, m=640, n_s=10,
                 L=100, rope_base=None, alibi_exp=8.0)
    _run_small(sa, wl, q_zero=True)


def test_workload4_segment_with_topk(sa):
    from structured_sparse_attention_attn_amd.pipeline import TopK
    wl = W.WORKLOADS[4]
    log("workload 4: inputs")
    inp = W.make_inputs(wl)
    S, P, H, d = wl.n_q, wl.P, wl.h_q, wl.d
    n_long = H - wl.n_local
    dev = "cuda"
    q = inp["q"].to(dev)
    kcat = torch.empty((1, H, P + S, d), dtype=torch.bfloat16, device=dev)
    vcat = torch.empty_like(kcat)
    kcat[:, :, P:] = inp["k_seg"].to(dev)
    vcat[:, :, P:] = inp["v_seg"].to(dev)
    kcat[:, :wl.n_local, :P] = inp["k_tail"].to(dev)
    vcat[:, :wl.n_local, :P] = inp["v_tail"].to(dev)
    kpool, vpool = inp["k_pool"][0].to(dev), inp["v_pool"][0].to(dev)
    idx = torch.empty((n_long, P), dtype=torch.int32, device=dev)
    score = torch.empty((n_long, P), dtype=torch.float64, device=dev)
    topk = TopK(n_long, wl.pool_len)
    topk(q[0, wl.n_local:, S - 1, :], kpool, P, idx, score=score, pool_v=vpool,
         pref_k=kcat[0, wl.n_local:, :P], pref_v=vcat[0, wl.n_local:, :P])
    sa_obj = device_mask(wl)
    sa_obj.build_plan()
    lse = torch.empty((1, H, S), dtype=torch.float32, device=dev)
    o = sa_obj.forward(q, kcat, vcat, lse=lse, rope_base=wl.rope_base, scale=wl.scale)
    torch.cuda.synchronize()
    log("workload 4: oracle top-k")
    spec = spec_of(wl)
    ref_idx = []
    for hh in range(n_long):
        s = O.topk_scores(to64(inp["q"][0, wl.n_local + hh, S - 1]), to64(inp["k_pool"][0, hh]))
        ri = O.topk_select(s, P)
        np.testing.assert_array_equal(idx[hh].cpu().numpy(), ri)
        np.testing.assert_array_equal(score[hh].cpu().numpy(), s[ri])
        ref_idx.append(ri)
    rows = sample_rows(S, 128, 4)
    for h in [0, 23, 24, 31]:
        if h < wl.n_local:
            Kh = np.concatenate([to64(inp["k_tail"][0, h]), to64(inp["k_seg"][0, h])])
            Vh = np.concatenate([to64(inp["v_tail"][0, h]), to64(inp["v_seg"][0, h])])
        else:
            ri = ref_idx[h - wl.n_local]
            Kh = np.concatenate([to64(inp["k_pool"][0, h - wl.n_local])[ri], to64(inp["k_seg"][0, h])])
            Vh = np.concatenate([to64(inp["v_pool"][0, h - wl.n_local])[ri], to64(inp["v_seg"][0, h])])
        ref_o, ref_l = oracle_rows(to64(inp["q"][0, h])[None], Kh[None], Vh[None], spec,
                                   wl.rope_base, wl.scale, [0], rows)
        rr = torch.from_numpy(rows).cuda()
        stats = compare(to64(o[0, h][rr]), ref_o[0], to64(lse[0, h][rr]), ref_l[0], wl.dtype)
        log(f"workload 4 head {h}: max-abs {stats[0]:.2e} mean-abs {stats[1]:.2e} lse {stats[2]:.2e}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_topk_narrow_scores(sa, dtype):
    """Scores that all share their leading exponent bits (every score in
    [1, 2), or all equal): the selection runs its later digits over a
    candidate set of 4000 keys (kept on chip) or over more keys than that
    (read again from memory), with heavy ties resolved by the lower index."""
    from structured_sparse_attention_attn_amd.pipeline import TopK
    for n_heads, pool_len, k, seed, all_equal in [(2, 4000, 777, 11, False), (2, 10000, 5000, 12, False),
                                                  (1, 10000, 4321, 13, True)]:
        q, kp, vp = W.make_pool_inputs(n_heads, pool_len, 128, seed, dtype)
        q = torch.zeros_like(q)
        if not all_equal:
            q[:, 0] = 1.0
            g = torch.Generator().manual_seed(seed)
            kp[:, :, 0] = (1.0 + 0.99 * torch.rand((n_heads, pool_len), generator=g)).to(dtype)
        topk = TopK(n_heads, pool_len)
        idx = torch.empty((n_heads, k), dtype=torch.int32, device="cuda")
        score = torch.empty((n_heads, k), dtype=torch.float64, device="cuda")
        topk(q.cuda(), kp.cuda(), k, idx, score=score)
        torch.cuda.synchronize()
        for h in range(n_heads):
            s_ = O.topk_scores(q[h].double().numpy(), kp[h].double().numpy())
            ri = O.topk_select(s_, k)
            np.testing.assert_array_equal(idx[h].cpu().numpy(), ri)
            np.testing.assert_array_equal(score[h].cpu().numpy(), s_[ri])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_topk_bitexact(sa, dtype):
    from structured_sparse_attention_attn_amd.pipeline import TopK
    for n_heads, pool_len, d, ks, seed in [(8, 32768, 128, (1, 1024, 32768), 1), (3, 1000, 64, (1, 7, 999, 1000), 2),
                                           (2, 5000, 128, (100,), 3), (2, 40000, 128, (1, 333, 40000), 4),
                                           (1, 70000, 64, (4096,), 5)]:
        q, kp, vp = W.make_pool_inputs(n_heads, pool_len, d, seed, dtype)
        if seed == 3:
            kp = (kp * 2).round() / 2  # coarse values: many exactly tied scores
            q = q.round()
        qd, kd, vd = q.cuda(), kp.cuda(), vp.cuda()
        topk = TopK(n_heads, pool_len)
        for k in ks:
            idx = torch.empty((n_heads, k), dtype=torch.int32, device="cuda")
            score = torch.empty((n_heads, k), dtype=torch.float64, device="cuda")
            pk = torch.zeros((n_heads, k, d), dtype=dtype, device="cuda")
            pv = torch.zeros_like(pk)
            topk(qd, kd, k, idx, score=score, pool_v=vd, pref_k=pk, pref_v=pv)
            torch.cuda.synchronize()
            for h in range(n_heads):
                s = O.topk_scores(q[h].double().numpy(), kp[h].double().numpy())
                ri = O.topk_select(s, k)
                np.testing.assert_array_equal(idx[h].cpu().numpy(), ri)
                np.testing.assert_array_equal(score[h].cpu().numpy(), s[ri])
                assert torch.equal(pk[h].cpu(), kp[h][torch.from_numpy(ri).long()])
                assert torch.equal(pv[h].cpu(), vp[h][torch.from_numpy(ri).long()])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_topk_shapes(sa, dtype):
    """Shapes at the edges of the selection's work split: a pool of 33 keys
    (3 groups of 16; k below, at and above the group count), 300 heads (one
    work group each), k equal to the group count and one more (the lower
    bound from the group maxima used, then not), one key past a single pass
    over the head's buckets, a pool length that is not a multiple of 8, and a
    bound so low that the list of keys above it overflows (k = 2000 of 2048
    group maxima)."""
    from structured_sparse_attention_attn_amd.pipeline import TopK
    for n_heads, pool_len, d, ks, seed in [(1, 33, 64, (1, 2, 3, 33), 21), (300, 100, 64, (7,), 22),
                                           (2, 2048, 128, (128, 129), 23), (2, 32769, 128, (1000,), 24),
                                           (4, 4100, 128, (2050,), 25), (2, 32768, 128, (2000,), 26)]:
        log(f"topk shapes {dtype}: heads {n_heads} pool {pool_len} d {d} k {ks}")
        q, kp, vp = W.make_pool_inputs(n_heads, pool_len, d, seed, dtype)
        qd, kd, vd = q.cuda(), kp.cuda(), vp.cuda()
        topk = TopK(n_heads, pool_len)
        for k in ks:
            idx = torch.empty((n_heads, k), dtype=torch.int32, device="cuda")
            score = torch.empty((n_heads, k), dtype=torch.float64, device="cuda")
            pk = torch.zeros((n_heads, k, d), dtype=dtype, device="cuda")
            pv = torch.zeros_like(pk)
            topk(qd, kd, k, idx, score=score, pool_v=vd, pref_k=pk, pref_v=pv)
            torch.cuda.synchronize()
            got_i, got_s = idx.cpu().numpy(), score.cpu().numpy()
            for h in range(n_heads):
                s_ = O.topk_scores(q[h].double().numpy(), kp[h].double().numpy())
                ri = O.topk_select(s_, k)
                np.testing.assert_array_equal(got_i[h], ri)
                np.testing.assert_array_equal(got_s[h], s_[ri])
            sel = torch.from_numpy(got_i).long()
            assert torch.equal(pk.cpu(), torch.gather(kp, 1, sel[:, :, None].expand(-1, -1, d)))
            assert torch.equal(pv.cpu(), torch.gather(vp, 1, sel[:, :, None].expand(-1, -1, d)))


# Several segments end to end: forward, tail carry, pool append, retrieval by the
# segment-end query (segmented-execution page, overall framework), against the oracle's
# segment recurrence.
@pytest.mark.parametrize("dtype,S,M,N", [("bf16", 300, 128, 3), ("bf16", 100, 128, 4),
                                         ("f32", 200, 64, 3)])
def test_segment_runner_vs_oracle(sa, dtype, S, M, N):
    from structured_sparse_attention_attn_amd.pipeline import SegmentRunner
    H, nl, base = 4, 2, 10000.0
    d = 128 if dtype == "bf16" else 64
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    scale = d ** -0.5
    stream = W.make_segment_stream(H, S, d, N, seed=77 + S, dtype=tdt)
    runner = SegmentRunner(H, nl, d, S, M, N * S, rope_base=base, scale=scale, dtype=tdt)
    got = []
    for i, (q, k, v) in enumerate(stream):
        log(f"segment runner {dtype} S={S} M={M}: segment {i}")
        ks, vs = runner.seg_kv()
        ks.copy_(k.cuda())
        vs.copy_(v.cuda())
        lse = torch.empty((1, H, S), dtype=torch.float32, device="cuda")
        P = runner.P
        o = runner.step(q.cuda(), lse=lse)
        torch.cuda.synchronize()
        got.append((to64(o[0]), to64(lse[0]), P, runner.idx.cpu().numpy().copy()))
    ref, state = O.segmented_run([to64(x[0][0]) for x in stream], [to64(x[1][0]) for x in stream],
                                 [to64(x[2][0]) for x in stream], nl, M, M, base, scale)
    for i in range(N):
        o_g, l_g, P, idx_g = got[i]
        assert P == ref[i]["P"]
        compare(o_g, ref[i]["O"], l_g, ref[i]["LSE"], dtype)
        if i + 1 < N:
            np.testing.assert_array_equal(idx_g, ref[i + 1]["idx"])
    # the final state is a byte copy of the history
    k_long = torch.cat([x[1][0, nl:] for x in stream], dim=1)
    assert torch.equal(runner.pool_k[:, :N * S].cpu(), k_long)
    keep = runner.P
    nk, nv = runner.bufs[runner.cur]
    k_loc = torch.cat([x[1][0, :nl] for x in stream], dim=1)
    v_loc = torch.cat([x[2][0, :nl] for x in stream], dim=1)
    assert torch.equal(nk[0, :nl, M - keep:M].cpu(), k_loc[:, N * S - keep:])
    assert torch.equal(nv[0, :nl, M - keep:M].cpu(), v_loc[:, N * S - keep:])
    np.testing.assert_array_equal(to64(nk[0, :nl, M - keep:M]), state["tail_k"])


# Backward (dQ, dK, dV) against the oracle's gradient formulas.
BWD_SMALL = [
    (W.SEPLLM, dict(m=700, a=4, w=64, p_sep=0.1), 10000.0, None),
    (W.SEPLLM, dict(m=500, a=70, w=100, p_sep=0.2, h_q=4, h_kv=2, batch=2), 10000.0, None),
    (W.SEPLLM, dict(m=300, a=0, w=1, p_sep=0.3), None, None),
    (W.LAMBDA, dict(m=900, n_s=10, L=300), 10000.0, None),
    (W.LAMBDA, dict(m=600, n_s=100, L=64, h_q=4, h_kv=1), 10000.0, None),
    (W.LAMBDA, dict(m=300, n_s=10, L=0), 10000.0, None),
    (W.LAMBDA, dict(m=700, n_s=10, L=100), None, 8.0),
    (W.SEGMENT, dict(m=600, P=200), 10000.0, None),
    (W.SEGMENT, dict(m=129, P=1, h_q=4, h_kv=2), 10000.0, None),
    (W.SEPLLM, dict(m=1, a=4, w=64, p_sep=0.5), 10000.0, None),
    # initial tokens over two 128-key groups (both dispatched first and walked
    # last to first with the separator groups), GQA
    (W.SEPLLM, dict(m=900, a=150, w=64, p_sep=0.15, h_q=4, h_kv=2), 10000.0, None),
]


def _bwd_stats(got, ref):
    err = np.abs(got - ref)
    return float(err.max()), float(err.mean()), float(np.abs(ref).max()), float(np.abs(ref).mean())


def bwd_compare(name, got, ref):
    """Gradient bar, relative to the gradient's own size (gradients have no fixed scale).

    The outputs are bf16 (rounding alone: relative 2^-9 per element); P, dS and the
    rotated q, k enter the products as bf16 (relative 2^-9 each) and P carries the
    forward's logit error (a few 1e-3), so elements sit within a few 2^-9 of the
    reference relative to the terms they sum.  Bar: max-abs <= 1e-2 * max|ref| and
    mean-abs <= 1e-2 * mean|ref| (floor 1e-3 for vanishing references).
    """
    mx, mean, rmx, rmean = _bwd_stats(got, ref)
    log(f"  {name}: max-abs {mx:.3e} mean-abs {mean:.3e} | ref max {rmx:.3e} mean {rmean:.3e}")
    assert np.isfinite(got).all(), name
    assert mx <= 1e-2 * max(rmx, 0.1), (name, mx, rmx)
    assert mean <= 1e-2 * max(rmean, 0.1), (name, mean, rmean)


@pytest.mark.parametrize("case", range(len(BWD_SMALL)))
def test_bwd_small(sa, case):
    mode, kw, rope, alibi = BWD_SMALL[case]
    wl = W.small(mode, seed=500 + case, rope_base=rope, alibi_exp=alibi, **kw)
    log(f"bwd small {case}: {mode} {kw} rope={rope} alibi={alibi}")
    inp = W.make_small_inputs(wl)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    sep = inp.get("sep")
    sa_obj = device_mask(wl, None if sep is None else sep.cuda())
    sa_obj.build_plan()
    lse = torch.empty((wl.batch, wl.h_q, wl.n_q), dtype=torch.float32, device="cuda")
    o = sa_obj.forward(q, k, v, lse=lse, rope_base=wl.rope_base, scale=wl.scale, alibi_exp=wl.alibi_exp)
    dout = W.make_grad(tuple(q.shape), seed=900 + case).cuda()
    dq, dk, dv = sa_obj.backward(q, k, v, o, lse, dout, rope_base=wl.rope_base, scale=wl.scale,
                                 alibi_exp=wl.alibi_exp)
    torch.cuda.synchronize()
    spec = spec_of(wl, None if sep is None else sep.numpy())
    for b in range(wl.batch):
        rq, rk, rv = O.attention_backward(to64(inp["q"][b]), to64(inp["k"][b]), to64(inp["v"][b]),
                                          to64(dout[b]), spec, wl.rope_base, wl.scale,
                                          alibi_exp=wl.alibi_exp)
        for name, got, ref in (("dq", dq[b], rq), ("dk", dk[b], rk), ("dv", dv[b], rv)):
            bwd_compare(f"b{b} {name}", to64(got), ref)


@pytest.mark.parametrize("case", range(len(BWD_SMALL)))
def test_bwd_small_bf16_d64(sa, case):
    """bf16 with 64-element heads: the vector-ALU backward (bf16 rows, fp32 sums)."""
    mode, kw, rope, alibi = BWD_SMALL[case]
    wl = W.small(mode, seed=800 + case, d=64, rope_base=rope, alibi_exp=alibi, **kw)
    log(f"bwd d64 {case}: {mode} {kw} rope={rope} alibi={alibi}")
    inp = W.make_small_inputs(wl)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    sep = inp.get("sep")
    sa_obj = device_mask(wl, None if sep is None else sep.cuda())
    sa_obj.build_plan()
    lse = torch.empty((wl.batch, wl.h_q, wl.n_q), dtype=torch.float32, device="cuda")
    o = sa_obj.forward(q, k, v, lse=lse, rope_base=wl.rope_base, scale=wl.scale, alibi_exp=wl.alibi_exp)
    dout = W.make_grad(tuple(q.shape), seed=980 + case).cuda()
    dq, dk, dv = sa_obj.backward(q, k, v, o, lse, dout, rope_base=wl.rope_base, scale=wl.scale,
                                 alibi_exp=wl.alibi_exp)
    torch.cuda.synchronize()
    spec = spec_of(wl, None if sep is None else sep.numpy())
    for b in range(wl.batch):
        rq, rk, rv = O.attention_backward(to64(inp["q"][b]), to64(inp["k"][b]), to64(inp["v"][b]),
                                          to64(dout[b]), spec, wl.rope_base, wl.scale,
                                          alibi_exp=wl.alibi_exp)
        for name, got, ref in (("dq", dq[b], rq), ("dk", dk[b], rk), ("dv", dv[b], rv)):
            bwd_compare(f"b{b} {name}", to64(got), ref)


@pytest.mark.parametrize("case", [1, 3, 6])
def test_bwd_strided(sa, case):
    """The backward on [B, T, H, d] storage viewed as [B, H, T, d]: strided q, k, v, dout
    and gradients written through the same strides."""
    mode, kw, rope, alibi = BWD_SMALL[case]
    wl = W.small(mode, seed=500 + case, rope_base=rope, alibi_exp=alibi, **kw)
    log(f"bwd strided {case}: {mode} {kw} rope={rope} alibi={alibi}")
    inp = W.make_small_inputs(wl)
    strided = lambda t: t.permute(0, 2, 1, 3).contiguous().cuda().permute(0, 2, 1, 3)  # noqa: E731
    q, k, v = (strided(inp[x]) for x in ("q", "k", "v"))
    assert q.stride(2) != q.shape[3]
    sep = inp.get("sep")
    sa_obj = device_mask(wl, None if sep is None else sep.cuda())
    sa_obj.build_plan()
    lse = torch.empty((wl.batch, wl.h_q, wl.n_q), dtype=torch.float32, device="cuda")
    o = sa_obj.forward(q, k, v, o=strided(torch.zeros(tuple(q.shape), dtype=q.dtype)), lse=lse,
                       rope_base=wl.rope_base, scale=wl.scale, alibi_exp=wl.alibi_exp)
    dout_c = W.make_grad(tuple(q.shape), seed=900 + case)
    dq, dk, dv = sa_obj.backward(q, k, v, o, lse, strided(dout_c), rope_base=wl.rope_base, scale=wl.scale,
                                 alibi_exp=wl.alibi_exp, dq=strided(torch.zeros(tuple(q.shape), dtype=q.dtype)),
                                 dk=strided(torch.zeros(tuple(k.shape), dtype=k.dtype)),
                                 dv=strided(torch.zeros(tuple(v.shape), dtype=v.dtype)))
    torch.cuda.synchronize()
    assert dq.stride() == q.stride() and dk.stride() == k.stride()
    spec = spec_of(wl, None if sep is None else sep.numpy())
    for b in range(wl.batch):
        rq, rk, rv = O.attention_backward(to64(inp["q"][b]), to64(inp["k"][b]), to64(inp["v"][b]),
                                          to64(dout_c[b]), spec, wl.rope_base, wl.scale,
                                          alibi_exp=wl.alibi_exp)
        for name, got, ref in (("dq", dq[b], rq), ("dk", dk[b], rk), ("dv", dv[b], rv)):
            bwd_compare(f"b{b} {name}", to64(got), ref)


# fp32 backward: every product and sum in fp32 on both passes; the oracle in fp64.
BWD_F32 = [
    (W.SEPLLM, dict(m=700, a=4, w=64, p_sep=0.1, d=64), None, None),
    (W.SEPLLM, dict(m=500, a=70, w=100, p_sep=0.2, h_q=4, h_kv=2, batch=2), 10000.0, None),
    (W.LAMBDA, dict(m=900, n_s=10, L=300), 10000.0, None),
    (W.LAMBDA, dict(m=600, n_s=100, L=64, h_q=4, h_kv=1, d=64), 10000.0, None),
    (W.LAMBDA, dict(m=700, n_s=10, L=100), None, 8.0),
    (W.SEGMENT, dict(m=129, P=1, h_q=4, h_kv=2), 10000.0, None),
    (W.SEGMENT, dict(m=300, P=200, d=64), 10000.0, None),
    (W.SEPLLM, dict(m=1, a=4, w=64, p_sep=0.5), 10000.0, None),
]


def f32_grad_compare(name, got, ref):
    """fp32 gradient bar: max-abs <= 1e-5 * max(1, max|ref|), the fp32 forward's 1e-5 read
    relative to the gradient's own scale (the sums hold up to a few hundred terms of
    relative rounding 2^-24 each, and P carries the forward's LSE error of ~1e-6)."""
    err = np.abs(got - ref)
    rmx = float(np.abs(ref).max()) if ref.size else 0.0
    log(f"  {name}: max-abs {err.max():.3e} | ref max {rmx:.3e}")
    assert np.isfinite(got).all(), name
    assert err.max() <= 1e-5 * max(1.0, rmx), (name, float(err.max()), rmx)


def _bwd_f32_case(sa, wl, seed):
    inp = W.make_small_inputs(wl)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    assert q.dtype == torch.float32
    sep = inp.get("sep")
    sa_obj = device_mask(wl, None if sep is None else sep.cuda())
    sa_obj.build_plan()
    lse = torch.empty((wl.batch, wl.h_q, wl.n_q), dtype=torch.float32, device="cuda")
    o = sa_obj.forward(q, k, v, lse=lse, rope_base=wl.rope_base, scale=wl.scale, alibi_exp=wl.alibi_exp)
    dout = W.make_grad(tuple(q.shape), seed=seed, dtype=torch.float32).cuda()
    dq, dk, dv = sa_obj.backward(q, k, v, o, lse, dout, rope_base=wl.rope_base, scale=wl.scale,
                                 alibi_exp=wl.alibi_exp)
    torch.cuda.synchronize()
    spec = spec_of(wl, None if sep is None else sep.numpy())
    for b in range(wl.batch):
        rq, rk, rv = O.attention_backward(to64(inp["q"][b]), to64(inp["k"][b]), to64(inp["v"][b]),
                                          to64(dout[b]), spec, wl.rope_base, wl.scale,
                                          alibi_exp=wl.alibi_exp)
        for name, got, ref in (("dq", dq[b], rq), ("dk", dk[b], rk), ("dv", dv[b], rv)):
            f32_grad_compare(f"b{b} {name}", to64(got), ref)
    return dq, dk, dv


@pytest.mark.parametrize("case", range(len(BWD_F32)))
def test_bwd_f32_small(sa, case):
    mode, kw, rope, alibi = BWD_F32[case]
    wl = W.small(mode, seed=600 + case, dtype="f32", rope_base=rope, alibi_exp=alibi, **kw)
    log(f"bwd f32 {case}: {mode} {kw} rope={rope} alibi={alibi}")
    _bwd_f32_case(sa, wl, 950 + case)


def test_workload1_backward(sa):
    """The tiny fp32 SepLLM configuration (2 heads, d = 64, m = 512, no RoPE): every gradient
    row against the oracle, and a second run bit-identical (fixed summation order)."""
    wl = W.WORKLOADS[1]
    log("workload 1 backward")
    first = _bwd_f32_case(sa, wl, 1001)
    again = _bwd_f32_case(sa, wl, 1001)
    for a_, b_ in zip(first, again):
        assert torch.equal(a_, b_)


def test_sep_max_bound(sa):
    """A caller bound on the separator count (sep_max): with the exact count the plan, the
    forward and the backward are bit-identical to the unbounded ones (and the forward matches
    the oracle); one below it, sa_plan_status reports SA_ENOSPACE, every kernel stays inside
    its buffers (guard bytes after the exactly sized workspace), and O, the LSE and dQ come
    out NaN instead of silently missing keys."""
    wl = W.small(W.SEPLLM, seed=777, m=1000, a=4, w=64, p_sep=0.2, h_q=4, h_kv=2)
    inp = W.make_small_inputs(wl)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    sep = inp["sep"]
    g0 = 64 * math.ceil(wl.a / 64)
    n_sep = int(sep[g0:].sum())
    log(f"sep_max bound: {n_sep} separators at j >= {g0}")
    assert n_sep > 100
    dout = W.make_grad(tuple(q.shape), seed=778).cuda()
    runs = {}
    for name, bound in (("free", 0), ("exact", n_sep), ("short", n_sep - 5)):
        sa_obj = device_mask(wl, sep.cuda(), sep_max=bound)
        sa_obj.build_plan()
        if name == "short":
            with pytest.raises(sa.SparseAttnError) as e:
                sa.sa_plan_status(sa_obj.plan)
            assert e.value.code == sa.SA_ENOSPACE
        else:
            hdr = sa.sa_plan_status(sa_obj.plan)
            assert hdr.n_sep == n_sep and hdr.cap_sep == (n_sep if bound else wl.n_k)
        args0 = sa_obj.args(q, k, v, torch.empty_like(q))
        need = sa.sa_fwd_workspace_bytes(sa_obj.mask, args0)
        guard = 1 << 16
        store = torch.full((need + guard,), 0xA5, dtype=torch.uint8, device="cuda")
        sa_obj.ws = store[:need]
        lse = torch.empty((wl.batch, wl.h_q, wl.n_q), dtype=torch.float32, device="cuda")
        o = sa_obj.forward(q, k, v, lse=lse, rope_base=wl.rope_base, scale=wl.scale)
        grads = sa_obj.backward(q, k, v, o, lse, dout, rope_base=wl.rope_base, scale=wl.scale)
        torch.cuda.synchronize()
        assert torch.all(store[need:] == 0xA5), f"{name}: workspace guard overwritten"
        runs[name] = (o, lse) + tuple(grads)
    for a_, b_ in zip(runs["free"], runs["exact"]):
        assert torch.equal(a_, b_)
    o, lse = runs["exact"][:2]
    spec = spec_of(wl, sep.numpy())
    ref_o, ref_l = O.attention(to64(inp["q"][0]), to64(inp["k"][0]), to64(inp["v"][0]), spec,
                               wl.rope_base, wl.scale)
    compare(to64(o[0]), ref_o, to64(lse[0]), ref_l, wl.dtype)
    o, lse, dq = runs["short"][:3]
    assert torch.isnan(o).all() and torch.isnan(lse).all() and torch.isnan(dq).all()


def _workload_bwd_parity(sa, cid, dq_heads, n_random, key_block, dk_kv_head, expect_sep=False):
    """Backward at a workload's full size: dQ on sampled rows of some heads; dK, dV on one
    key block of one kv head, from every query row that sees a key of that block (the
    oracle sums those rows' contributions, over the kv head's whole GQA group)."""
    wl = W.WORKLOADS[cid]
    log(f"workload {cid} backward: inputs")
    inp = W.make_inputs(wl)
    sep = inp.get("sep")
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    sa_obj = device_mask(wl, None if sep is None else sep.cuda())
    sa_obj.build_plan()
    lse = torch.empty((wl.batch, wl.h_q, wl.n_q), dtype=torch.float32, device="cuda")
    o = sa_obj.forward(q, k, v, lse=lse, rope_base=wl.rope_base, scale=wl.scale, alibi_exp=wl.alibi_exp)
    dout = W.make_grad(tuple(q.shape), seed=wl.seed + 11).cuda()
    dq, dk, dv = sa_obj.backward(q, k, v, o, lse, dout, rope_base=wl.rope_base, scale=wl.scale,
                                 alibi_exp=wl.alibi_exp)
    torch.cuda.synchronize()
    spec = spec_of(wl, None if sep is None else sep.numpy())
    group = wl.h_q // wl.h_kv
    slope = (lambda h: None) if wl.alibi_exp is None else (lambda h: O.alibi_slope(h, wl.h_q, wl.alibi_exp))
    r_ = np.random.default_rng(cid)
    rows = np.array(sorted(set(range(64)) | set(range(wl.n_q - 64, wl.n_q))
                           | set(r_.choice(wl.n_q, size=n_random, replace=False).tolist())))
    for h in dq_heads:
        g = h // group
        log(f"workload {cid} backward: dq head {h}")
        rq, _, _ = O.attention_grad_rows(to64(inp["q"][0, h]), to64(inp["k"][0, g]), to64(inp["v"][0, g]),
                                         to64(dout[0, h]), rows, spec, wl.rope_base, wl.scale, slope(h))
        bwd_compare(f"w{cid} dq h{h}", to64(dq[0, h][torch.from_numpy(rows).cuda()]), rq)
    keys = np.arange(64 * key_block, min(wl.n_k, 64 * key_block + 64))
    sel = np.ones(len(keys), dtype=bool)
    if expect_sep:
        n_sep_blk = int(sep.numpy()[keys].sum())
        assert n_sep_blk > 0
        log(f"workload {cid} backward: block {key_block} holds {n_sep_blk} separators")
    cand = np.arange(max(0, keys[0] - wl.P), wl.n_q)
    seen = O.visible(spec, cand[:, None], keys[sel][None, :]).any(axis=1)
    qrows = cand[seen]
    log(f"workload {cid} backward: dk/dv kv head {dk_kv_head}, block {key_block}, {len(qrows)} query rows")
    rk = np.zeros((len(keys), wl.d))
    rv = np.zeros((len(keys), wl.d))
    Kg, Vg = to64(inp["k"][0, dk_kv_head]), to64(inp["v"][0, dk_kv_head])
    for h in range(dk_kv_head * group, (dk_kv_head + 1) * group):
        dkc, dvc = O.attention_grad_keys_fast(to64(inp["q"][0, h]), Kg, Vg, to64(dout[0, h]), spec,
                                              wl.rope_base, wl.scale, keys, qrows, slope(h))
        rk += dkc
        rv += dvc
    gk = to64(dk[0, dk_kv_head, torch.from_numpy(keys).cuda()])
    gv = to64(dv[0, dk_kv_head, torch.from_numpy(keys).cuda()])
    bwd_compare(f"w{cid} dk g{dk_kv_head} blk{key_block}", gk[sel], rk[sel])
    bwd_compare(f"w{cid} dv g{dk_kv_head} blk{key_block}", gv[sel], rv[sel])


# key blocks near the end keep the oracle's share small (fewer query rows read them)
def test_workload3_backward_sampled(sa):
    _workload_bwd_parity(sa, 3, dq_heads=[0, 31], n_random=64, key_block=505, dk_kv_head=31)


def test_workload5_backward_sampled(sa):
    # block 2020 (keys 129280..129343) holds separators read by every later query: through
    # the window blocks by the queries within w = 1024 and through the gathered separator
    # chunks by the ~700 queries after that; their dK, dV sum over all those rows of the
    # kv head's 4 query heads (the gathered path's scatter back to the key rows)
    _workload_bwd_parity(sa, 5, dq_heads=[31], n_random=32, key_block=2020, dk_kv_head=7,
                         expect_sep=True)


def test_workload6_backward_sampled(sa):
    _workload_bwd_parity(sa, 6, dq_heads=[0], n_random=64, key_block=505, dk_kv_head=0)


# Streaming decode with the generation-time cache (SepLLM page, part 6.2), against the
# oracle's closed-form held set and decode attention, every step.
STREAM_CASES = [
    dict(B=2, h_q=8, h_kv=2, a=4, s=8, w=16, c=60, n=300, p=0.3, rope=10000.0),
    dict(B=1, h_q=4, h_kv=1, a=4, s=64, w=128, c=324, n=700, p=0.1, rope=10000.0),
    dict(B=1, h_q=2, h_kv=2, a=0, s=1, w=1, c=3, n=60, p=0.5, rope=None),
    dict(B=1, h_q=8, h_kv=1, a=3, s=4, w=6, c=30, n=200, p=1.0, rope=500000.0),
]


@pytest.mark.parametrize("case", range(len(STREAM_CASES)))
def test_stream_decode(sa, case):
    from structured_sparse_attention_attn_amd.pipeline import StreamDecoder
    cfg = STREAM_CASES[case]
    B, hq, hkv, d = cfg["B"], cfg["h_q"], cfg["h_kv"], 128
    log(f"stream decode {case}: {cfg}")
    q, k, v, flags = W.make_decode_stream(B, hq, hkv, d, cfg["n"], seed=1300 + case, p_sep=cfg["p"])
    dec = StreamDecoder(B, hq, hkv, d, cfg["a"], cfg["s"], cfg["w"], cfg["c"], rope_base=cfg["rope"])
    # slots never written hold NaN bit patterns: a slot that is not held must take no part
    dec.state.fill_(0xFF)
    dec.reset()
    scale = d ** -0.5
    group = hq // hkv
    lse = torch.empty((B, hq), dtype=torch.float32, device="cuda")
    errs = []
    for t in range(cfg["n"]):
        o = dec.step(q[t].cuda(), k[t].cuda(), v[t].cuda(), flags[t].cuda(), lse=lse)
        torch.cuda.synchronize()
        for b in range(B):
            fl = flags[:t + 1, b].numpy()
            toks = O.stream_cache_tokens(t, fl, cfg["a"], cfg["s"], cfg["w"], cfg["c"])
            if t % 7 == 0 or t == cfg["n"] - 1:
                assert dec.held(b) == toks.tolist(), (t, b)
            ro = np.zeros((hq, d))
            rl = np.zeros(hq)
            for h in range(hq):
                ro[h], rl[h] = O.decode_attention(to64(q[t, b, h]), to64(k[:t + 1, b, h // group]),
                                                  to64(v[:t + 1, b, h // group]), t, toks, cfg["rope"], scale)
            errs.append(compare(to64(o[b]), ro, to64(lse[b]), rl, "bf16"))
    log(f"  max-abs {max(e[0] for e in errs):.3e}, lse {max(e[2] for e in errs):.3e}")


# LM-Infinite top-k middle tokens against the oracle.  The selection is decided by
# floating point: indices must agree except where the oracle's score lies within the
# scores' error band of the k-th best (either choice is then correct), and the GPU's
# scores of its choices must match the oracle's within that band.
MID_CASES = [
    (dict(m=900, n_s=10, L=100), 8, 10000.0),
    (dict(m=700, n_s=0, L=64, h_q=4, h_kv=1), 3, 10000.0),
    (dict(m=300, n_s=10, L=0), 1, None),
    (dict(m=200, n_s=10, L=250), 4, 10000.0),
    (dict(m=600, n_s=70, L=130, batch=2), 5, 500000.0),
    # lists beyond 8 entries (16- and 64-entry selection lists)
    (dict(m=700, n_s=10, L=100, h_q=4, h_kv=2), 16, 10000.0),
    (dict(m=500, n_s=4, L=64), 40, 10000.0),
]


def _check_mid_sel(row, i, wl):
    """One query's selection: the chosen indices first, then -1; chosen indices distinct and
    middle tokens of query i, n_starting <= j < i - L (LM-Infinite page, section "method")."""
    n = int((row >= 0).sum())
    assert (row[:n] >= 0).all() and (row[n:] == -1).all(), (i, row)
    g = row[:n].tolist()
    assert len(set(g)) == n, (i, row)
    assert all(wl.n_s <= j < i - wl.L for j in g), (i, row)


@pytest.mark.parametrize("case", range(len(MID_CASES)))
def test_topk_middle(sa, case):
    kw, kmid, rope = MID_CASES[case]
    wl = W.small(W.LAMBDA, seed=700 + case, rope_base=rope, **kw)
    log(f"topk middle {case}: {kw} k={kmid} rope={rope}")
    inp = W.make_small_inputs(wl)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    sa_obj = device_mask(wl)
    sa_obj.build_plan()
    lse = torch.empty((wl.batch, wl.h_q, wl.n_q), dtype=torch.float32, device="cuda")
    o = sa_obj.forward(q, k, v, lse=lse, rope_base=wl.rope_base, scale=wl.scale)
    sel, score = sa_obj.topk_middle(q, k, v, o, lse, kmid, rope_base=wl.rope_base, scale=wl.scale)
    torch.cuda.synchronize()
    spec = spec_of(wl)
    group = wl.h_q // wl.h_kv
    n_near = 0
    for b in range(wl.batch):
        for h in range(wl.h_q):
            Q, K, V = to64(inp["q"][b, h]), to64(inp["k"][b, h // group]), to64(inp["v"][b, h // group])
            ro, rl, rsel = O.attention_topk_middle(Q, K, V, range(wl.n_q), spec, wl.rope_base, wl.scale, kmid)
            gsel = sel[b, h].cpu().numpy()
            gsc = score[b, h].cpu().numpy().astype(np.float64) * math.log(2.0)
            for i in range(wl.n_q):
                jm, sm = O.middle_scores(Q, K, spec, i, wl.rope_base, wl.scale)
                g = gsel[i][gsel[i] >= 0]
                assert len(g) == min(kmid, len(jm)), (i, g)
                _check_mid_sel(gsel[i], i, wl)
                if not len(jm):
                    continue
                sc = dict(zip(jm.tolist(), sm.tolist()))
                kth = float(np.sort(sm)[::-1][len(g) - 1])
                eps = 1e-3 * max(1.0, abs(kth))
                for jj, gs in zip(gsel[i][:len(g)], gsc[i][:len(g)]):
                    assert abs(gs - sc[int(jj)]) <= eps, (i, jj, gs, sc[int(jj)])
                diff = set(g.tolist()) ^ set(rsel[i].tolist())
                for jj in diff:
                    assert abs(sc[jj] - kth) <= eps, (i, jj, sc[jj], kth)
                n_near += len(diff) > 0
            compare(to64(o[b, h]), ro, to64(lse[b, h]), rl, "bf16")
    log(f"  queries with a near-tie swap: {n_near}")


def test_workload3_topk_middle_sampled(sa):
    wl = W.WORKLOADS[3]
    kmid = 8
    log("workload 3 top-k middle: inputs")
    inp = W.make_inputs(wl)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    sa_obj = device_mask(wl)
    sa_obj.build_plan()
    lse = torch.empty((wl.batch, wl.h_q, wl.n_q), dtype=torch.float32, device="cuda")
    o = sa_obj.forward(q, k, v, lse=lse, rope_base=wl.rope_base, scale=wl.scale)
    sel, score = sa_obj.topk_middle(q, k, v, o, lse, kmid, rope_base=wl.rope_base, scale=wl.scale)
    torch.cuda.synchronize()
    spec = spec_of(wl)
    r_ = np.random.default_rng(3)
    rows = np.array(sorted(set(range(4090, 4230)) | set(range(wl.n_q - 64, wl.n_q))
                           | set(r_.choice(np.arange(4200, wl.n_q), size=48, replace=False).tolist())))
    for h in (0, 31):
        log(f"workload 3 top-k middle: head {h}")
        Q, K, V = to64(inp["q"][0, h]), to64(inp["k"][0, h]), to64(inp["v"][0, h])
        ro, rl, rsel = O.attention_topk_middle(Q, K, V, rows, spec, wl.rope_base, wl.scale, kmid)
        gsel = sel[0, h].cpu().numpy()
        gsc = score[0, h].cpu().numpy().astype(np.float64) * math.log(2.0)
        for r, i in enumerate(rows):
            jm, sm = O.middle_scores(Q, K, spec, int(i), wl.rope_base, wl.scale)
            g = gsel[i][gsel[i] >= 0]
            assert len(g) == min(kmid, len(jm))
            _check_mid_sel(gsel[i], int(i), wl)
            if not len(jm):
                continue
            sc = dict(zip(jm.tolist(), sm.tolist()))
            kth = float(np.sort(sm)[::-1][len(g) - 1])
            eps = 1e-3 * max(1.0, abs(kth))
            for jj, gs in zip(gsel[i][:len(g)], gsc[i][:len(g)]):
                assert abs(gs - sc[int(jj)]) <= eps
            for jj in set(g.tolist()) ^ set(rsel[r].tolist()):
                assert abs(sc[jj] - kth) <= eps
        compare(to64(o[0, h][torch.from_numpy(rows).cuda()]), ro, to64(lse[0, h][torch.from_numpy(rows).cuda()]),
                rl, "bf16")


# LM-Infinite decode: the starting span and the window t-L .. t, starting keys capped,
# against the oracle's Lambda attention of the new query over its t + 1 tokens.
LAM_DECODE_CASES = [
    dict(B=2, h_q=8, h_kv=2, n_s=4, L=32, n=200, rope=10000.0),
    dict(B=1, h_q=2, h_kv=2, n_s=0, L=16, n=60, rope=None),
    dict(B=1, h_q=4, h_kv=1, n_s=10, L=64, n=150, rope=500000.0),
]


@pytest.mark.parametrize("case", range(len(LAM_DECODE_CASES)))
def test_lambda_decode(sa, case):
    from structured_sparse_attention_attn_amd.pipeline import StreamDecoder
    cfg = LAM_DECODE_CASES[case]
    B, hq, hkv, d = cfg["B"], cfg["h_q"], cfg["h_kv"], 128
    log(f"lambda decode {case}: {cfg}")
    q, k, v, _ = W.make_decode_stream(B, hq, hkv, d, cfg["n"], seed=1500 + case, p_sep=0.0)
    dec = StreamDecoder(B, hq, hkv, d, cfg["n_s"], rope_base=cfg["rope"], kind="lambda", L_pretrain=cfg["L"])
    dec.state.fill_(0xFF)  # NaN bit patterns in every slot not yet written
    dec.reset()
    scale = d ** -0.5
    group = hq // hkv
    lse = torch.empty((B, hq), dtype=torch.float32, device="cuda")
    for t in range(cfg["n"]):
        o = dec.step(q[t].cuda(), k[t].cuda(), v[t].cuda(), lse=lse)
        torch.cuda.synchronize()
        spec = O.MaskSpec(O.LAMBDA, t + 1, t + 1, n_s=cfg["n_s"], L=cfg["L"])
        for b in range(B):
            if t % 5 == 0 or t == cfg["n"] - 1:
                assert dec.held(b) == O.key_set(spec, t).tolist(), (t, b)
            ro = np.zeros((hq, d))
            rl = np.zeros(hq)
            for h in range(hq):
                oo, ll = O.attention_rows(to64(q[:t + 1, b, h]), to64(k[:t + 1, b, h // group]),
                                          to64(v[:t + 1, b, h // group]), [t], spec, cfg["rope"], scale)
                ro[h], rl[h] = oo[0], ll[0]
            compare(to64(o[b]), ro, to64(lse[b]), rl, "bf16")


# Repeat runs and guard canaries beyond the forward: the backward, the top-k middle tokens
# and the streaming decode write only their outputs and give the same bits every time.
def _guarded(shape, dtype, fill=7.0, guard=4096):
    n = int(np.prod(shape))
    store = torch.full((guard * 2 + n,), fill, dtype=dtype, device="cuda")
    return store, store[guard:guard + n].view(shape)


def _guards_intact(store, fill=7.0, guard=4096):
    return bool(torch.all(store[:guard] == fill)) and bool(torch.all(store[-guard:] == fill))


def test_bwd_repeat_and_canary(sa):
    mode, kw, rope, alibi = BWD_SMALL[1]
    wl = W.small(mode, seed=800, rope_base=rope, alibi_exp=alibi, **kw)
    inp = W.make_small_inputs(wl)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    sep = inp.get("sep")
    sa_obj = device_mask(wl, None if sep is None else sep.cuda())
    sa_obj.build_plan()
    lse = torch.empty((wl.batch, wl.h_q, wl.n_q), dtype=torch.float32, device="cuda")
    o = sa_obj.forward(q, k, v, lse=lse, rope_base=rope, scale=wl.scale)
    dout = W.make_grad(tuple(q.shape), seed=801).cuda()
    outs = []
    for rep in range(2):
        sq, dq = _guarded(tuple(q.shape), q.dtype)
        sk, dk = _guarded(tuple(k.shape), k.dtype)
        sv, dv = _guarded(tuple(v.shape), v.dtype)
        sa_obj.backward(q, k, v, o, lse, dout, rope_base=rope, scale=wl.scale, dq=dq, dk=dk, dv=dv)
        torch.cuda.synchronize()
        assert _guards_intact(sq) and _guards_intact(sk) and _guards_intact(sv), rep
        outs.append((dq.clone(), dk.clone(), dv.clone()))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)


def test_topk_middle_repeat_and_canary(sa):
    kw, kmid, rope = MID_CASES[4]
    wl = W.small(W.LAMBDA, seed=810, rope_base=rope, **kw)
    inp = W.make_small_inputs(wl)
    q, k, v = (inp[x].cuda() for x in ("q", "k", "v"))
    sa_obj = device_mask(wl)
    sa_obj.build_plan()
    outs = []
    shp = (wl.batch, wl.h_q, wl.n_q, kmid)
    for rep in range(2):
        so, o = _guarded(tuple(q.shape), q.dtype)
        sl, lse = _guarded((wl.batch, wl.h_q, wl.n_q), torch.float32)
        sa_obj.forward(q, k, v, o=o, lse=lse, rope_base=rope, scale=wl.scale)
        ss, sel = _guarded(shp, torch.int32, fill=7)
        sc, score = _guarded(shp, torch.float32)
        sa.sparse_attn_topk_middle(sa_obj.mask, sa_obj.args(q, k, v, o, lse, rope, wl.scale), kmid, sel, score)
        torch.cuda.synchronize()
        assert all(_guards_intact(x) for x in (so, sl, sc)) and _guards_intact(ss, fill=7), rep
        outs.append((o.clone(), lse.clone(), sel.clone(), score.clone()))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)


def test_topk_repeat_and_canary(sa):
    """topk_retrieve twice on a workspace refilled with arbitrary bytes in
    between: the same indices, scores and copied rows bit for bit, and no write
    outside idx, score or the prefix rows (guard regions around each)."""
    from structured_sparse_attention_attn_amd.pipeline import TopK
    H, n, d, k = 4, 4100, 128, 1500
    q, kp, vp = W.make_pool_inputs(H, n, d, 830, torch.bfloat16)
    qd, kd, vd = q.cuda(), kp.cuda(), vp.cuda()
    topk = TopK(H, n)
    g = torch.Generator(device="cuda").manual_seed(831)
    outs = []
    for rep in range(2):
        topk.ws.copy_(torch.randint(0, 256, topk.ws.shape, generator=g, device="cuda", dtype=torch.int32)
                      .to(torch.uint8))
        si, idx = _guarded((H, k), torch.int32, fill=7)
        ss, score = _guarded((H, k), torch.float64)
        sk, pk = _guarded((H, k, d), torch.bfloat16)
        sv, pv = _guarded((H, k, d), torch.bfloat16)
        topk(qd, kd, k, idx, score=score, pool_v=vd, pref_k=pk, pref_v=pv)
        torch.cuda.synchronize()
        assert _guards_intact(si, fill=7) and all(_guards_intact(x) for x in (ss, sk, sv)), rep
        outs.append((idx.clone(), score.clone(), pk.clone(), pv.clone()))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)
    ri = O.topk_select(O.topk_scores(q[1].double().numpy(), kp[1].double().numpy()), k)
    np.testing.assert_array_equal(outs[0][0][1].cpu().numpy(), ri)


def test_topk_workspace_offset(sa):
    """The C ABI asks only 8-byte alignment of the top-k workspace; the
    launcher rounds up to its sections' 256-byte boundaries inside it."""
    H, n, d, k = 2, 3000, 64, 77
    q, kp, vp = W.make_pool_inputs(H, n, d, 840, torch.float32)
    need = sa.sa_topk_workspace_bytes(H, n)
    buf = torch.zeros(need + 8, dtype=torch.uint8, device="cuda")
    ws = buf[8:]  # 8 bytes past a 256-byte boundary
    assert ws.data_ptr() % 256 == 8
    idx = torch.empty((H, k), dtype=torch.int32, device="cuda")
    score = torch.empty((H, k), dtype=torch.float64, device="cuda")
    sa.topk_retrieve(q.cuda(), kp.cuda(), k, idx, ws, score=score)
    torch.cuda.synchronize()
    for h in range(H):
        s_ = O.topk_scores(q[h].double().numpy(), kp[h].double().numpy())
        ri = O.topk_select(s_, k)
        np.testing.assert_array_equal(idx[h].cpu().numpy(), ri)
        np.testing.assert_array_equal(score[h].cpu().numpy(), s_[ri])


@pytest.mark.parametrize("kind", ["sepllm", "lambda"])
def test_decode_repeat_and_canary(sa, kind):
    from structured_sparse_attention_attn_amd.pipeline import StreamDecoder
    B, hq, hkv, d, n = 2, 8, 2, 128, 200
    q, k, v, flags = W.make_decode_stream(B, hq, hkv, d, n, 820, 0.2)
    decs = [StreamDecoder(B, hq, hkv, d, 4, 8, 16, 60, rope_base=10000.0, kind=kind, L_pretrain=50)
            for _ in range(2)]
    for t in range(n):
        res = []
        for dec in decs:
            so, o = _guarded((B, hq, d), torch.bfloat16)
            sl, lse = _guarded((B, hq), torch.float32)
            dec.step(q[t].cuda(), k[t].cuda(), v[t].cuda(), flags[t].cuda(), o=o, lse=lse)
            res.append((so, sl, o, lse))
        torch.cuda.synchronize()
        for so, sl, _, _ in res:
            assert _guards_intact(so) and _guards_intact(sl), t
        assert torch.equal(res[0][2], res[1][2]) and torch.equal(res[0][3], res[1][3]), t
