"""The forward kernel's online-softmax update rule, replayed on the CPU.

A float32 model of the rule (tests/_softmax_model.py) runs over inputs whose
logit range is wide: queries scaled by 4, and rows whose one key lies 150
natural units above the rest, visited after the keys that set the row's
reference (the capped starting key under LM-Infinite's Lambda mask, visited
last; a SepLLM or segment diagonal key after the gathered separators or the
prefix; the first key under the clipped ALiBi bias, visited last).  The
earlier rule, which divided by the unit's largest weight however large,
yields NaN there; the current rule computes such a unit again with its exact
row maximum and matches the oracle's LSE (SepLLM page, part 6.1: softmax over
the kept entries; LM-Infinite page, section "method": the capped logit).
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from _helpers import spec_of
from _softmax_model import replay, spike_queries

CASES = [
    (W.SEPLLM, dict(m=450, a=4, w=64, p_sep=0.1), 10000.0, None),
    (W.LAMBDA, dict(m=500, n_s=10, L=100), 10000.0, None),
    (W.SEGMENT, dict(m=400, P=200), 10000.0, None),
    (W.LAMBDA, dict(m=600, n_s=10, L=300), None, 8.0),
]


def _inputs(case, spike):
    mode, kw, rope, alibi = CASES[case]
    wl = W.small(mode, seed=500 + case, rope_base=rope, alibi_exp=alibi, **kw)
    inp = W.make_small_inputs(wl)
    sep = inp.get("sep")
    spec = spec_of(wl, None if sep is None else sep.numpy())
    q = inp["q"].double().numpy()
    k = inp["k"].double().numpy()
    slope = (lambda h: O.alibi_slope(h, wl.h_q, alibi)) if alibi else None
    if spike:
        rows = list(range(wl.n_q // 2, wl.n_q, 7))
        q = spike_queries(q, k, spec, rows, 150.0, wl.scale, rope_base=rope, slope=slope,
                          h_q=wl.h_q, h_kv=wl.h_kv)
    else:
        q = q * 4.0
    q = torch.from_numpy(q).to(torch.bfloat16).double().numpy()
    return wl, spec, q, k, inp["v"].double().numpy(), slope


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("spike", [False, True])
def test_update_rule_wide_logits(case, spike):
    wl, spec, q, k, v, slope = _inputs(case, spike)
    s0 = slope(0) if slope else None
    old, lse_old = replay(q[0, 0], k[0, 0], spec, wl.rope_base, wl.scale, slope=s0, old_rule=True)
    new, lse_new = replay(q[0, 0], k[0, 0], spec, wl.rope_base, wl.scale, slope=s0)
    assert new["rescale"]
    _, ref = O.attention(q[0], k[0], v[0], spec, wl.rope_base, wl.scale, heads=[0],
                         alibi_exp=wl.alibi_exp)
    rows = sorted(lse_new)
    ref2 = ref[0][rows] / math.log(2.0)
    got = np.array([lse_new[r] for r in rows])
    # float32 state: m_ref and log2(l) each within a few ulp of values up to ~2^8
    np.testing.assert_allclose(got, ref2, rtol=0, atol=1e-4)
    if spike:
        assert old["overflow"] and new["recompute"]
        assert np.isnan([lse_old[r] for r in rows]).any()
    else:
        assert not new["recompute"]
