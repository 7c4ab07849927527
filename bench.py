#!/usr/bin/env python3
"""Benchmark: one layer of structured sparse causal attention on one MI355X.

A step is one pass of the whole hot path over one batch of seeded synthetic
input already resident in HBM: the plan, the RoPE stage and the fused sparse
forward (plus the top-k retrieval for the segment workload), all 32 heads of
one layer.  The default workload is the 32K LM-Infinite Lambda mask (batch 1,
32 heads, d = 128, n_starting = 10, L_pretrain = 4096, RoPE base 10000), the
configuration the "ms/layer at 32K" figure is quoted on.

Prints one JSON line: effective TFLOP/s over the unmasked pairs
(4 * d * pairs * heads per step / step time), the per-stage times measured
with HIP events on the launch stream, the roofline of the fused forward and
the fp64 CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective TFLOP/s (unmasked pairs) & % bf16 MFMA peak; ms/layer at 32K"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


def pair_count_per_head(wl, sep_np):
    """Exact |A| summed over queries (closed forms of the three key sets)."""
    import numpy as np
    i = np.arange(wl.n_q, dtype=np.int64)
    if wl.mode == "lambda":
        return int((np.minimum(i, wl.L) + 1 + np.minimum(wl.n_s, np.maximum(0, i - wl.L))).sum())
    if wl.mode == "segment":
        return wl.n_q * wl.P + wl.n_q * (wl.n_q + 1) // 2
    # SepLLM: window min(i+1, w) + sinks and separators at j <= i - w
    flags = sep_np.astype(np.int64) * (np.arange(wl.n_k) >= wl.a)
    cs = np.concatenate([[0], np.cumsum(flags)])
    far = i - wl.w
    ok = far >= 0
    extra = np.where(ok, np.minimum(wl.a, far + 1) + cs[np.clip(far + 1, 0, wl.n_k)], 0)
    return int((np.minimum(i + 1, wl.w) + extra).sum())


def issued_flops(wl, host_plan):
    """MFMA work the fused forward issues: every unit of a tile is a full
    64-key x 128-query block (both products), masked pairs included.  With
    RoPE, a Lambda tile's capped blocks get a capped pass, and the ordinary
    pass skips those of them farther than L from the tile's first query."""
    import numpy as np
    tp = host_plan["tile_ptr"].astype(np.int64)
    items = host_plan["items"].astype(np.int64)
    n_items = tp[1:] - tp[:-1]
    n_cap = np.zeros_like(n_items)
    n_skip = np.zeros_like(n_items)
    if wl.mode == "lambda" and wl.rope_base is not None:
        capped = ((items >> 24) & 2) != 0
        tile = np.repeat(np.arange(len(n_items), dtype=np.int64), n_items)
        skip = capped & ((items & 0xFFFFFF) * 64 + 63 < tile * 128 - wl.L)
        cs = np.concatenate([[0], np.cumsum(capped)])
        ks = np.concatenate([[0], np.cumsum(skip)])
        n_cap = cs[tp[1:]] - cs[tp[:-1]]
        n_skip = ks[tp[1:]] - ks[tp[:-1]]
    n_ch = (host_plan["sep_count"].astype(np.int64) + 63) // 64 if wl.mode == "sepllm" else 0
    units = int((n_items - n_skip + n_cap + n_ch).sum())
    return 4.0 * 64 * 128 * wl.d * units * wl.h_q * wl.batch


def stage_bytes(wl, sep_np, plan_bytes):
    """Algorithmic HBM bytes per launch of the plan, RoPE and top-k stages."""
    import numpy as np
    esz = 2 if wl.dtype == "bf16" else 4
    d, B = wl.d, wl.batch
    n_sep = 0
    if wl.mode == "sepllm" and sep_np is not None:
        g0 = 64 * ((wl.a + 63) // 64)
        n_sep = int(sep_np[g0:].astype(np.int64).sum())
    rot = wl.rope_base is not None
    n_cap = min(wl.n_s, wl.n_k) if (wl.mode == "lambda" and rot) else 0
    # the rotated query copy (fp32 only: bf16 queries are rotated and scaled
    # inside the fused forward), rotated keys, the gathered separator rows
    # (read K and V, write both) and the capped keys
    n_qrows = 2 * wl.h_q * wl.n_q if (rot and wl.dtype != "bf16") else 0
    n_krows = 2 * wl.h_kv * wl.n_k if rot else 0
    rope = esz * d * B * (n_qrows + n_krows + 3 * wl.h_kv * n_sep + wl.h_kv * n_cap)
    plan = (wl.n_k if sep_np is not None else 0) + plan_bytes
    out = {"plan": plan, "rope": rope}
    if wl.mode == "segment":
        nl = wl.n_local
        out["topk"] = esz * d * (wl.h_q - nl) * (wl.pool_len + 1 + 4 * wl.P)
    return out


def gemm_ceiling_tflops(torch):
    """Dense bf16 GEMM through torch (hipBLASLt), 16384^3: a measured MFMA ceiling."""
    n = 16384
    a = torch.randn(n, n, dtype=torch.bfloat16, device="cuda")
    b = torch.randn(n, n, dtype=torch.bfloat16, device="cuda")
    for _ in range(3):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    return 2.0 * n ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12


def multi_segment(wl, inp, n_seg, torch):
    """The segment workload run as n_seg consecutive segments of one layer: forward
    (RoPE stage + fused forward), tail carry, pool append and retrieval per segment.
    Every segment reuses the workload's q / K / V (timing only); the pool grows to
    n_seg * S rows."""
    from structured_sparse_attention_attn_amd.pipeline import SegmentRunner
    S, M, H, d, nl = wl.n_q, wl.P, wl.h_q, wl.d, wl.n_local
    run = SegmentRunner(H, nl, d, S, M, n_seg * S, rope_base=wl.rope_base, scale=wl.scale)
    for kb, vb in run.bufs:
        kb[:, :, M:] = inp["k_seg"].to("cuda")
        vb[:, :, M:] = inp["v_seg"].to("cuda")
    q = inp["q"].to("cuda")
    o = torch.empty_like(q)

    def one_pass():
        run.reset()
        for _ in range(n_seg):
            run.step(q, o=o)

    one_pass()  # builds the plans, warms up
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    one_pass()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    pairs = sum(S * min(M, i * S) + S * (S + 1) // 2 for i in range(n_seg)) * H
    return {"segments": n_seg, "ms_per_segment": round(ms / n_seg, 4),
            "effective_tflops": round(4.0 * d * pairs / (ms * 1e-3) / 1e12, 2),
            "pool_rows_final": n_seg * S,
            "note": "forward + tail carry + pool append + top-k retrieval per segment"}


def backward_timing(sa_mod, sa, q, k, v, o, lse, wl, steps, torch):
    """The backward (sparse_attn_bwd: RoPE stage, row sums, dQ, dK/dV, finish) on the
    forward's outputs, timed with HIP events on the launch stream."""
    from structured_sparse_attention_attn_amd import bwd_args, sparse_attn_bwd
    import workloads as W
    dout = W.make_grad(tuple(q.shape), seed=wl.seed + 11).to("cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fa = sa.args(q, k, v, o, lse, wl.rope_base, wl.scale, wl.alibi_exp)
    ga = bwd_args(dout, dq, dk, dv)
    need = sa_mod.sa_bwd_workspace_bytes(sa.mask, fa)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    sparse_attn_bwd(sa.mask, sa.plan, fa, ga, ws)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        sparse_attn_bwd(sa.mask, sa.plan, fa, ga, ws)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, need


def decode_timing(steps, torch, batch=64, graph=False):
    """Streaming decode with the generation-time cache (SepLLM page, part 6.2) for a
    Llama-3-8B-shaped layer (32 query heads on 8 kv heads, d = 128, RoPE 500000): a = 4,
    s = 64, w = 128, c = 324 (the page's PG19 setting s = 64, c = 324).  The cache is run
    to its steady state (several compressions) untimed, then `steps` decode steps are timed.
    Bytes per step: the held K and V rows read once, plus the new rows, queries and
    outputs."""
    import workloads as W
    from structured_sparse_attention_attn_amd.pipeline import StreamDecoder
    B, hq, hkv, d = batch, 32, 8, 128
    a, s, w, c = 4, 64, 128, 324
    dec = StreamDecoder(B, hq, hkv, d, a, s, w, c, rope_base=500000.0)
    q, k, v, flags = W.make_decode_stream(B, hq, hkv, d, 1, seed=7000, p_sep=0.06)
    q, k, v = q[0].cuda(), k[0].cuda(), v[0].cuda()
    fl = (torch.arange(B) % 16 == 0).to(torch.uint8).cuda()  # every 16th sequence sees a separator
    o = torch.empty_like(q)
    for _ in range(600):
        dec.step(q, k, v, fl, o=o)
    torch.cuda.synchronize()
    held = [len(dec.held(b)) for b in range(B)]
    run = (lambda: dec.step(q, k, v, fl, o=o))
    g = None
    if graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run()
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run()
        run = g.replay
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = (sum(held) * hkv * 2 * d * 2 + B * (2 * hq + 2 * hkv) * d * 2)
    return {"config": {"batch": B, "h_q": hq, "h_kv": hkv, "head_dim": d, "a": a, "s": s, "w": w, "c": c,
                       "rope_base": 500000.0},
            "graph": graph, "ms_per_step": round(ms, 5), "tokens_per_s": round(B / (ms * 1e-3), 1),
            "held_slots_mean": round(sum(held) / B, 1),
            "hbm_gbs": round(nbytes / (ms * 1e-3) / 1e9, 1), "bytes_per_step": nbytes}


def topk_middle_timing(sa, q, k, v, o, lse, wl, kmid, steps, torch):
    """LM-Infinite top-k middle tokens on the Lambda layer's forward output: scoring
    of every middle pair (n_starting <= j < i - L) on MFMA, per-query selection, merge."""
    import numpy as np
    from structured_sparse_attention_attn_amd import sparse_attn_topk_middle
    B, h_q, n_q, _ = q.shape
    sel = torch.empty((B, h_q, n_q, kmid), dtype=torch.int32, device="cuda")
    score = torch.empty((B, h_q, n_q, kmid), dtype=torch.float32, device="cuda")
    fa = sa.args(q, k, v, o, lse, wl.rope_base, wl.scale)
    sparse_attn_topk_middle(sa.mask, fa, kmid, sel, score)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        sparse_attn_topk_middle(sa.mask, fa, kmid, sel, score)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    i = np.arange(n_q, dtype=np.int64)
    mid_pairs = int(np.maximum(0, i - wl.L - wl.n_s).sum()) * h_q * B
    flops = 2.0 * wl.d * mid_pairs  # one product per middle pair (the kernel issues two: q high, q low)
    return {"k_mid": kmid, "ms": round(ms, 4), "middle_pairs": mid_pairs,
            "effective_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "issued_tflops": round(2 * flops / (ms * 1e-3) / 1e12, 2),
            "note": "scoring + selection + merge; o, lse rewritten in place (run after the timed forward steps)"}


def lambda_decode_timing(steps, torch, batch=16):
    """LM-Infinite decode (Lambda set of the new query: starting span + window, starting
    keys capped) for a Llama-2-7B-shaped layer: 32 heads, d = 128, n_starting = 10,
    L_pretrain = 4096, RoPE 10000; timed once the window is full (4107 held slots)."""
    import workloads as W
    from structured_sparse_attention_attn_amd.pipeline import StreamDecoder
    B, hq, hkv, d, n_s, L = batch, 32, 32, 128, 10, 4096
    dec = StreamDecoder(B, hq, hkv, d, n_s, rope_base=10000.0, kind="lambda", L_pretrain=L)
    q, k, v, _ = W.make_decode_stream(B, hq, hkv, d, 1, seed=7100, p_sep=0.0)
    q, k, v = q[0].cuda(), k[0].cuda(), v[0].cuda()
    o = torch.empty_like(q)
    for _ in range(n_s + L + 200):
        dec.step(q, k, v, o=o)
    torch.cuda.synchronize()
    held = [len(dec.held(b)) for b in range(B)]
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        dec.step(q, k, v, o=o)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = sum(held) * hkv * 2 * d * 2 + B * (2 * hq + 2 * hkv) * d * 2
    return {"config": {"batch": B, "h_q": hq, "h_kv": hkv, "head_dim": d, "n_starting": n_s, "L_pretrain": L,
                       "rope_base": 10000.0},
            "ms_per_step": round(ms, 5), "tokens_per_s": round(B / (ms * 1e-3), 1),
            "held_slots_mean": round(sum(held) / B, 1),
            "hbm_gbs": round(nbytes / (ms * 1e-3) / 1e9, 1), "bytes_per_step": nbytes}


FWD_SOURCES = ("sa_fwd.hip", "sa_device.h", "sa_common.h")


def source_sha(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def fwd_source_sha():
    """Hash of the sources the fused forward is compiled from."""
    csrc = os.path.join(ROOT, "structured_sparse_attention_attn_amd", "csrc")
    return source_sha([os.path.join(csrc, f) for f in FWD_SOURCES])


ROPE_SOURCES = ("sa_rope.hip", "sa_common.h")


def rope_source_sha():
    """Hash of the sources the RoPE stage is compiled from."""
    csrc = os.path.join(ROOT, "structured_sparse_attention_attn_amd", "csrc")
    return source_sha([os.path.join(csrc, f) for f in ROPE_SOURCES])


def load_traffic(workload_name, stage="attend"):
    """HBM bytes per launch of the fused forward ("attend") or of the RoPE stage
    ("rope") from committed rocprofv3 PMC counters, or None when absent or taken
    on a different kernel source."""
    p = os.path.join(ROOT, "profiles", f"{stage}_{workload_name}_pmc.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("source_sha") != (fwd_source_sha() if stage == "attend" else rope_source_sha()):
        return None
    return (d["fetch_kib"] * d["copy_factor_fetch"] + d["write_kib"] * d["copy_factor_write"]) * 1024.0


_CPU = {}


def _cpu_worker_init():
    try:
        from threadpoolctl import threadpool_limits
        _CPU["limit"] = threadpool_limits(1)  # one thread per process: the pool spreads the work
    except Exception:  # pragma: no cover
        pass


def _cpu_tile(task):
    """One (head, query tile) of the oracle's fast mode; skipped once the deadline passed."""
    import numpy as np

    import oracle as O
    h, t = task
    if time.time() > _CPU["deadline"]:
        return 0, 0
    wl, spec, Q, K, V = _CPU["wl"], _CPU["spec"], _CPU["q"], _CPU["k"], _CPU["v"]
    g = h // (wl.h_q // wl.h_kv)
    rows = np.arange(128 * t, min(wl.n_q, 128 * t + 128))
    slope = None if wl.alibi_exp is None else O.alibi_slope(h, wl.h_q, wl.alibi_exp)
    O.attention_fast(Q[h].astype(np.float64), K[g].astype(np.float64), V[g].astype(np.float64), spec,
                     wl.rope_base, wl.scale, [rows], alibi=slope)
    return int(O.mask_rows(spec, rows).sum()), 1


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(wl, inp, budget_s):
    """The fp64 oracle (as it stands) on a bounded sample of the workload: its fast mode
    over (head, query tile) tasks, last tiles first (the ones with the most keys), in a
    process pool of one single-threaded worker per core this process may run on, for
    about budget_s seconds of wall time.  Run before the GPU is touched."""
    import multiprocessing as mp

    import numpy as np

    import oracle as O
    cores = len(os.sched_getaffinity(0))
    sep = inp.get("sep")
    spec = O.MaskSpec(wl.mode, wl.n_q, wl.n_k, a=wl.a, w=wl.w,
                      sep=None if sep is None else sep.numpy(), n_s=wl.n_s, L=wl.L, P=wl.P)
    if wl.mode == "segment":
        k = np.concatenate([inp["k_tail"][0, :1].float().numpy(), inp["k_seg"][0, :1].float().numpy()], axis=1)
        v = np.concatenate([inp["v_tail"][0, :1].float().numpy(), inp["v_seg"][0, :1].float().numpy()], axis=1)
        q = inp["q"][0, :1].float().numpy()
        heads = [0]
    else:
        q, k, v = (inp[x][0].float().numpy() for x in ("q", "k", "v"))
        heads = list(range(wl.h_q))
    n_tiles = -(-wl.n_q // 128)
    tasks = [(h, t) for t in range(n_tiles - 1, -1, -1) for h in heads]
    _CPU.update(wl=wl if wl.mode != "segment" else dataclass_replace(wl, h_q=1, h_kv=1),
                spec=spec, q=q, k=k, v=v)
    t0 = time.time()
    _CPU["deadline"] = t0 + budget_s
    pairs = done = 0
    # Tasks past the deadline return at once, so the queue drains within the
    # running tasks' time; the pool is then closed and joined without signals
    # (a profiler's signal handler in the forked workers can keep a terminated
    # worker from exiting).
    pool = mp.get_context("fork").Pool(cores, initializer=_cpu_worker_init)
    try:
        for pr, n in pool.imap_unordered(_cpu_tile, tasks, chunksize=1):
            pairs += pr
            done += n
    finally:
        pool.close()
        pool.join()
    el = time.time() - t0
    return {"value": 4.0 * wl.d * pairs / el / 1e12, "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{done} (head, 128-row query tile) tasks of {len(tasks)}, last tiles first, "
                      f"fast mode fp64, {cores} single-threaded processes, {el:.1f} s wall; rate scaled "
                      f"to the effective FLOPs of the sampled rows"}


def dataclass_replace(obj, **kw):
    import dataclasses
    return dataclasses.replace(obj, **kw)


def measure_layer(wl, inp, steps, warmup, torch):
    """Times `steps` passes of the hot path on one workload (inputs moved to HBM first):
    plan, RoPE stage and fused forward (plus top-k retrieval for the segment workload),
    each bracketed by HIP events on the launch stream.  Returns the layer's figures and
    the objects the optional extra measurements reuse."""
    import numpy as np

    from structured_sparse_attention_attn_amd import (fwd_args, plan_to_host, sparse_attn_attend,
                                                      sparse_attn_plan, sparse_attn_rope)
    from structured_sparse_attention_attn_amd.pipeline import SparseAttention, TopK

    dev = "cuda"
    sep = inp.get("sep")
    stream = torch.cuda.current_stream()
    topk = None
    run_topk = None
    if wl.mode == "segment":
        S, P, H, d = wl.n_q, wl.P, wl.h_q, wl.d
        nl = wl.n_local
        q = inp["q"].to(dev)
        k = torch.empty((1, H, P + S, d), dtype=torch.bfloat16, device=dev)
        v = torch.empty_like(k)
        k[:, :, P:] = inp["k_seg"].to(dev)
        v[:, :, P:] = inp["v_seg"].to(dev)
        k[:, :nl, :P] = inp["k_tail"].to(dev)
        v[:, :nl, :P] = inp["v_tail"].to(dev)
        kpool, vpool = inp["k_pool"][0].to(dev), inp["v_pool"][0].to(dev)
        idx = torch.empty((H - nl, P), dtype=torch.int32, device=dev)
        topk = TopK(H - nl, wl.pool_len)

        def run_topk():
            topk(q[0, nl:, S - 1, :], kpool, P, idx, pool_v=vpool, pref_k=k[0, nl:, :P],
                 pref_v=v[0, nl:, :P])
    else:
        q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    sa = SparseAttention(wl.mode, wl.n_q, wl.n_k, a=wl.a, w=wl.w,
                         sep=None if sep is None else sep.to(dev), n_starting=wl.n_s,
                         L_pretrain=wl.L, prefix_len=wl.P)
    o = torch.empty_like(q)
    lse = torch.empty((wl.batch, wl.h_q, wl.n_q), dtype=torch.float32, device=dev)
    fa = fwd_args(q, k, v, o, lse=lse, rope_base=wl.rope_base, scale=wl.scale,
                  alibi_exp=wl.alibi_exp, mask=sa.mask)
    sa.ensure_workspace(fa)
    torch.cuda.synchronize()

    def step(ev):
        ev[0].record(stream)
        if run_topk is not None:
            run_topk()
        ev[1].record(stream)
        sparse_attn_plan(sa.mask, sa.plan)
        ev[2].record(stream)
        sparse_attn_rope(sa.mask, sa.plan, fa, sa.ws)
        ev[3].record(stream)
        sparse_attn_attend(sa.mask, sa.plan, fa, sa.ws)
        ev[4].record(stream)

    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(5)]  # noqa: E731
    for _ in range(warmup):
        step(mk())
    torch.cuda.synchronize()
    evs = [mk() for _ in range(steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for e in evs:
        step(e)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / steps
    stage = {name: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs]))
             for i, name in enumerate(["topk", "plan", "rope", "attend"])}
    if run_topk is None:
        stage.pop("topk")

    def spread(vals):
        x = np.asarray(vals, dtype=np.float64)
        return {"median": round(float(np.median(x)), 4), "p10": round(float(np.percentile(x, 10)), 4),
                "p90": round(float(np.percentile(x, 90)), 4)}

    step_spread = {"step": spread([e[0].elapsed_time(e[4]) for e in evs]),
                   "attend": spread([e[3].elapsed_time(e[4]) for e in evs])}
    in_bytes = sum(t.numel() * t.element_size() for t in (q, k, v, o))
    cache = ("warm: q, k, v and o fit in the 256 MB last-level cache" if in_bytes <= (256 << 20)
             else "cold: q, k, v and o exceed the 256 MB last-level cache")
    pairs_head = pair_count_per_head(wl, None if sep is None else sep.numpy())
    flops = 4.0 * wl.d * pairs_head * wl.h_q * wl.batch
    value = flops / (ms_step * 1e-3) / 1e12
    attend_tflops = flops / (stage["attend"] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(attend_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(attend_tflops / PEAK_BF16_TFLOPS, 4),
                "traffic": load_traffic(wl.name)}
    host_plan = plan_to_host(sa.mask, sa.plan)
    iflops = issued_flops(wl, host_plan)
    issued = {"flops_per_launch": iflops, "ratio_to_effective": round(iflops / flops, 4),
              "tflops": round(iflops / (stage["attend"] * 1e-3) / 1e12, 2),
              "frac": round(iflops / (stage["attend"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    sb = stage_bytes(wl, None if sep is None else sep.numpy(), int(host_plan["header"].total_bytes))
    stage_roofline = {}
    for name_, nbytes in sb.items():
        if name_ in stage and nbytes > 0 and stage[name_] > 0:
            gbs = nbytes / (stage[name_] * 1e-3) / 1e9
            stage_roofline[name_] = {"bound": "hbm", "bytes": nbytes, "achieved": round(gbs, 1),
                                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)}
            if name_ == "rope":
                stage_roofline[name_]["traffic"] = load_traffic(wl.name, "rope")
    res = {
        "value": value, "ms_step": ms_step, "flops": flops, "pairs_head": pairs_head,
        "ms_per_layer": round(stage["rope"] + stage["attend"], 4),
        "pct_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "stages_ms": {k_: round(v_, 4) for k_, v_ in stage.items()},
        "per_step_ms": step_spread, "cache": cache, "roofline": roofline, "issued_mfma": issued,
        "stages_roofline": stage_roofline,
    }
    ctx = dict(sa=sa, q=q, k=k, v=v, o=o, lse=lse)
    return res, ctx


def config_of(wl, pairs_head):
    return {"workload": wl.name, "mode": wl.mode, "batch": wl.batch, "h_q": wl.h_q,
            "h_kv": wl.h_kv, "head_dim": wl.d, "n_q": wl.n_q, "n_k": wl.n_k,
            "a": wl.a, "w": wl.w, "p_sep": wl.p_sep, "n_starting": wl.n_s,
            "L_pretrain": wl.L, "prefix_len": wl.P, "rope_base": wl.rope_base,
            "alibi_exp": wl.alibi_exp, "pairs_per_head": pairs_head}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3, help="1..7 (default: the 32K Lambda layer)")
    ap.add_argument("--no-128k", action="store_true",
                    help="with the default workload, skip the 128K GQA SepLLM layer's sub-object")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    ap.add_argument("--no-gemm-ceiling", action="store_true",
                    help="skip the dense bf16 GEMM reference measurement")
    ap.add_argument("--backward", type=int, default=0,
                    help="also time the backward over this many steps (0: skip)")
    ap.add_argument("--topk-middle", type=int, default=0,
                    help="Lambda workloads: also time the top-k middle tokens with this k (0: skip)")
    ap.add_argument("--decode", type=int, default=0,
                    help="also time this many streaming decode steps (0: skip)")
    ap.add_argument("--segments", type=int, default=8,
                    help="segment workload: also run this many consecutive segments (0: skip)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 256 MiB device copy (scale for PMC byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(heads or query tiles would shard with no or one exchange step)", file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads as W

    wl = W.WORKLOADS[args.workload]
    inp = W.make_inputs(wl)
    # the oracle sample runs first, on the host cores, before the GPU is touched
    cpu = None if args.no_cpu_baseline else cpu_baseline(wl, inp, args.cpu_budget_s)

    torch.cuda.set_device(0)
    res, ctx = measure_layer(wl, inp, args.steps, args.warmup, torch)
    if args.copy_calib:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    props = torch.cuda.get_device_properties(0)
    out = {
        "metric": METRIC,
        "value": round(res["value"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) Q/K/V" + (", Bernoulli separator flags" if "sep" in inp else "")
                + ", resident in HBM)",
        "config": config_of(wl, res["pairs_head"]),
    }
    for key in ("ms_per_layer", "pct_bf16_peak", "stages_ms", "per_step_ms", "cache", "roofline",
                "issued_mfma", "stages_roofline"):
        out[key] = res[key]
    out["device"] = {"name": props.name, "cus": props.multi_processor_count}
    sa, q, k, v, o, lse = (ctx[x] for x in ("sa", "q", "k", "v", "o", "lse"))
    flops = res["flops"]
    if args.backward > 0 and wl.dtype == "bf16":
        import structured_sparse_attention_attn_amd as sa_mod
        bms, bws = backward_timing(sa_mod, sa, q, k, v, o, lse, wl, args.backward, torch)
        bflops = 2.5 * flops  # five products per visible pair (S, dP, dV, dQ, dK) against two
        out["backward"] = {"ms": round(bms, 4), "effective_tflops": round(bflops / (bms * 1e-3) / 1e12, 2),
                           "frac": round(bflops / (bms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                           "workspace_bytes": bws,
                           "note": "2.5x the forward's effective flops (5 products per pair vs 2)"}
    if args.topk_middle > 0 and wl.mode == "lambda" and wl.alibi_exp is None:
        out["topk_middle"] = topk_middle_timing(sa, q, k, v, o, lse, wl, args.topk_middle, 3, torch)
    if args.decode > 0:
        out["decode"] = decode_timing(args.decode, torch)
        out["decode_graph"] = decode_timing(args.decode, torch, graph=True)
        out["decode_lambda"] = lambda_decode_timing(args.decode, torch)
    if wl.mode == "segment" and args.segments > 0:
        out["multi_segment"] = multi_segment(wl, inp, args.segments, torch)
    del ctx, sa, q, k, v, o, lse
    if args.workload == 3 and not args.no_128k:
        # the second configuration the 50%-of-peak target names: 128K GQA SepLLM layer
        wl5 = W.WORKLOADS[5]
        inp5 = W.make_inputs(wl5)
        r5, _ = measure_layer(wl5, inp5, max(3, args.steps // 4), max(1, args.warmup), torch)
        out["w128k"] = {"config": config_of(wl5, r5["pairs_head"]), "steps": max(3, args.steps // 4),
                        "effective_tflops": round(r5["value"], 3), "ms_per_step": round(r5["ms_step"], 4)}
        for key in ("ms_per_layer", "pct_bf16_peak", "stages_ms", "per_step_ms", "cache", "roofline",
                    "issued_mfma", "stages_roofline"):
            out["w128k"][key] = r5[key]
        del inp5
    if not args.no_gemm_ceiling:
        out["gemm_ceiling_tflops"] = round(gemm_ceiling_tflops(torch), 1)
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
