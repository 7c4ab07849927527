"""CPU tests of the C ABI: the library loads, exports every declared symbol,
its structs match the header, and argument checks fail before any launch.
No test here launches device work."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_attn.h")

sa = pytest.importorskip("structured_sparse_attention_attn_amd")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert {"sparse_attn_plan", "sparse_attn_fwd", "topk_retrieve", "sa_last_error"} <= set(names)
    lib = ctypes.CDLL(sa.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", sa.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if " T " in line)
    assert set(names) <= exported


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc missing")
def test_struct_layout_matches_header(tmp_path):
    src = tmp_path / "lay.c"
    src.write_text(r"""
#include <stdio.h>
#include <stddef.h>
#include "sparse_attn.h"
#define P(T, f) printf(#T "." #f " %zu\n", offsetof(T, f));
int main(void) {
  printf("sa_mask_t %zu\nsa_fwd_args_t %zu\nsa_plan_header_t %zu\n", sizeof(sa_mask_t),
         sizeof(sa_fwd_args_t), sizeof(sa_plan_header_t));
  P(sa_mask_t, sep) P(sa_mask_t, prefix_len) P(sa_fwd_args_t, alibi_exp) P(sa_fwd_args_t, q)
  P(sa_fwd_args_t, k_stride)
  P(sa_fwd_args_t, o_stride) P(sa_fwd_args_t, lse) P(sa_plan_header_t, off_tile_ptr)
  P(sa_plan_header_t, total_bytes)
  return 0;
}
""")
    exe = tmp_path / "lay"
    r = subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include", "-I/opt/rocm/include",
                        str(src), "-o", str(exe)], capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("HIP headers not usable with gcc: " + r.stderr[:200])
    got = dict(line.rsplit(" ", 1) for line in subprocess.run([str(exe)], capture_output=True,
                                                              text=True).stdout.splitlines())
    assert int(got["sa_mask_t"]) == ctypes.sizeof(sa.sa_mask_t)
    assert int(got["sa_fwd_args_t"]) == ctypes.sizeof(sa.sa_fwd_args_t)
    assert int(got["sa_plan_header_t"]) == ctypes.sizeof(sa.sa_plan_header_t)
    for key, val in got.items():
        if "." in key:
            T, f = key.split(".")
            assert getattr(getattr(sa, T), f).offset == int(val), key


def _code(fn, *args):
    return fn(*args)


def test_plan_layout_and_validation():
    m = sa.mask(sa.SA_MASK_SEPLLM, 131072, 131072, a=4, w=1024)
    lay = sa.sa_plan_layout(m)
    assert lay.n_tiles == 1024 and lay.n_blocks == 2048 and lay.g0 == 64
    assert lay.max_items_per_tile == 1 + (1024 + 127 + 63) // 64 + 2
    assert lay.total_bytes == sa.sa_plan_bytes(m) and lay.total_bytes % 256 == 0
    offs = [lay.off_tile_ptr, lay.off_items, lay.off_sep_count, lay.off_sep_idx, lay.off_sep_bits,
            lay.off_blk_sep, lay.total_bytes]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    bad = [
        sa.mask(sa.SA_MASK_SEPLLM, 100, 100, a=4, w=0),
        sa.mask(sa.SA_MASK_SEPLLM, 100, 101, a=4, w=3),
        sa.mask(sa.SA_MASK_LAMBDA, 100, 100, n_starting=-1, L_pretrain=5),
        sa.mask(sa.SA_MASK_SEGMENT, 100, 150, prefix_len=49),
        sa.mask(7, 100, 100),
        sa.mask(sa.SA_MASK_LAMBDA, 0, 0),
        sa.mask(sa.SA_MASK_SEPLLM, 100, 100, a=4, w=3, sep_max=-1),
    ]
    for b in bad:
        with pytest.raises(sa.SparseAttnError) as e:
            sa.sa_plan_bytes(b)
        assert e.value.code == sa.SA_EINVAL and sa.sa_last_error()
    lib = sa._lib
    # plan: NULL buffer and too-small buffer are refused before any launch
    assert lib.sparse_attn_plan(ctypes.byref(m), None, 1 << 30, None) == sa.SA_EINVAL
    assert lib.sparse_attn_plan(ctypes.byref(m), 256, 1024, None) == sa.SA_ENOSPACE
    assert "too small" in sa.sa_last_error()
    # plan status: NULL or header-less buffers are refused before any device call
    assert lib.sa_plan_status(None, 1 << 20, None, None) == sa.SA_EINVAL
    assert lib.sa_plan_status(256, 16, None, None) == sa.SA_EINVAL


def test_sep_max_bounds_plan_and_workspace():
    """A caller bound on the separators sizes the plan's sep_idx section and the gathered
    separator rows of the forward and backward workspaces instead of n_k."""
    n = 131072
    sep = 1 << 20  # any non-NULL device address: layouts never dereference it
    free = sa.mask(sa.SA_MASK_SEPLLM, n, n, a=4, w=1024)
    free.sep = sep
    lay0 = sa.sa_plan_layout(free)
    assert lay0.cap_sep == n
    args = _args()
    w0 = sa.sa_fwd_workspace_layout(free, args)
    assert w0.sep_rows == n
    for bound, rows in ((8000, 8000), (8001, 8064), (1, 64), (n + 5, n)):
        m = sa.mask(sa.SA_MASK_SEPLLM, n, n, a=4, w=1024, sep_max=bound)
        m.sep = sep
        lay = sa.sa_plan_layout(m)
        assert lay.cap_sep == min(bound, n)
        assert lay.total_bytes < lay0.total_bytes or bound >= n
        w = sa.sa_fwd_workspace_layout(m, args)
        assert w.sep_rows == rows
        assert w.vsep - w.ksep == w.sep_rows * 128 * 2 * args.h_kv
        assert (w.total < w0.total) == (bound < n)
        assert sa.sa_bwd_workspace_bytes(m, args) <= sa.sa_bwd_workspace_bytes(free, args)
    # other kinds ignore the field
    lam = sa.mask(sa.SA_MASK_LAMBDA, n, n, n_starting=10, L_pretrain=4096, sep_max=-3)
    assert sa.sa_plan_layout(lam).cap_sep == 0


def _args(**kw):
    a = sa.sa_fwd_args_t()
    a.dtype, a.batch, a.h_q, a.h_kv, a.d = sa.SA_BF16, 1, 4, 2, 128
    a.rope, a.rope_base, a.scale = sa.SA_ROPE_HALF, 10000.0, 0.088
    for name in ("q", "k", "v", "o"):
        setattr(a, name, 4096)
        getattr(a, name + "_stride")[:] = [4 * 300 * 128, 300 * 128, 128]
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_fwd_workspace_and_validation():
    lib = sa._lib
    m = sa.mask(sa.SA_MASK_LAMBDA, 300, 300, n_starting=10, L_pretrain=100)
    a = _args()
    ws = sa.sa_fwd_workspace_bytes(m, a)
    # rotated k (2 heads) plus 64 capped-key rows per kv head (bf16 queries are
    # rotated inside the forward)
    expect = 2 * 300 * 256 + 2 * 64 * 256
    assert ws >= expect and ws - expect < 3 * 256
    # the backward also keeps the rotated, scaled queries (4 heads)
    bws = sa.sa_bwd_workspace_bytes(m, a)
    assert bws >= expect + 4 * 300 * 256
    plan_bytes = sa.sa_plan_bytes(m)
    cases = [
        (dict(dtype=5), sa.SA_EINVAL),
        (dict(d=96), sa.SA_EUNSUPPORTED),
        (dict(h_q=3), sa.SA_EINVAL),
        (dict(rope=9), sa.SA_EINVAL),
        (dict(rope_base=0.5), sa.SA_EINVAL),
        (dict(q=None), sa.SA_EINVAL),
        (dict(k=4100), sa.SA_EINVAL),  # misaligned
        (dict(batch=0), sa.SA_EINVAL),
        (dict(rope=sa.SA_ALIBI, alibi_exp=0.0), sa.SA_EINVAL),
        (dict(rope=sa.SA_ALIBI, alibi_exp=float("inf")), sa.SA_EINVAL),
    ]
    for kw, code in cases:
        assert lib.sparse_attn_fwd(ctypes.byref(m), 256, plan_bytes, ctypes.byref(_args(**kw)), 512,
                                   ws, None) == code, kw
    bad_stride = _args()
    bad_stride.v_stride[2] = 100  # 200 bytes: not a multiple of 16
    assert lib.sparse_attn_fwd(ctypes.byref(m), 256, plan_bytes, ctypes.byref(bad_stride), 512, ws,
                               None) == sa.SA_EINVAL
    # a token stride past 64 MiB: block rows are addressed with 32-bit offsets
    huge_stride = _args()
    huge_stride.k_stride[2] = (1 << 25) + 8  # bf16 elements: 64 MiB + 16 bytes
    assert lib.sparse_attn_fwd(ctypes.byref(m), 256, plan_bytes, ctypes.byref(huge_stride), 512, ws,
                               None) == sa.SA_EUNSUPPORTED
    assert lib.sparse_attn_fwd(ctypes.byref(m), 256, plan_bytes - 1, ctypes.byref(a), 512, ws,
                               None) == sa.SA_ENOSPACE
    assert lib.sparse_attn_fwd(ctypes.byref(m), 256, plan_bytes, ctypes.byref(a), 512, ws - 1,
                               None) == sa.SA_ENOSPACE
    assert lib.sparse_attn_fwd(ctypes.byref(m), None, plan_bytes, ctypes.byref(a), 512, ws,
                               None) == sa.SA_EINVAL
    # the ALiBi bias: Lambda masks only; nothing rotated, so the forward needs no workspace
    # (its queries are scaled in registers) and the backward only the scaled queries
    al = _args(rope=sa.SA_ALIBI, alibi_exp=8.0)
    assert sa.sa_fwd_workspace_bytes(m, al) == 0
    assert sa.sa_bwd_workspace_bytes(m, al) >= 4 * 300 * 256
    ms = sa.mask(sa.SA_MASK_SEPLLM, 300, 300, a=4, w=16)
    assert lib.sparse_attn_fwd(ctypes.byref(ms), 256, sa.sa_plan_bytes(ms), ctypes.byref(al), 512,
                               1 << 20, None) == sa.SA_EUNSUPPORTED
    assert "LAMBDA" in sa.sa_last_error()


def test_topk_validation():
    lib = sa._lib
    # 256-byte alignment slack, order keys, buckets, maxima of 16 buckets
    ws = 256 + 8 * 32768 * 8 + 8 * 32768 * 2 + 8 * 2048 * 2
    assert sa.sa_topk_workspace_bytes(8, 32768) == ws
    # rows padded to 64 entries per head, each section to 256 bytes
    assert sa.sa_topk_workspace_bytes(3, 100) == 256 + 3 * 128 * 8 + 3 * 128 * 2 + 256
    args = [sa.SA_BF16, 8, 32768, 128, 1024, 256, 128, 512, None, 32768 * 128, 128, 768, None,
            None, None, 0, 0, 1024, ws, None]
    for pos, val, code in [(4, 0, sa.SA_EINVAL), (4, 32769, sa.SA_EINVAL), (3, 96, sa.SA_EUNSUPPORTED),
                           (0, 3, sa.SA_EINVAL), (18, 100, sa.SA_ENOSPACE), (5, None, sa.SA_EINVAL)]:
        a = list(args)
        a[pos] = val
        assert lib.topk_retrieve(*a) == code, (pos, val)
    # gather requested without destination rows
    a = list(args)
    a[8] = 4096
    assert lib.topk_retrieve(*a) == sa.SA_EINVAL


def test_topk_binding_rejects_mismatched_tensors():
    # checked in the binding before the C call (CPU tensors: no device is touched)
    import torch
    H, n, d, k = 3, 500, 64, 10
    bf = torch.bfloat16
    pk, pv = torch.zeros(H, n, d, dtype=bf), torch.zeros(H, n, d, dtype=bf)
    q = torch.zeros(H, d, dtype=bf)
    idx, score = torch.zeros(H, k, dtype=torch.int32), torch.zeros(H, k, dtype=torch.float64)
    rk, rv = torch.zeros(H, k, d, dtype=bf), torch.zeros(H, k, d, dtype=bf)
    ws = torch.zeros(sa.sa_topk_workspace_bytes(H, n), dtype=torch.uint8)
    good = dict(score=score, pool_v=pv, pref_k=rk, pref_v=rv)

    def call(q_=q, pk_=pk, idx_=idx, **kw):
        args = dict(good)
        args.update(kw)
        sa.topk_retrieve(q_, pk_, k, idx_, ws, **args)

    bad = [
        dict(pk_=torch.zeros(H, n, d, dtype=torch.float16)),          # dtype
        dict(pk_=torch.zeros(n, d, dtype=bf)),                        # rank
        dict(q_=torch.zeros(H + 1, d, dtype=bf)),                     # query rows
        dict(q_=torch.zeros(H, d, dtype=torch.float32)),              # query dtype
        dict(idx_=torch.zeros(H, k - 1, dtype=torch.int32)),          # short idx
        dict(idx_=torch.zeros(H, k, dtype=torch.int64)),              # idx dtype
        dict(idx_=torch.zeros(k, H, dtype=torch.int32).t()),          # not contiguous
        dict(score=torch.zeros(H, k, dtype=torch.float32)),           # score dtype
        dict(pool_v=torch.zeros(H, n + 1, d, dtype=bf)),              # pool_v shape
        dict(pool_v=torch.zeros(H, d, n, dtype=bf).transpose(1, 2)),  # pool_v strides
        dict(pref_k=None),                                            # rows without a destination
        dict(pref_k=torch.zeros(H, k - 1, d, dtype=bf)),              # too few prefix rows
        dict(pref_v=torch.zeros(H, k + 5, d, dtype=bf)),              # pref_v strides differ
    ]
    for case in bad:
        with pytest.raises(ValueError):
            call(**case)


def test_decode_binding_rejects_mismatched_tensors():
    # checked in the binding before the C call (CPU tensors: no device is touched)
    import torch
    B, hq, hkv, d = 2, 8, 2, 128
    cfg = sa.stream_cfg(B, hq, hkv, d, 4, 8, 16, 60, rope_base=10000.0)
    state = torch.zeros(64, dtype=torch.uint8)
    bf = torch.bfloat16
    good = dict(q=torch.zeros(B, hq, d, dtype=bf), k=torch.zeros(B, hkv, d, dtype=bf),
                v=torch.zeros(B, hkv, d, dtype=bf), is_sep=torch.zeros(B, dtype=torch.uint8),
                o=torch.zeros(B, hq, d, dtype=bf), lse=torch.zeros(B, hq))
    bad = [dict(q=torch.zeros(B, hq + 1, d, dtype=bf)), dict(q=torch.zeros(B, hq, d)),
           dict(k=torch.zeros(B, hq, d, dtype=bf)), dict(v=torch.zeros(B, hkv, d, dtype=torch.float16)),
           dict(is_sep=torch.zeros(B, dtype=torch.int32)), dict(o=torch.zeros(B, d, hq, dtype=bf).transpose(1, 2)),
           dict(lse=torch.zeros(B, hq, dtype=torch.float64)), dict(lse=torch.zeros(B + 1, hq))]
    for case in bad:
        t = dict(good)
        t.update(case)
        with pytest.raises(ValueError):
            sa.sparse_attn_decode_step(cfg, state, t["q"], t["k"], t["v"], t["is_sep"], t["o"], state,
                                       lse=t["lse"])
        with pytest.raises(ValueError):
            sa.sparse_attn_decode_step_static(cfg, state, t["q"], t["k"], t["v"], t["is_sep"], t["o"],
                                              lse=t["lse"])


def test_carry_binding_rejects_mismatched_tensors():
    # checked in the binding before the C call (CPU tensors: no device is touched)
    import torch
    H, nl, P, S, M, cap, d = 4, 2, 16, 32, 16, 128, 64
    bf = torch.bfloat16
    good = dict(k=torch.zeros(H, P + S, d, dtype=bf), v=torch.zeros(H, P + S, d, dtype=bf),
                tail_k=torch.zeros(nl, M, d, dtype=bf), tail_v=torch.zeros(nl, M, d, dtype=bf),
                pool_k=torch.zeros(H - nl, cap, d, dtype=bf), pool_v=torch.zeros(H - nl, cap, d, dtype=bf))
    bad = [dict(k=torch.zeros(H, P + S - 1, d, dtype=bf), v=torch.zeros(H, P + S - 1, d, dtype=bf)),
           dict(v=torch.zeros(H, P + S, d)),
           dict(tail_k=torch.zeros(nl, M - 1, d, dtype=bf), tail_v=torch.zeros(nl, M - 1, d, dtype=bf)),
           dict(tail_k=torch.zeros(nl + 1, M, d, dtype=bf), tail_v=torch.zeros(nl + 1, M, d, dtype=bf)),
           dict(pool_k=torch.zeros(H - nl, cap, d + 8, dtype=bf), pool_v=torch.zeros(H - nl, cap, d + 8, dtype=bf)),
           dict(pool_v=torch.zeros(H - nl, cap, d, dtype=torch.float16)),
           dict(pool_v=torch.zeros(H - nl, d, cap, dtype=bf).transpose(1, 2))]
    for case in bad:
        t = dict(good)
        t.update(case)
        with pytest.raises(ValueError):
            sa.sparse_attn_segment_carry(t["k"], t["v"], nl, P, S, M, t["tail_k"], t["tail_v"], t["pool_k"],
                                         t["pool_v"], 0)


def test_import_fails_loudly_without_library(tmp_path):
    # a copy of the binding next to no library must refuse to import
    pkg = tmp_path / "sa_copy"
    pkg.mkdir()
    shutil.copy(os.path.join(os.path.dirname(sa.__file__), "__init__.py"), pkg / "__init__.py")
    r = subprocess.run(["python", "-c", "import sa_copy"], cwd=tmp_path, capture_output=True, text=True)
    assert r.returncode != 0 and "is missing" in r.stderr


def test_segment_carry_validation():
    lib = sa._lib
    H, nl, d, P, S, M = 4, 2, 128, 64, 100, 64
    row = d * 2
    kv = 1 << 20                       # fake device addresses: only host checks run
    hs = (P + S) * d
    args = dict(dtype=sa.SA_BF16, n_heads=H, n_local=nl, d=d, prefix_len=P, seg_len=S, tail_len=M,
                k=kv, v=kv + (1 << 24), kv_hs=hs, kv_rs=d,
                tail_k=kv + (2 << 24), tail_v=kv + (3 << 24), t_hs=M * d, t_rs=d,
                pool_k=kv + (4 << 24), pool_v=kv + (5 << 24), p_hs=1000 * d, p_rs=d,
                pool_len=0, pool_cap=1000)

    def call(**kw):
        a = dict(args, **kw)
        return lib.sparse_attn_segment_carry(
            a["dtype"], a["n_heads"], a["n_local"], a["d"], a["prefix_len"], a["seg_len"],
            a["tail_len"], a["k"], a["v"], a["kv_hs"], a["kv_rs"], a["tail_k"], a["tail_v"],
            a["t_hs"], a["t_rs"], a["pool_k"], a["pool_v"], a["p_hs"], a["p_rs"], a["pool_len"],
            a["pool_cap"], None)
    assert call(dtype=7) == sa.SA_EINVAL
    assert call(n_local=5) == sa.SA_EINVAL
    assert call(d=4) == sa.SA_EINVAL                       # 8 bytes: not a multiple of 16
    assert call(pool_len=950) == sa.SA_ENOSPACE            # 950 + 100 > 1000
    assert call(t_rs=d - 8) == sa.SA_EINVAL                # destination rows overlap
    assert call(k=kv + 8) == sa.SA_EINVAL                  # misaligned
    assert call(tail_k=0) == sa.SA_EINVAL                  # NULL tail with local heads
    # in place: the tail written to rows 0..M-1 of the same buffer whose rows
    # P+S-M .. P+S-1 are read overlaps when P + S < 2 M
    assert call(tail_k=kv, tail_v=kv + (1 << 24), t_hs=(60 + 40) * d, kv_hs=100 * d, prefix_len=60,
                seg_len=40, tail_len=64) == sa.SA_EINVAL
    assert "overlap" in sa.sa_last_error()
    # the pool written over the segment rows it reads
    assert call(pool_k=kv + nl * hs * 2 + P * row, p_hs=hs) == sa.SA_EINVAL
    # nothing to do (no local rows kept, no long heads): returns before any device call
    assert call(n_local=H, tail_len=0) == sa.SA_OK



def _grads(**kw):
    g = sa.sa_bwd_args_t()
    for name in ("dout", "dq", "dk", "dv"):
        setattr(g, name, 4096)
        getattr(g, name + "_stride")[:] = [4 * 300 * 128, 300 * 128, 128]
    for k, v in kw.items():
        setattr(g, k, v)
    return g


def test_bwd_validation():
    lib = sa._lib
    m = sa.mask(sa.SA_MASK_LAMBDA, 300, 300, n_starting=10, L_pretrain=100)
    plan_bytes = sa.sa_plan_bytes(m)
    a = _args(lse=8192)
    ws = sa.sa_bwd_workspace_bytes(m, a)

    def call(args=a, grads=_grads(), plan=256, pb=plan_bytes, wsp=1 << 20, wsb=ws):
        return lib.sparse_attn_bwd(ctypes.byref(m), plan, pb, ctypes.byref(args),
                                   None if grads is None else ctypes.byref(grads), wsp, wsb, None)

    assert call(args=_args()) == sa.SA_EINVAL and "lse" in sa.sa_last_error()  # no lse
    assert call(args=_args(lse=8192, d=96)) == sa.SA_EUNSUPPORTED  # d is 64 or 128
    # fp32 gradients: 16-byte rows checked with 4-byte elements (a 4-element row stride is 16 bytes
    # in fp32 but only 8 in bf16)
    g4 = _grads()
    g4.dq_stride[2] = 4
    assert call(args=_args(lse=8192, dtype=sa.SA_F32, d=64), grads=g4, wsp=None) == sa.SA_EINVAL
    assert "workspace" in sa.sa_last_error()
    assert call(grads=g4) == sa.SA_EINVAL and "dq" in sa.sa_last_error()
    assert call(grads=None) == sa.SA_EINVAL
    assert call(grads=_grads(dout=None)) == sa.SA_EINVAL
    bad = _grads()
    bad.dk_stride[1] = 100  # 200 bytes: not a multiple of 16
    assert call(grads=bad) == sa.SA_EINVAL
    assert call(plan=None) == sa.SA_EINVAL
    assert call(pb=plan_bytes - 1) == sa.SA_ENOSPACE
    assert call(wsb=ws - 1) == sa.SA_ENOSPACE
    assert call(wsp=None) == sa.SA_EINVAL


def test_stream_cfg_validation():
    ok = sa.stream_cfg(2, 8, 2, 128, 4, 8, 16, 60, rope_base=10000.0)
    assert sa.sa_stream_state_bytes(ok) > 0 and sa.sa_decode_workspace_bytes(ok) > 0
    lam = sa.stream_cfg(2, 8, 2, 128, 10, rope_base=10000.0, kind=sa.SA_MASK_LAMBDA, L_pretrain=4096,
                        s=0, w=0, c=0)
    assert sa.sa_stream_state_bytes(lam) > 0
    bad = [
        (sa.stream_cfg(2, 8, 2, 128, 4, 8, 16, 28), sa.SA_EINVAL),          # c <= a + s + w
        (sa.stream_cfg(2, 8, 2, 128, 4, 0, 16, 60), sa.SA_EINVAL),          # s = 0
        (sa.stream_cfg(2, 8, 2, 128, 4, 8, 16, 5000), sa.SA_EUNSUPPORTED),  # c > 4096
        (sa.stream_cfg(2, 18, 2, 128, 4, 8, 16, 60), sa.SA_EUNSUPPORTED),   # 9 query heads per kv head
        (sa.stream_cfg(2, 8, 3, 128, 4, 8, 16, 60), sa.SA_EINVAL),          # h_q not a multiple of h_kv
        (sa.stream_cfg(2, 8, 2, 64, 4, 8, 16, 60), sa.SA_EUNSUPPORTED),     # d = 64
        (sa.stream_cfg(0, 8, 2, 128, 4, 8, 16, 60), sa.SA_EINVAL),          # batch 0
        (sa.stream_cfg(2, 8, 2, 128, 4, 8, 16, 60, rope_base=0.5), sa.SA_EINVAL),
        (sa.stream_cfg(2, 8, 2, 128, 4, 8, 16, 60, kind=7), sa.SA_EINVAL),
        (sa.stream_cfg(2, 8, 2, 128, 10, 0, 0, 0, kind=sa.SA_MASK_LAMBDA, L_pretrain=65530), sa.SA_EINVAL),
    ]
    for cfg, code in bad:
        with pytest.raises(sa.SparseAttnError) as e:
            sa.sa_stream_state_bytes(cfg)
        assert e.value.code == code, (cfg.batch, cfg.h_q, cfg.h_kv, cfg.d, cfg.a, cfg.s, cfg.w, cfg.c)
    # decode step: state and workspace sizes are checked before any launch
    lib = sa._lib
    sb, wb = sa.sa_stream_state_bytes(ok), sa.sa_decode_workspace_bytes(ok)
    step = lambda st, sbytes, w, wbytes, is_sep=512: lib.sparse_attn_decode_step(  # noqa: E731
        ctypes.byref(ok), st, sbytes, 256, 256, 256, is_sep, 256, None, w, wbytes, None)
    assert step(1 << 20, sb - 1, 1 << 24, wb) == sa.SA_ENOSPACE
    assert step(1 << 20, sb, 1 << 24, wb - 1) == sa.SA_ENOSPACE
    assert step(None, sb, 1 << 24, wb) == sa.SA_EINVAL
    assert step(1 << 20, sb, 1 << 24, wb, is_sep=None) == sa.SA_EINVAL  # SEPLLM needs the flags


def test_topk_middle_validation():
    lib = sa._lib
    lam = sa.mask(sa.SA_MASK_LAMBDA, 300, 300, n_starting=10, L_pretrain=100)
    sep = sa.mask(sa.SA_MASK_SEPLLM, 300, 300, a=4, w=16)
    a = _args(lse=8192)
    call = lambda m, args, k: lib.sparse_attn_topk_middle(ctypes.byref(m), ctypes.byref(args), k,  # noqa: E731
                                                          1 << 20, 1 << 21, None)
    assert call(sep, a, 4) == sa.SA_EINVAL
    assert call(lam, _args(lse=8192, rope=sa.SA_ALIBI, alibi_exp=8.0), 4) == sa.SA_EUNSUPPORTED
    assert call(lam, _args(lse=8192, dtype=sa.SA_F32, d=64), 4) == sa.SA_EUNSUPPORTED
    assert call(lam, a, 0) == sa.SA_EINVAL and call(lam, a, sa.SA_TOPK_MIDDLE_MAX + 1) == sa.SA_EINVAL
    assert call(lam, _args(), 4) == sa.SA_EINVAL  # no lse


def test_binding_rejects_mismatched_tensors():
    """The ctypes binding checks what the C ABI cannot see (it receives pointers and strides
    only): shapes against the mask and each other, one dtype and device, the lse buffer, the
    gradient buffers, and the top-k middle-token outputs.  CPU tensors: nothing is launched."""
    import torch
    m = sa.mask(sa.SA_MASK_LAMBDA, 300, 300, n_starting=10, L_pretrain=100)
    bf = torch.bfloat16
    q = torch.zeros((1, 4, 300, 128), dtype=bf)
    k = torch.zeros((1, 2, 300, 128), dtype=bf)
    lse = torch.zeros((1, 4, 300), dtype=torch.float32)
    sa.fwd_args(q, k, k, q.clone(), lse=lse, mask=m)  # accepted
    bad = [
        dict(k=torch.zeros((1, 2, 299, 128), dtype=bf)),                 # n_k differs from the mask
        dict(q=torch.zeros((1, 4, 299, 128), dtype=bf)),                 # n_q differs from the mask
        dict(v=torch.zeros((1, 2, 300, 128), dtype=torch.float32)),      # dtype differs
        dict(o=torch.zeros((1, 3, 300, 128), dtype=bf)),                 # o not shaped like q
        dict(v=torch.zeros((1, 2, 300, 64), dtype=bf)),                  # d differs
        dict(lse=torch.zeros((1, 4, 300), dtype=bf)),                    # lse not float32
        dict(lse=torch.zeros((1, 4, 299), dtype=torch.float32)),         # lse too short
        dict(lse=torch.zeros((1, 300, 4), dtype=torch.float32).transpose(1, 2)),  # not contiguous
        dict(q=torch.zeros((1, 4, 300, 128), dtype=torch.float16)),      # unsupported dtype
    ]
    for kw in bad:
        t = dict(q=q, k=k, v=k, o=q.clone(), lse=lse)
        t.update(kw)
        with pytest.raises(ValueError):
            sa.fwd_args(t["q"], t["k"], t["v"], t["o"], lse=t["lse"], mask=m)
    # gradient buffers shaped like q (dout, dq) and k (dk, dv)
    sa.bwd_args(q, q, k, k, q=q, k=k)
    for args in ((q[:, :3], q, k, k), (q, q, k[:, :1], k), (q, q, k, k.float())):
        with pytest.raises(ValueError):
            sa.bwd_args(*args, q=q, k=k)
    # top-k middle tokens: sel int32 and score float32 [B, h_q, n_q, k_mid], contiguous
    a = sa.fwd_args(q, k, k, q.clone(), lse=lse, mask=m)
    for sel, score in ((torch.zeros((1, 4, 300, 7), dtype=torch.int32), torch.zeros((1, 4, 300, 8))),
                       (torch.zeros((1, 4, 300, 8), dtype=torch.int64), torch.zeros((1, 4, 300, 8))),
                       (torch.zeros((1, 4, 300, 8), dtype=torch.int32), torch.zeros((1, 4, 300, 8), dtype=bf))):
        with pytest.raises(ValueError):
            sa.sparse_attn_topk_middle(m, a, 8, sel, score)
