"""Python binding of libsparse_attn.so (ctypes; argument marshalling only).

The functions below carry the C ABI's names and call it directly; every step
of the computation runs in the library's HIP kernels.  torch tensors supply
device memory and the current HIP stream.  Importing this module fails loudly
when the library has not been built: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsparse_attn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python structured_sparse_attention_attn_amd/build.py` "
        "(the sparse attention path has no fallback)")

# torch is imported first so the library binds to the HIP runtime torch
# already loaded (same SONAME): one runtime per process, shared device
# pointers and streams.  Loading a second copy of the runtime next to torch's
# leaves one of the two without a device.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

SA_OK, SA_EINVAL, SA_EUNSUPPORTED, SA_ENOSPACE, SA_EHIP = 0, -1, -2, -3, -4
SA_MASK_SEPLLM, SA_MASK_LAMBDA, SA_MASK_SEGMENT = 0, 1, 2
SA_F32, SA_BF16 = 0, 1
SA_ROPE_NONE, SA_ROPE_HALF, SA_ALIBI = 0, 1, 2
SA_TQ, SA_BK = 128, 64
SA_TOPK_MIDDLE_MAX = 64
SA_DECODE_STATIC_SCRATCH_BYTES = 32 << 20
SA_ITEM_FULL, SA_ITEM_CAPPED = 1, 2

_i32, _i64, _f32, _vp, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


class sa_mask_t(ctypes.Structure):
    _fields_ = [("kind", _i32), ("n_q", _i32), ("n_k", _i32), ("a", _i32), ("w", _i32),
                ("sep", _vp), ("n_starting", _i32), ("L_pretrain", _i32), ("prefix_len", _i32),
                ("sep_max", _i32)]


class sa_plan_header_t(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint32), ("version", _i32), ("kind", _i32), ("tq", _i32),
                ("bk", _i32), ("n_q", _i32), ("n_k", _i32), ("n_tiles", _i32), ("n_blocks", _i32),
                ("n_items", _i32), ("n_sep", _i32), ("g0", _i32), ("cap_items", _i32),
                ("cap_sep", _i32), ("max_items_per_tile", _i32), ("reserved", _i32),
                ("off_tile_ptr", _i64), ("off_items", _i64), ("off_sep_count", _i64),
                ("off_sep_idx", _i64), ("off_sep_bits", _i64), ("off_blk_sep", _i64),
                ("total_bytes", _i64)]


class sa_fwd_args_t(ctypes.Structure):
    _fields_ = [("dtype", _i32), ("batch", _i32), ("h_q", _i32), ("h_kv", _i32), ("d", _i32),
                ("rope", _i32), ("rope_base", _f32), ("scale", _f32), ("alibi_exp", _f32),
                ("q", _vp), ("q_stride", _i64 * 3), ("k", _vp), ("k_stride", _i64 * 3),
                ("v", _vp), ("v_stride", _i64 * 3), ("o", _vp), ("o_stride", _i64 * 3),
                ("lse", _vp)]


class sa_fwd_ws_layout_t(ctypes.Structure):
    _fields_ = [("krot", _i64), ("ksep", _i64), ("vsep", _i64), ("kcap", _i64), ("qrot", _i64),
                ("sep_rows", _i64), ("cap_rows", _i64), ("total", _i64)]


class sa_bwd_args_t(ctypes.Structure):
    _fields_ = [("dout", _vp), ("dout_stride", _i64 * 3), ("dq", _vp), ("dq_stride", _i64 * 3),
                ("dk", _vp), ("dk_stride", _i64 * 3), ("dv", _vp), ("dv_stride", _i64 * 3)]


class sa_stream_cfg_t(ctypes.Structure):
    _fields_ = [("batch", _i32), ("h_q", _i32), ("h_kv", _i32), ("d", _i32), ("a", _i32), ("s", _i32),
                ("w", _i32), ("c", _i32), ("rope", _i32), ("rope_base", _f32), ("scale", _f32),
                ("kind", _i32), ("L_pretrain", _i32)]


_MASKP = ctypes.POINTER(sa_mask_t)
_ARGSP = ctypes.POINTER(sa_fwd_args_t)
_lib.sa_last_error.restype = ctypes.c_char_p
_lib.sa_last_error.argtypes = []
_lib.sa_plan_layout.argtypes = [_MASKP, ctypes.POINTER(sa_plan_header_t)]
_lib.sa_plan_bytes.argtypes = [_MASKP, ctypes.POINTER(_sz)]
_lib.sparse_attn_plan.argtypes = [_MASKP, _vp, _sz, _vp]
_lib.sa_plan_status.argtypes = [_vp, _sz, _vp, ctypes.POINTER(sa_plan_header_t)]
_lib.sa_fwd_workspace_bytes.argtypes = [_MASKP, _ARGSP, ctypes.POINTER(_sz)]
_lib.sa_fwd_workspace_layout.argtypes = [_MASKP, _ARGSP, ctypes.POINTER(sa_fwd_ws_layout_t)]
_lib.sparse_attn_fwd.argtypes = [_MASKP, _vp, _sz, _ARGSP, _vp, _sz, _vp]
_lib.sparse_attn_rope.argtypes = [_MASKP, _vp, _sz, _ARGSP, _vp, _sz, _vp]
_lib.sparse_attn_attend.argtypes = [_MASKP, _vp, _sz, _ARGSP, _vp, _sz, _vp]
_lib.sa_topk_workspace_bytes.argtypes = [_i32, _i32, ctypes.POINTER(_sz)]
_lib.topk_retrieve.argtypes = [_i32, _i32, _i32, _i32, _i32, _vp, _i64, _vp, _vp, _i64, _i64,
                               _vp, _vp, _vp, _vp, _i64, _i64, _vp, _sz, _vp]
_lib.sparse_attn_segment_carry.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _i64,
                                           _i64, _vp, _vp, _i64, _i64, _vp, _vp, _i64, _i64, _i64,
                                           _i64, _vp]
_lib.sa_bwd_workspace_bytes.argtypes = [_MASKP, _ARGSP, ctypes.POINTER(_sz)]
_lib.sparse_attn_bwd.argtypes = [_MASKP, _vp, _sz, _ARGSP, ctypes.POINTER(sa_bwd_args_t), _vp, _sz, _vp]
_CFGP = ctypes.POINTER(sa_stream_cfg_t)
_lib.sa_stream_state_bytes.argtypes = [_CFGP, ctypes.POINTER(_sz)]
_lib.sa_decode_workspace_bytes.argtypes = [_CFGP, ctypes.POINTER(_sz)]
_lib.sa_stream_layout.argtypes = [_CFGP, ctypes.POINTER(_i64)]
_lib.sparse_attn_stream_reset.argtypes = [_CFGP, _vp, _sz, _vp]
_lib.sparse_attn_decode_step.argtypes = [_CFGP, _vp, _sz, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.sparse_attn_decode_step_static.argtypes = [_CFGP, _vp, _sz, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.sparse_attn_topk_middle.argtypes = [_MASKP, _ARGSP, _i32, _vp, _vp, _vp]
_lib.sparse_attn_topk_middle.restype = ctypes.c_int
for _name in ("sa_stream_state_bytes", "sa_decode_workspace_bytes", "sa_stream_layout",
              "sparse_attn_stream_reset", "sparse_attn_decode_step", "sparse_attn_decode_step_static"):
    getattr(_lib, _name).restype = ctypes.c_int
for _name in ("sa_plan_layout", "sa_plan_bytes", "sparse_attn_plan", "sa_plan_status", "sa_fwd_workspace_bytes",
              "sa_fwd_workspace_layout",
              "sparse_attn_fwd", "sparse_attn_rope", "sparse_attn_attend", "sa_topk_workspace_bytes",
              "topk_retrieve", "sparse_attn_segment_carry", "sa_bwd_workspace_bytes",
              "sparse_attn_bwd"):
    getattr(_lib, _name).restype = ctypes.c_int


class SparseAttnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


def _check(code: int) -> None:
    if code != SA_OK:
        raise SparseAttnError(code, sa_last_error())


def sa_last_error() -> str:
    return _lib.sa_last_error().decode()


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def mask(kind: int, n_q: int, n_k: int, *, a: int = 0, w: int = 1, sep=None, n_starting: int = 0,
         L_pretrain: int = 0, prefix_len: int = 0, sep_max: int = 0) -> sa_mask_t:
    """Build an sa_mask_t; `sep` is a device uint8 tensor [n_k] (kept alive by the caller);
    `sep_max` > 0 bounds the separators the plan lists (0 = no bound)."""
    return sa_mask_t(kind, n_q, n_k, a, w, _ptr(sep), n_starting, L_pretrain, prefix_len, sep_max)


def sa_plan_layout(m: sa_mask_t) -> sa_plan_header_t:
    out = sa_plan_header_t()
    _check(_lib.sa_plan_layout(ctypes.byref(m), ctypes.byref(out)))
    return out


def sa_plan_bytes(m: sa_mask_t) -> int:
    out = _sz()
    _check(_lib.sa_plan_bytes(ctypes.byref(m), ctypes.byref(out)))
    return out.value


def sparse_attn_plan(m: sa_mask_t, plan, stream=None) -> None:
    """Enqueue the plan kernels for mask m into the uint8 device tensor `plan`."""
    _check(_lib.sparse_attn_plan(ctypes.byref(m), _ptr(plan), _nbytes(plan), _stream(stream)))


def sa_plan_status(plan, stream=None) -> sa_plan_header_t:
    """Wait for the plan's stream and return its header; raises SparseAttnError (SA_ENOSPACE)
    when the mask held more separators than the plan's sep_max bound lets it list."""
    out = sa_plan_header_t()
    _check(_lib.sa_plan_status(_ptr(plan), _nbytes(plan), _stream(stream), ctypes.byref(out)))
    return out


def _check_4d(name, t, shape, dtype, device):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name}: device {t.device}, expected {device}")
    if t.stride(-1) != 1:
        raise ValueError(f"{name}: last dimension must be contiguous")


def _check_lse(lse, shape, device):
    import torch
    if lse is None:
        return
    if tuple(lse.shape) != tuple(shape) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError(f"lse: must be a contiguous float32 tensor of shape {tuple(shape)} "
                         f"(got {tuple(lse.shape)}, {lse.dtype})")
    if lse.device != device:
        raise ValueError(f"lse: device {lse.device}, expected {device}")


def fwd_args(q, k, v, o, *, lse=None, rope_base: Optional[float] = None,
             scale: Optional[float] = None, alibi_exp: Optional[float] = None,
             mask: Optional[sa_mask_t] = None) -> sa_fwd_args_t:
    """sa_fwd_args_t for [B,H,T,d] tensors (last dimension contiguous).

    ``alibi_exp`` = E selects SA_ALIBI (slopes 2^(-E (h+1) / h_q)) instead of RoPE.
    q and o must be [B, h_q, n_q, d], k and v [B, h_kv, n_k, d], all of one dtype and
    device, with n_q and n_k those of ``mask`` when it is given; lse (optional) a
    contiguous float32 [B, h_q, n_q].  The C ABI sees only pointers and strides, so
    these are checked here (ValueError).
    """
    import torch
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"q: dtype {q.dtype} is neither float32 nor bfloat16")
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v and o must be 4-d [B, H, T, d]")
    dtype = {torch.float32: SA_F32, torch.bfloat16: SA_BF16}[q.dtype]
    B, h_q, n_q, d = q.shape
    h_kv, n_k = k.shape[1], k.shape[2]
    if mask is not None and (n_q != mask.n_q or n_k != mask.n_k):
        raise ValueError(f"q / k token counts ({n_q}, {n_k}) differ from the mask's ({mask.n_q}, {mask.n_k})")
    _check_4d("q", q, (B, h_q, n_q, d), q.dtype, q.device)
    _check_4d("o", o, (B, h_q, n_q, d), q.dtype, q.device)
    _check_4d("k", k, (B, h_kv, n_k, d), q.dtype, q.device)
    _check_4d("v", v, (B, h_kv, n_k, d), q.dtype, q.device)
    _check_lse(lse, (B, h_q, n_q), q.device)
    a = sa_fwd_args_t()
    a.dtype, a.batch, a.h_q, a.h_kv, a.d = dtype, B, h_q, h_kv, d
    if alibi_exp is not None:
        if rope_base:
            raise ValueError("rope_base and alibi_exp are exclusive")
        a.rope, a.rope_base, a.alibi_exp = SA_ALIBI, 0.0, float(alibi_exp)
    else:
        a.rope = SA_ROPE_HALF if rope_base else SA_ROPE_NONE
        a.rope_base = float(rope_base or 0.0)
    a.scale = float(scale if scale is not None else d ** -0.5)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        setattr(a, name, t.data_ptr())
        getattr(a, name + "_stride")[:] = list(t.stride()[:3])
    a.lse = _ptr(lse)
    return a


def sa_fwd_workspace_bytes(m: sa_mask_t, args: sa_fwd_args_t) -> int:
    out = _sz()
    _check(_lib.sa_fwd_workspace_bytes(ctypes.byref(m), ctypes.byref(args), ctypes.byref(out)))
    return out.value


def sa_fwd_workspace_layout(m: sa_mask_t, args: sa_fwd_args_t) -> sa_fwd_ws_layout_t:
    out = sa_fwd_ws_layout_t()
    _check(_lib.sa_fwd_workspace_layout(ctypes.byref(m), ctypes.byref(args), ctypes.byref(out)))
    return out


def sparse_attn_fwd(m: sa_mask_t, plan, args: sa_fwd_args_t, ws, stream=None) -> None:
    """Enqueue the RoPE stage and the fused forward (see include/sparse_attn.h)."""
    _check(_lib.sparse_attn_fwd(ctypes.byref(m), _ptr(plan), _nbytes(plan), ctypes.byref(args),
                                _ptr(ws), _nbytes(ws),
                                _stream(stream)))


def sparse_attn_rope(m: sa_mask_t, plan, args: sa_fwd_args_t, ws, stream=None) -> None:
    """Enqueue only the RoPE stage of sparse_attn_fwd."""
    _check(_lib.sparse_attn_rope(ctypes.byref(m), _ptr(plan), _nbytes(plan), ctypes.byref(args),
                                 _ptr(ws), _nbytes(ws),
                                 _stream(stream)))


def sparse_attn_attend(m: sa_mask_t, plan, args: sa_fwd_args_t, ws, stream=None) -> None:
    """Enqueue only the fused forward of sparse_attn_fwd (after sparse_attn_rope)."""
    _check(_lib.sparse_attn_attend(ctypes.byref(m), _ptr(plan), _nbytes(plan), ctypes.byref(args),
                                   _ptr(ws), _nbytes(ws),
                                   _stream(stream)))


def sa_topk_workspace_bytes(n_heads: int, pool_len: int) -> int:
    out = _sz()
    _check(_lib.sa_topk_workspace_bytes(n_heads, pool_len, ctypes.byref(out)))
    return out.value


def topk_retrieve(q_score, pool_k, k: int, idx, ws, *, score=None, pool_v=None, pref_k=None,
                  pref_v=None, stream=None) -> None:
    """Top-k pool rows per head (see include/sparse_attn.h).

    q_score [n_heads, d] (row stride free, d contiguous); pool_k / pool_v
    [n_heads, pool_len, d] with equal strides; idx int32 [n_heads, k]; score
    float64 [n_heads, k] or None; pref_k / pref_v [n_heads, >=k, d] views with
    equal strides receiving the rows.  Shapes, dtypes, devices and those
    strides are checked here (ValueError); the C ABI checks the rest.
    """
    import torch
    if pool_k.dim() != 3 or pool_k.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("pool_k: must be a float32 or bfloat16 tensor [n_heads, pool_len, d]")
    dtype = {torch.float32: SA_F32, torch.bfloat16: SA_BF16}[pool_k.dtype]
    n_heads, pool_len, d = pool_k.shape
    dev = pool_k.device
    if pool_k.stride(-1) != 1:
        raise ValueError("pool_k: last dimension must be contiguous")
    if q_score.dim() != 2 or tuple(q_score.shape) != (n_heads, d) or q_score.dtype != pool_k.dtype \
            or q_score.stride(-1) != 1:
        raise ValueError(f"q_score: must be a {pool_k.dtype} tensor [{n_heads}, {d}] with contiguous rows")
    outs = [("idx", idx, torch.int32)] + ([("score", score, torch.float64)] if score is not None else [])
    for name, t, dt in outs:
        if tuple(t.shape) != (n_heads, k) or t.dtype != dt or not t.is_contiguous():
            raise ValueError(f"{name}: must be a contiguous {dt} tensor of shape {(n_heads, k)}")
    if pool_v is not None:
        if tuple(pool_v.shape) != tuple(pool_k.shape) or pool_v.dtype != pool_k.dtype \
                or pool_v.stride() != pool_k.stride():
            raise ValueError("pool_v: must match pool_k in shape, dtype and strides")
        if pref_k is None or pref_v is None:
            raise ValueError("pref_k and pref_v are required with pool_v")
        for name, t in (("pref_k", pref_k), ("pref_v", pref_v)):
            if t.dim() != 3 or t.shape[0] != n_heads or t.shape[1] < k or t.shape[2] != d \
                    or t.dtype != pool_k.dtype or t.stride(-1) != 1:
                raise ValueError(f"{name}: must be a {pool_k.dtype} tensor [{n_heads}, >= {k}, {d}] "
                                 "with contiguous rows")
        if pref_v.stride() != pref_k.stride():
            raise ValueError("pref_v: must have pref_k's strides")
    for name, t in (("q_score", q_score), ("idx", idx), ("score", score), ("pool_v", pool_v),
                    ("pref_k", pref_k), ("pref_v", pref_v), ("ws", ws)):
        if t is not None and t.device != dev:
            raise ValueError(f"{name}: device {t.device}, expected {dev}")
    prs = pref_k.stride() if pref_k is not None else (0, 0, 1)
    _check(_lib.topk_retrieve(dtype, n_heads, pool_len, d, k, _ptr(q_score), q_score.stride(0),
                              _ptr(pool_k), _ptr(pool_v), pool_k.stride(0), pool_k.stride(1),
                              _ptr(idx), _ptr(score), _ptr(pref_k), _ptr(pref_v), prs[0], prs[1],
                              _ptr(ws), _nbytes(ws), _stream(stream)))


def plan_to_host(m: sa_mask_t, plan) -> dict:
    """Copy a plan to the host and split it into its sections (numpy arrays)."""
    import numpy as np
    lay = sa_plan_layout(m)
    raw = plan.cpu().numpy().view(np.uint8)
    hdr = sa_plan_header_t.from_buffer_copy(raw[:ctypes.sizeof(sa_plan_header_t)].tobytes())

    def sec(off, n, dt):
        return raw[off:off + n * np.dtype(dt).itemsize].view(dt).copy()

    return {
        "header": hdr,
        "n_tiles": lay.n_tiles, "n_blocks": lay.n_blocks,
        "tile_ptr": sec(lay.off_tile_ptr, lay.n_tiles + 1, np.int32),
        "items": sec(lay.off_items, hdr.n_items, np.int32),
        "sep_count": sec(lay.off_sep_count, lay.n_tiles, np.int32),
        "sep_idx": sec(lay.off_sep_idx, min(hdr.n_sep, lay.cap_sep), np.int32),
        "sep_bits": sec(lay.off_sep_bits, lay.n_blocks, np.uint64),
        "blk_sep": sec(lay.off_blk_sep, lay.n_blocks + 1, np.int32),
    }


def sparse_attn_segment_carry(k, v, n_local: int, prefix_len: int, seg_len: int, tail_len: int,
                              tail_k, tail_v, pool_k, pool_v, pool_len: int, stream=None) -> None:
    """Tail and pool update after a segment (see include/sparse_attn.h).

    k, v [n_heads, prefix_len + seg_len, d]; tail_k / tail_v [n_local, >=keep, d] or None;
    pool_k / pool_v [n_heads - n_local, pool_cap, d] or None (d contiguous everywhere).
    """
    import torch
    if k.dim() != 3 or k.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("k: must be a float32 or bfloat16 tensor [n_heads, prefix_len + seg_len, d]")
    dtype = {torch.float32: SA_F32, torch.bfloat16: SA_BF16}[k.dtype]
    n_heads, rows, d = k.shape
    if rows < prefix_len + seg_len:
        raise ValueError(f"k, v: {rows} rows per head, the segment needs {prefix_len + seg_len}")
    keep = min(tail_len, prefix_len + seg_len)
    n_long = n_heads - n_local
    for name, t, h, r in (("v", v, n_heads, rows), ("tail_k", tail_k, n_local, keep),
                          ("tail_v", tail_v, n_local, keep), ("pool_k", pool_k, n_long, None),
                          ("pool_v", pool_v, n_long, None)):
        if t is None:
            continue
        if t.dim() != 3 or t.shape[0] != h or t.shape[2] != d or (r is not None and t.shape[1] < r) \
                or t.dtype != k.dtype or t.device != k.device:
            raise ValueError(f"{name}: must be a {k.dtype} tensor [{h}, >= {r or 1}, {d}] on {k.device} "
                             f"(got {tuple(t.shape)}, {t.dtype}, {t.device})")
    for a, b in ((k, v), (tail_k, tail_v), (pool_k, pool_v)):
        if a is not None and (b is None or a.stride() != b.stride() or a.stride(-1) != 1):
            raise ValueError("k/v, tail_k/tail_v and pool_k/pool_v pairs need equal strides, "
                             "d contiguous")
    ts = tail_k.stride()[:2] if tail_k is not None else (0, 0)
    ps = pool_k.stride()[:2] if pool_k is not None else (0, 0)
    cap = pool_k.shape[1] if pool_k is not None else 0
    _check(_lib.sparse_attn_segment_carry(dtype, n_heads, n_local, d, prefix_len, seg_len, tail_len,
                                          _ptr(k), _ptr(v), k.stride(0), k.stride(1), _ptr(tail_k),
                                          _ptr(tail_v), ts[0], ts[1], _ptr(pool_k), _ptr(pool_v),
                                          ps[0], ps[1], pool_len, cap, _stream(stream)))


def bwd_args(dout, dq, dk, dv, *, q=None, k=None) -> sa_bwd_args_t:
    """sa_bwd_args_t for [B,H,T,d] tensors (last dimension contiguous).

    With the forward's q and k given, dout and dq must match q (shape, dtype, device)
    and dk, dv must match k (ValueError otherwise)."""
    if q is not None:
        for name, t in (("dout", dout), ("dq", dq)):
            _check_4d(name, t, tuple(q.shape), q.dtype, q.device)
    if k is not None:
        for name, t in (("dk", dk), ("dv", dv)):
            _check_4d(name, t, tuple(k.shape), k.dtype, k.device)
    g = sa_bwd_args_t()
    for name, t in (("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        if t.stride(-1) != 1:
            raise ValueError(f"{name}: last dimension must be contiguous")
        setattr(g, name, t.data_ptr())
        getattr(g, name + "_stride")[:] = list(t.stride()[:3])
    return g


def sa_bwd_workspace_bytes(m: sa_mask_t, args: sa_fwd_args_t) -> int:
    out = _sz()
    _check(_lib.sa_bwd_workspace_bytes(ctypes.byref(m), ctypes.byref(args), ctypes.byref(out)))
    return out.value


def sparse_attn_bwd(m: sa_mask_t, plan, args: sa_fwd_args_t, grads: sa_bwd_args_t, ws,
                    stream=None) -> None:
    """Enqueue the backward (see include/sparse_attn.h)."""
    _check(_lib.sparse_attn_bwd(ctypes.byref(m), _ptr(plan), _nbytes(plan), ctypes.byref(args),
                                ctypes.byref(grads), _ptr(ws),
                                _nbytes(ws),
                                _stream(stream)))


def stream_cfg(batch: int, h_q: int, h_kv: int, d: int, a: int, s: int, w: int, c: int, *,
               rope_base: Optional[float] = None, scale: Optional[float] = None,
               kind: int = SA_MASK_SEPLLM, L_pretrain: int = 0) -> sa_stream_cfg_t:
    """SEPLLM: the four-part cache (a, s, w, c).  LAMBDA: a = n_starting and L_pretrain
    (s, w, c unused)."""
    return sa_stream_cfg_t(batch, h_q, h_kv, d, a, s, w, c, SA_ROPE_HALF if rope_base else SA_ROPE_NONE,
                           float(rope_base or 0.0), float(scale if scale is not None else d ** -0.5),
                           kind, L_pretrain)


def sa_stream_state_bytes(cfg: sa_stream_cfg_t) -> int:
    out = _sz()
    _check(_lib.sa_stream_state_bytes(ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def sa_decode_workspace_bytes(cfg: sa_stream_cfg_t) -> int:
    out = _sz()
    _check(_lib.sa_decode_workspace_bytes(ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def sa_stream_layout(cfg: sa_stream_cfg_t):
    out = (_i64 * 5)()
    _check(_lib.sa_stream_layout(ctypes.byref(cfg), out))
    return list(out)


def sparse_attn_stream_reset(cfg: sa_stream_cfg_t, state, stream=None) -> None:
    _check(_lib.sparse_attn_stream_reset(ctypes.byref(cfg), _ptr(state), _nbytes(state), _stream(stream)))


def _check_decode(cfg: sa_stream_cfg_t, state, q, k, v, is_sep, o, lse, ws=None) -> None:
    """The decode step's tensors against its configuration: q, o bf16 [B, h_q, d];
    k, v bf16 [B, h_kv, d]; is_sep uint8 [B] (None allowed for the LM-Infinite
    cache; the C ABI requires it for SepLLM); lse fp32 [B, h_q] or None; all
    contiguous and on the state's device (ValueError otherwise)."""
    import torch
    B, hq, hkv, d = cfg.batch, cfg.h_q, cfg.h_kv, cfg.d
    want = [("q", q, (B, hq, d), torch.bfloat16), ("k", k, (B, hkv, d), torch.bfloat16),
            ("v", v, (B, hkv, d), torch.bfloat16), ("o", o, (B, hq, d), torch.bfloat16)]
    if is_sep is not None:
        want.append(("is_sep", is_sep, (B,), torch.uint8))
    if lse is not None:
        want.append(("lse", lse, (B, hq), torch.float32))
    for name, t, shape, dt in want:
        if tuple(t.shape) != shape or t.dtype != dt or not t.is_contiguous():
            raise ValueError(f"{name}: must be a contiguous {dt} tensor of shape {shape} "
                             f"(got {tuple(t.shape)}, {t.dtype})")
    for name, t in [(w[0], w[1]) for w in want] + [("ws", ws)]:
        if t is not None and t.device != state.device:
            raise ValueError(f"{name}: device {t.device}, expected {state.device}")


def sparse_attn_decode_step(cfg: sa_stream_cfg_t, state, q, k, v, is_sep, o, ws, lse=None,
                            stream=None) -> None:
    """One decode step (see include/sparse_attn.h): q [B,h_q,d], k, v [B,h_kv,d], is_sep uint8 [B]."""
    _check_decode(cfg, state, q, k, v, is_sep, o, lse, ws)
    _check(_lib.sparse_attn_decode_step(ctypes.byref(cfg), _ptr(state), _nbytes(state),
                                        _ptr(q), _ptr(k), _ptr(v), _ptr(is_sep), _ptr(o), _ptr(lse),
                                        _ptr(ws), _nbytes(ws), _stream(stream)))


def sparse_attn_decode_step_static(cfg: sa_stream_cfg_t, state, q, k, v, is_sep, o, lse=None,
                                   stream=None) -> None:
    """The decode step with the library's static scratch instead of a workspace (see
    include/sparse_attn.h): it allocates nothing."""
    _check_decode(cfg, state, q, k, v, is_sep, o, lse)
    _check(_lib.sparse_attn_decode_step_static(ctypes.byref(cfg), _ptr(state),
                                               _nbytes(state), _ptr(q), _ptr(k),
                                               _ptr(v), _ptr(is_sep), _ptr(o), _ptr(lse), _stream(stream)))


def sparse_attn_topk_middle(m: sa_mask_t, args: sa_fwd_args_t, k_mid: int, sel, score, stream=None) -> None:
    """LM-Infinite top-k middle tokens on a forward's o and lse (see include/sparse_attn.h).

    sel (int32) and score (float32) must be contiguous [batch, h_q, n_q, k_mid]."""
    import torch
    shape = (args.batch, args.h_q, m.n_q, k_mid)
    for name, t, dt in (("sel", sel, torch.int32), ("score", score, torch.float32)):
        if tuple(t.shape) != shape or t.dtype != dt or not t.is_contiguous():
            raise ValueError(f"{name}: must be a contiguous {dt} tensor of shape {shape}")
    _check(_lib.sparse_attn_topk_middle(ctypes.byref(m), ctypes.byref(args), k_mid, _ptr(sel), _ptr(score),
                                        _stream(stream)))

