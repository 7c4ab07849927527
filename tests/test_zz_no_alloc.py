"""The no-allocation decode step (sparse_attn_decode_step_static) against the
decode step with a caller workspace (sparse_attn_decode_step), through the C ABI.

Both run the same kernels; the static variant keeps its per-step scratch in the
library's per-GPU array.  Two decode streams run one after the other, the second
smaller than the first (fewer sequences and heads, a smaller cache), so the
second reads the array after a larger call left other contents in it.  Every
step's output and LSE must equal the workspace variant's bit for bit (the same
arithmetic in the same order), and the held token sets must agree."""
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import structured_sparse_attention_attn_amd as m
    return m


CONFIGS = [
    # (batch, h_q, h_kv, a, s, w, c, steps, kind, L, rope)
    (8, 32, 8, 4, 64, 128, 324, 400, "sepllm", 0, 10000.0),
    (2, 8, 2, 2, 8, 16, 40, 120, "sepllm", 0, 500000.0),
    (3, 16, 4, 10, 1, 1, 0, 300, "lambda", 200, 10000.0),
    (1, 4, 1, 3, 1, 1, 0, 150, "lambda", 50, None),
]


def _run(sa, cfg_t, seed):
    from structured_sparse_attention_attn_amd.pipeline import StreamDecoder
    B, hq, hkv, a, s, w, c, n, kind, L, rope = cfg_t
    d = 128
    q, k, v, flags = W.make_decode_stream(B, hq, hkv, d, n, seed, 0.1)
    dec_ws = StreamDecoder(B, hq, hkv, d, a, s, w, c, rope_base=rope, kind=kind, L_pretrain=L)
    dec_st = StreamDecoder(B, hq, hkv, d, a, s, w, c, rope_base=rope, kind=kind, L_pretrain=L)
    print(f"no-alloc decode: B={B} h={hq}/{hkv} kind={kind} steps={n}", flush=True)
    for t in range(n):
        qt, kt, vt, ft = (x[t].cuda() for x in (q, k, v, flags))
        o1 = torch.empty_like(qt)
        o2 = torch.full_like(qt, 7.0)
        l1 = torch.empty((B, hq), dtype=torch.float32, device="cuda")
        l2 = torch.full((B, hq), 7.0, dtype=torch.float32, device="cuda")
        dec_ws.step(qt, kt, vt, ft, o=o1, lse=l1)
        sa.sparse_attn_decode_step_static(dec_st.cfg, dec_st.state, qt, kt, vt, ft, o2, lse=l2)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), (t, (o1.float() - o2.float()).abs().max().item())
        assert torch.equal(l1, l2), t
        if t % 50 == 0 or t == n - 1:
            for b in range(B):
                assert dec_ws.held(b) == dec_st.held(b)


def test_static_decode_matches_workspace_variant(sa):
    # larger first, then smaller: the second calls find the first calls' contents in the array
    _run(sa, CONFIGS[0], 71)
    _run(sa, CONFIGS[1], 72)


def test_static_decode_lambda_matches_workspace_variant(sa):
    _run(sa, CONFIGS[2], 73)
    _run(sa, CONFIGS[3], 74)


def test_static_decode_rejects_oversized_config(sa):
    # 64 sequences x 32 query heads x 4107 slots needs about 70 MB of scratch: refused, nothing launched
    cfg = sa.stream_cfg(64, 32, 8, 128, 10, 1, 1, 0, rope_base=10000.0, kind=sa.SA_MASK_LAMBDA,
                        L_pretrain=4096)
    assert sa.sa_decode_workspace_bytes(cfg) > sa.SA_DECODE_STATIC_SCRATCH_BYTES
    state = torch.empty(sa.sa_stream_state_bytes(cfg), dtype=torch.uint8, device="cuda")
    x = torch.zeros((64, 32, 128), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((64, 8, 128), dtype=torch.bfloat16, device="cuda")
    is_sep = torch.zeros(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(sa.SparseAttnError) as e:
        sa.sparse_attn_decode_step_static(cfg, state, x, kv, kv, is_sep, x)
    assert e.value.code == sa.SA_ENOSPACE
