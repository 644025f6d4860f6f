"""Calls on a side stream: the binding allocates each call's workspace on the stream the
call runs on, so memory freed when the call returns cannot be handed to work on another
stream while the kernels still write their partial states there.  Each case holds the
side stream back with a short spin, enqueues the call behind it, then allocates and
fills buffers of the workspace's size on the current stream before the side stream
runs; the outputs must still match the oracle."""
import numpy as np
import pytest
import torch

import paged_kv_cache_79_amd as pkv
import workloads as W
from oracle import paged as O
from tests.gpu_helpers import TOL, dev, host, rownorm_err

pytestmark = pytest.mark.gpu

SPIN_CYCLES = 20_000_000          # a few milliseconds of one wave on the side stream


def churn(num_bytes):
    """Allocate and fill buffers of num_bytes on the current stream."""
    keep = []
    for _ in range(4):
        t = torch.empty(max(num_bytes, 1), dtype=torch.uint8, device="cuda")
        t.fill_(0xFF)
        keep.append(t)
    del keep


def on_side_stream(call, ws_bytes):
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        torch.cuda._sleep(SPIN_CYCLES)
    call(s)
    churn(ws_bytes)
    s.synchronize()
    torch.cuda.synchronize()


def test_decode_side_stream():
    b = W.gqa(num_seqs=12, seed=811)
    print(f"side-stream decode S={b.context_lens.shape[0]} max_ctx={b.max_context_len}", flush=True)
    k, v, q = dev(b.k_pool), dev(b.v_pool), dev(b.q)
    tab, ctx = dev(b.block_tables), dev(b.context_lens)
    pkv.paged_kv_write(k, v, dev(b.k_new), dev(b.v_new), dev(b.slot_mapping))
    out = torch.empty(q.shape, dtype=q.dtype, device="cuda")
    ws = pkv.paged_attention_decode_workspace_bytes(*q.shape[:2], b.num_kv_heads, b.head_dim,
                                                    b.max_context_len)
    assert ws > 0
    on_side_stream(lambda s: pkv.paged_attention_decode(out, q, k, v, tab, ctx, b.max_context_len,
                                                        b.scale, stream=s), ws)
    kw = O.kv_write(b.k_pool, b.k_new, b.slot_mapping)
    vw = O.kv_write(b.v_pool, b.v_new, b.slot_mapping)
    want = O.decode(b.q, kw, vw, b.block_tables, b.context_lens, b.scale, "bf16", b.num_kv_heads)
    err = rownorm_err(O.widen(host(out), "bf16"), want)
    assert err <= TOL["bf16"], f"row-normalised error {err:.3e}"


def test_split_prefill_side_stream():
    pre, kp, vp, _ = W.prefill_only(seed=812, chunk_lens=[300, 16, 5], contexts=[2000, 3000, 40],
                                    num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16)
    print("side-stream split prefill", flush=True)
    q, k, v = dev(pre.q), dev(kp), dev(vp)
    cu, tab, ctx = dev(pre.cu_q_lens), dev(pre.block_tables), dev(pre.context_lens)
    out = torch.empty(q.shape, dtype=q.dtype, device="cuda")
    ws = pkv.paged_attention_prefill_chunk_workspace_bytes(8, 2, 128)
    assert ws > 0
    on_side_stream(lambda s: pkv.paged_attention_prefill_chunk(
        out, q, cu, k, v, tab, ctx, pre.max_q_len, pre.max_context_len, pre.scale, split=True,
        stream=s), ws)
    want = O.prefill_chunk(pre.q, pre.cu_q_lens, kp, vp, pre.block_tables, pre.context_lens,
                           pre.scale, "bf16", 2)
    err = rownorm_err(O.widen(host(out), "bf16"), want)
    assert err <= TOL["bf16"], f"row-normalised error {err:.3e}"


def test_multi_query_side_stream():
    sb = W.spec_decode(num_seqs=8, draft=3, seed=813)
    pre = sb.prefill
    nq = sb.draft + 1
    print(f"side-stream multi-query S={pre.num_chunks} k+1={nq}", flush=True)
    k, v = dev(sb.k_pool), dev(sb.v_pool)
    pkv.paged_kv_write(k, v, dev(sb.k_new), dev(sb.v_new), dev(sb.slot_mapping))
    q, tab, ctx = dev(pre.q), dev(pre.block_tables), dev(pre.context_lens)
    out = torch.empty(q.shape, dtype=q.dtype, device="cuda")
    ws = pkv.paged_attention_decode_multi_query_workspace_bytes(pre.num_chunks, nq, pre.num_q_heads,
                                                                pre.num_kv_heads, pre.head_dim)
    on_side_stream(lambda s: pkv.paged_attention_decode_multi_query(
        out, q, k, v, tab, ctx, nq, pre.max_context_len, pre.scale, stream=s), ws)
    kw = O.kv_write(sb.k_pool, sb.k_new, sb.slot_mapping)
    vw = O.kv_write(sb.v_pool, sb.v_new, sb.slot_mapping)
    want = O.prefill_chunk(pre.q, pre.cu_q_lens, kw, vw, pre.block_tables, pre.context_lens,
                           pre.scale, "bf16", pre.num_kv_heads)
    err = rownorm_err(O.widen(host(out), "bf16"), want)
    assert err <= TOL["bf16"], f"row-normalised error {err:.3e}"
    assert np.isfinite(O.widen(host(out), "bf16")).all()
