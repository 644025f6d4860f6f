"""Entry points on pools the matrix-core kernels do not serve -- fp32, and bf16 with
head_dim 64 and block_size 4 (512-byte block runs) -- against the oracle: chunked
prefill and the multi-query decode go query by query on the vector units with the
decode's arithmetic, the shared-prefix decode is plain decode over the same tables, and
the contiguous baseline has its fp32 instantiation."""
import numpy as np
import pytest
import torch

import paged_kv_cache_79_amd as pkv
import workloads as W
from oracle import paged as O
from tests.gpu_helpers import TOL, DecodeRun, dev, host, rownorm_err

pytestmark = pytest.mark.gpu

TORCH = {"bf16": torch.bfloat16, "f32": torch.float32}


def prefill_case(dtype, chunk_lens, contexts, hq, hkv, d, bs, seed):
    print(f"vector-path prefill {dtype} chunks={list(chunk_lens)} ctx={list(contexts)} Hq={hq} "
          f"Hkv={hkv} D={d} bs={bs}", flush=True)
    pre, kp, vp, _ = W.prefill_only(seed=seed, dtype=dtype, chunk_lens=chunk_lens,
                                    contexts=contexts, num_q_heads=hq, num_kv_heads=hkv,
                                    head_dim=d, block_size=bs)
    want = O.prefill_chunk(pre.q, pre.cu_q_lens, kp, vp, pre.block_tables, pre.context_lens,
                           pre.scale, dtype, hkv)
    return pre, kp, vp, want


def run_prefill(pre, kp, vp, dtype):
    out = torch.full(pre.q.shape, float("nan"), dtype=TORCH[dtype], device="cuda")
    pkv.paged_attention_prefill_chunk(out, dev(pre.q), dev(pre.cu_q_lens), dev(kp), dev(vp),
                                      dev(pre.block_tables), dev(pre.context_lens), pre.max_q_len,
                                      pre.max_context_len, pre.scale)
    torch.cuda.synchronize()
    return O.widen(host(out), dtype)


@pytest.mark.parametrize("dtype,d,bs,hq,hkv", [("f32", 128, 16, 8, 2), ("f32", 64, 4, 4, 4),
                                               ("f32", 128, 32, 16, 2), ("f32", 64, 8, 7, 1),
                                               ("bf16", 64, 4, 8, 2), ("bf16", 64, 4, 4, 4)])
def test_prefill(dtype, d, bs, hq, hkv):
    # ragged chunks, a chunk that is its whole context, single queries, a long context
    pre, kp, vp, want = prefill_case(dtype, [37, 64, 1, 5], [100, 64, 1, 700], hq, hkv, d, bs,
                                     seed=d + bs + hq)
    got = run_prefill(pre, kp, vp, dtype)
    err = rownorm_err(got, want)
    assert err <= TOL[dtype], f"row-normalised error {err:.3e}"


def test_prefill_f32_last_row_is_decode():
    pre, kp, vp, want = prefill_case("f32", [48], [500], 8, 2, 128, 16, seed=6)
    got = run_prefill(pre, kp, vp, "f32")
    out = torch.empty((1, 8, 128), dtype=torch.float32, device="cuda")
    pkv.paged_attention_decode(out, dev(pre.q[-1:]), dev(kp), dev(vp), dev(pre.block_tables),
                               dev(pre.context_lens), 500, pre.scale)
    torch.cuda.synchronize()
    assert rownorm_err(got[-1:], O.widen(host(out), "f32")) <= TOL["f32"]
    assert rownorm_err(got, want) <= TOL["f32"]


@pytest.mark.parametrize("dtype,d,bs,n", [("f32", 128, 16, 4), ("f32", 64, 4, 3),
                                          ("bf16", 64, 4, 4)])
def test_multi_query(dtype, d, bs, n):
    """Equal chunks of n queries are the multi-query layout: query i of sequence s is row
    s * n + i and sits at position ctx_s - n + i."""
    S, hq, hkv = 5, 8, 2
    rng = np.random.Generator(np.random.PCG64(n + d))
    ctx = rng.integers(n, 400, size=S, endpoint=True).tolist()
    pre, kp, vp, want = prefill_case(dtype, [n] * S, ctx, hq, hkv, d, bs, seed=90 + n)
    out = torch.full(pre.q.shape, float("nan"), dtype=TORCH[dtype], device="cuda")
    pkv.paged_attention_decode_multi_query(out, dev(pre.q), dev(kp), dev(vp),
                                           dev(pre.block_tables), dev(pre.context_lens), n,
                                           pre.max_context_len, pre.scale)
    torch.cuda.synchronize()
    err = rownorm_err(O.widen(host(out), dtype), want)
    assert err <= TOL[dtype], f"row-normalised error {err:.3e}"


@pytest.mark.parametrize("dtype,d,bs", [("f32", 128, 16), ("bf16", 64, 4)])
def test_shared_prefix_is_plain_decode(dtype, d, bs):
    """One group sharing its first blocks: the call returns plain decode's bits."""
    S, hq, hkv, plen = 6, 8, 2, 8 * bs
    rng = np.random.Generator(np.random.PCG64(5))
    ctx = (plen + rng.integers(0, 100, size=S)).tolist()
    b = W.build_decode_batch(name=f"sp_{dtype}", dtype=dtype, context_lens=ctx, num_q_heads=hq,
                             num_kv_heads=hkv, head_dim=d, block_size=bs, seed=6)
    tables = b.block_tables.copy()
    tables[:, :plen // bs] = tables[0, :plen // bs]          # the prefix blocks of sequence 0
    r = DecodeRun(b, tables=tables)
    r.write()
    plain = r.decode(0)
    out = torch.empty_like(r.q)
    i32 = lambda x: dev(np.asarray(x, dtype=np.int32))
    pkv.paged_attention_decode_shared_prefix(out, r.q, r.k, r.v, r.tables, r.ctx, b.max_context_len,
                                             b.scale, i32([plen] * S), i32([0]), i32([S]),
                                             i32([plen]), S, plen)
    torch.cuda.synchronize()
    got = host(out)
    assert np.array_equal(got, plain)
    k, v = O.kv_write(b.k_pool, b.k_new, b.slot_mapping), O.kv_write(b.v_pool, b.v_new, b.slot_mapping)
    want = O.decode(b.q, k, v, tables, b.context_lens, b.scale, dtype, hkv)
    assert rownorm_err(O.widen(got, dtype), want) <= TOL[dtype]


@pytest.mark.parametrize("g,d", [(4, 128), (1, 64), (8, 128)])
def test_contiguous_f32(g, d):
    b = W.build_decode_batch(name=f"f32_contig_g{g}", dtype="f32",
                             context_lens=[1, 63, 64, 65, 200, 700, 0], num_q_heads=2 * g,
                             num_kv_heads=2, head_dim=d, block_size=16, seed=g, contiguous=True)
    print(f"contiguous f32 G={g} D={d}", flush=True)
    out = torch.empty(b.q.shape, dtype=torch.float32, device="cuda")
    pkv.contiguous_attention_decode(out, dev(b.q), dev(b.extra["k_cache"]), dev(b.extra["v_cache"]),
                                    dev(b.context_lens), b.max_context_len, b.scale)
    torch.cuda.synchronize()
    got = host(out)
    want = O.decode_contiguous(b.q, b.extra["k_cache"], b.extra["v_cache"], b.context_lens,
                               b.scale, "f32", b.num_kv_heads)
    assert rownorm_err(got.astype(np.float64), want) <= TOL["f32"]
    r = DecodeRun(b)
    r.write()
    assert np.array_equal(r.decode(0), got), "contiguous and paged fp32 decode differ"
