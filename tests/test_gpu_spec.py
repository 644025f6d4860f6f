"""Multi-token decode (speculative verification) on the GPU against the oracle: every
sequence writes its k + 1 newest tokens through slot_mapping, then attends with k + 1
causal queries at the last k + 1 positions of its context -- through the multi-query
decode (matrix cores, balanced split) and through chunked prefill."""
import numpy as np
import pytest
import torch

import paged_kv_cache_79_amd as pkv
import workloads as W
from oracle import paged as O
from tests.gpu_helpers import TOL, dev, host, rownorm_err

pytestmark = pytest.mark.gpu


def attend(path, pre, nq, k, v):
    out = torch.empty(pre.q.shape, dtype=torch.bfloat16, device="cuda")
    if path == "prefill":
        pkv.paged_attention_prefill_chunk(out, dev(pre.q), dev(pre.cu_q_lens), k, v,
                                          dev(pre.block_tables), dev(pre.context_lens), nq,
                                          pre.max_context_len, pre.scale)
    else:
        pkv.paged_attention_decode_multi_query(out, dev(pre.q), k, v, dev(pre.block_tables),
                                               dev(pre.context_lens), nq, pre.max_context_len,
                                               pre.scale)
    torch.cuda.synchronize()
    return host(out)


def run(sb, seqs, path="multi_query"):
    pre = sb.prefill
    nq = sb.draft + 1
    print(f"spec {path} S={pre.num_chunks} k+1={nq} Hq={pre.num_q_heads} "
          f"Hkv={pre.num_kv_heads} D={pre.head_dim} bs={pre.block_size} "
          f"max_ctx={pre.max_context_len}", flush=True)
    k, v = dev(sb.k_pool), dev(sb.v_pool)
    pkv.paged_kv_write(k, v, dev(sb.k_new), dev(sb.v_new), dev(sb.slot_mapping))
    raw = attend(path, pre, nq, k, v)
    got = O.widen(raw, "bf16")
    kw = O.kv_write(sb.k_pool, sb.k_new, sb.slot_mapping)
    vw = O.kv_write(sb.v_pool, sb.v_new, sb.slot_mapping)
    rows = [(s * nq + i, hq) for s in seqs for i in range(nq) for hq in range(pre.num_q_heads)]
    want = O.prefill_chunk(pre.q, pre.cu_q_lens, kw, vw, pre.block_tables, pre.context_lens,
                           pre.scale, "bf16", pre.num_kv_heads, rows=rows)
    err = rownorm_err(got, want)
    assert err <= TOL["bf16"], f"row-normalised error {err:.3e}"
    # the last query of every sequence is a plain decode over the whole context
    last = np.stack([got[s * nq + nq - 1] for s in seqs])
    want_last = O.decode(pre.q[[s * nq + nq - 1 for s in seqs]], kw, vw, pre.block_tables[seqs],
                         pre.context_lens[seqs], pre.scale, "bf16", pre.num_kv_heads)
    assert rownorm_err(last, want_last) <= TOL["bf16"]
    return raw, k, v


@pytest.mark.parametrize("path", ["multi_query", "prefill"])
@pytest.mark.parametrize("draft", [1, 3])
def test_small(draft, path):
    run(W.spec_decode(seed=draft, num_seqs=6, draft=draft, ctx_range=(1, 700)), list(range(6)),
        path)


@pytest.mark.parametrize("draft", [4, 5, 6, 7])
def test_drafts_past_one_matrix_tile(draft):
    """(k + 1) x 4 heads = 20..32 rows: more than the 16 columns of the multi-query
    kernel's matrix tile; the entry point serves them query by query on the vector
    units, and the prefill path serves them on the matrix cores."""
    sb = W.spec_decode(seed=70 + draft, num_seqs=6, draft=draft, ctx_range=(1, 700))
    mq, _, _ = run(sb, list(range(6)), "multi_query")
    pf, _, _ = run(sb, list(range(6)), "prefill")
    assert rownorm_err(O.widen(mq, "bf16"), O.widen(pf, "bf16")) <= TOL["bf16"]


@pytest.mark.parametrize("path", ["multi_query", "prefill"])
def test_group_one_and_block_32(path):
    run(W.spec_decode(seed=9, num_seqs=4, draft=4, ctx_range=(60, 300), num_q_heads=4,
                      num_kv_heads=4, block_size=32), list(range(4)), path)


@pytest.mark.parametrize("hq,hkv,draft,d,bs", [(8, 1, 1, 128, 16), (16, 2, 0, 64, 8),
                                               (6, 2, 4, 128, 16), (14, 2, 1, 64, 32),
                                               (2, 2, 15, 128, 8)])
def test_multi_query_shapes(hq, hkv, draft, d, bs):
    """Row packings of one tile: G = 8 x 2 queries, a single query (plain decode),
    G = 3 x 5, G = 7 x 2, G = 1 x 16; head dims 64/128, block sizes 8/16/32; contexts
    from a single tile to many, with every tail length."""
    sb = W.spec_decode(seed=100 + hq + draft, num_seqs=9, draft=draft, ctx_range=(1, 1300),
                       num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs)
    run(sb, list(range(9)))


def test_multi_query_matches_prefill_path():
    """Both paths on the same inputs agree to the attention tolerance row by row."""
    sb = W.spec_decode(seed=31, num_seqs=16, draft=3, ctx_range=(1, 3000))
    pre = sb.prefill
    raw, k, v = run(sb, list(range(16)))
    other = attend("prefill", pre, 4, k, v)
    assert rownorm_err(O.widen(raw, "bf16"), O.widen(other, "bf16")) <= TOL["bf16"]


@pytest.mark.parametrize("path", ["multi_query", "prefill"])
def test_full_sampled(path):
    sb = W.spec_decode()
    rng = np.random.Generator(np.random.PCG64(4))
    run(sb, sorted(rng.choice(sb.prefill.num_chunks, 10, replace=False).tolist()), path)


def test_many_sequences():
    """700 sequences of up to 300 tokens: the balanced split counts and locates past the
    first 256 sequences. Sampled rows against the oracle; every row against the prefill
    path."""
    sb = W.spec_decode(seed=33, num_seqs=700, draft=3, ctx_range=(4, 300), num_q_heads=8,
                       num_kv_heads=2)
    seqs = [0, 1, 255, 256, 257, 511, 512, 699]
    rng = np.random.Generator(np.random.PCG64(34))
    seqs = sorted(set(seqs) | set(rng.choice(700, 12, replace=False).tolist()))
    raw, k, v = run(sb, seqs)
    other = attend("prefill", sb.prefill, 4, k, v)
    assert rownorm_err(O.widen(raw, "bf16"), O.widen(other, "bf16")) <= TOL["bf16"]
