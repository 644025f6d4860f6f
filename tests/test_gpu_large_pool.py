"""Pools past 4 GiB: every kernel's byte offsets into the pool are 64-bit.  A small
batch is built on a compact host pool, then its blocks are placed at ids spread over
a 5.4 GB device pool (most of them past 4 GiB); the results must equal the oracle
on the compact pool (same contents, relabelled ids) -- decode (balanced and
partitioned), shared-prefix decode, multi-query decode, chunked prefill, the cache
write and block copy."""
import numpy as np
import pytest
import torch

import paged_kv_cache_79_amd as pkv
import workloads as W
from oracle import paged as O
from tests.gpu_helpers import TOL, dev, host, rownorm_err

pytestmark = pytest.mark.gpu

NB_BIG = 163840          # 32 KiB blocks (8 kv heads x 16 slots x 128 x bf16): 5.37 GB per pool


def big_ids(rng, n):
    """Distinct ids for n compact blocks: three quarters past 4 GiB, the rest below."""
    hi = rng.choice(np.arange(140000, NB_BIG), size=n - n // 4, replace=False)
    lo = rng.choice(np.arange(0, 100000), size=n // 4, replace=False)
    ids = np.concatenate([hi, lo])
    rng.shuffle(ids)
    return ids.astype(np.int64)


def place(pool_host, ids):
    """A big device pool holding pool_host's blocks at ids (other blocks uninitialised)."""
    nb, hkv, bs, d = pool_host.shape
    big = torch.empty((NB_BIG, hkv, bs, d), dtype=torch.bfloat16, device="cuda")
    big.index_copy_(0, torch.from_numpy(ids).cuda(), dev(pool_host))
    return big


def relabel_tables(tables, ids):
    t = tables.astype(np.int64)
    return np.where(t >= 0, ids[np.maximum(t, 0)], -1).astype(np.int32)


def relabel_slots(slots, ids, bs):
    s = slots.astype(np.int64)
    return np.where(s >= 0, ids[np.maximum(s, 0) // bs] * bs + s % bs, -1).astype(np.int64)


@pytest.fixture(scope="module", autouse=True)
def free_after():
    yield
    torch.cuda.empty_cache()


@pytest.mark.parametrize("partition_tokens", [0, 256])
def test_decode_and_write(partition_tokens):
    rng = np.random.Generator(np.random.PCG64(1201))
    ctx = rng.integers(1, 700, size=6, endpoint=True)
    b = W.build_decode_batch(name="large_pool", dtype="bf16", context_lens=ctx, num_q_heads=32,
                             num_kv_heads=8, head_dim=128, block_size=16, seed=1201)
    ids = big_ids(rng, b.k_pool.shape[0])
    print(f"large pool decode: {NB_BIG} blocks, max id {ids.max()}, part={partition_tokens}",
          flush=True)
    k, v = place(b.k_pool, ids), place(b.v_pool, ids)
    tables = dev(relabel_tables(b.block_tables, ids))
    pkv.paged_kv_write(k, v, dev(b.k_new), dev(b.v_new),
                       dev(relabel_slots(b.slot_mapping, ids, b.block_size)))
    q = dev(b.q)
    out = torch.empty_like(q)
    pkv.paged_attention_decode(out, q, k, v, tables, dev(b.context_lens), b.max_context_len,
                               b.scale, partition_tokens=partition_tokens)
    torch.cuda.synchronize()
    kw = O.kv_write(b.k_pool, b.k_new, b.slot_mapping)
    vw = O.kv_write(b.v_pool, b.v_new, b.slot_mapping)
    # the write landed bit for bit in the relabelled blocks
    idx = torch.from_numpy(ids).cuda()
    assert np.array_equal(host(k.index_select(0, idx)), kw)
    assert np.array_equal(host(v.index_select(0, idx)), vw)
    want = O.decode(b.q, kw, vw, b.block_tables, b.context_lens, b.scale, "bf16", b.num_kv_heads)
    err = rownorm_err(O.widen(host(out), "bf16"), want)
    assert err <= TOL["bf16"], f"row-normalised error {err:.3e}"
    # block copy between two blocks past 4 GiB
    src, dst = int(ids[0]), int(NB_BIG - 1) if int(ids[0]) != NB_BIG - 1 else int(NB_BIG - 2)
    pkv.copy_blocks(k, v, dev(np.array([[src, dst]], dtype=np.int64)))
    torch.cuda.synchronize()
    assert torch.equal(k[dst].view(torch.int16), k[src].view(torch.int16))
    assert torch.equal(v[dst].view(torch.int16), v[src].view(torch.int16))


def test_multi_query_and_prefill():
    rng = np.random.Generator(np.random.PCG64(1202))
    sb = W.spec_decode(seed=1202, num_seqs=5, draft=3, ctx_range=(4, 700), num_q_heads=32,
                       num_kv_heads=8)
    pre = sb.prefill
    nq = sb.draft + 1
    ids = big_ids(rng, sb.k_pool.shape[0])
    print(f"large pool multi-query: max id {ids.max()}", flush=True)
    k, v = place(sb.k_pool, ids), place(sb.v_pool, ids)
    tables = dev(relabel_tables(pre.block_tables, ids))
    pkv.paged_kv_write(k, v, dev(sb.k_new), dev(sb.v_new),
                       dev(relabel_slots(sb.slot_mapping, ids, pre.block_size)))
    kw = O.kv_write(sb.k_pool, sb.k_new, sb.slot_mapping)
    vw = O.kv_write(sb.v_pool, sb.v_new, sb.slot_mapping)
    want = O.prefill_chunk(pre.q, pre.cu_q_lens, kw, vw, pre.block_tables, pre.context_lens,
                           pre.scale, "bf16", pre.num_kv_heads)
    for path in ("multi_query", "prefill"):
        out = torch.empty(pre.q.shape, dtype=torch.bfloat16, device="cuda")
        if path == "multi_query":
            pkv.paged_attention_decode_multi_query(out, dev(pre.q), k, v, tables,
                                                   dev(pre.context_lens), nq, pre.max_context_len,
                                                   pre.scale)
        else:
            pkv.paged_attention_prefill_chunk(out, dev(pre.q), dev(pre.cu_q_lens), k, v, tables,
                                              dev(pre.context_lens), nq, pre.max_context_len,
                                              pre.scale)
        torch.cuda.synchronize()
        err = rownorm_err(O.widen(host(out), "bf16"), want)
        assert err <= TOL["bf16"], f"{path}: row-normalised error {err:.3e}"


def test_shared_prefix():
    rng = np.random.Generator(np.random.PCG64(1203))
    pg = W.prefix_groups(1203, [(5, 9), (2, 0), (4, 3)], num_q_heads=32, num_kv_heads=8)
    b = pg.batch
    ids = big_ids(rng, b.k_pool.shape[0])
    print(f"large pool shared prefix: max id {ids.max()}", flush=True)
    k, v = place(b.k_pool, ids), place(b.v_pool, ids)
    tables = dev(relabel_tables(b.block_tables, ids))
    pkv.paged_kv_write(k, v, dev(b.k_new), dev(b.v_new),
                       dev(relabel_slots(b.slot_mapping, ids, b.block_size)))
    q = dev(b.q)
    out = torch.empty_like(q)
    gnum, gpre = pg.group_num_seqs, pg.group_prefix_lens
    pkv.paged_attention_decode_shared_prefix(
        out, q, k, v, tables, dev(b.context_lens), b.max_context_len, b.scale,
        dev(pg.seq_prefix_lens), dev(pg.group_first_seq), dev(gnum), dev(gpre),
        int(gnum.max()), int(gpre.max()))
    torch.cuda.synchronize()
    kw = O.kv_write(b.k_pool, b.k_new, b.slot_mapping)
    vw = O.kv_write(b.v_pool, b.v_new, b.slot_mapping)
    want = O.decode(b.q, kw, vw, b.block_tables, b.context_lens, b.scale, "bf16", b.num_kv_heads)
    err = rownorm_err(O.widen(host(out), "bf16"), want)
    assert err <= TOL["bf16"], f"row-normalised error {err:.3e}"
