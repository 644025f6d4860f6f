"""Chunked-prefill attention on the GPU (matrix-core path) against the oracle."""
import numpy as np
import pytest
import torch

import paged_kv_cache_79_amd as pkv
import workloads as W
from oracle import paged as O
from tests import prefill_plan as PP
from tests.gpu_helpers import TOL, DecodeRun, dev, host, rownorm_err

pytestmark = pytest.mark.gpu


def run_prefill(pre, k_pool, v_pool, split=True):
    out = torch.empty(pre.q.shape, dtype=torch.bfloat16, device="cuda")
    pkv.paged_attention_prefill_chunk(out, dev(pre.q), dev(pre.cu_q_lens), k_pool, v_pool,
                                      dev(pre.block_tables), dev(pre.context_lens), pre.max_q_len,
                                      pre.max_context_len, pre.scale, split=split)
    torch.cuda.synchronize()
    return O.widen(host(out), "bf16")


def split_wgs(hq, hkv, d):
    """Workgroups of the balanced key split, from the workspace size: per workgroup two
    partial slots of 128 rows, each row (max, sum) in fp32 and d bf16 outputs, and one
    item descriptor of two int32."""
    per_wg = 2 * 128 * (2 * 4 + 2 * d) + 2 * 4
    n = pkv.paged_attention_prefill_chunk_workspace_bytes(hq, hkv, d)
    assert n % per_wg == 0
    return n // per_wg


def expect_split(pre):
    W = split_wgs(pre.num_q_heads, pre.num_kv_heads, pre.head_dim)
    mb = pre.block_tables.shape[1] * pre.block_size
    return PP.plan(pre.cu_q_lens, pre.context_lens, pre.num_q_heads // pre.num_kv_heads,
                   pre.num_kv_heads, W, pre.max_q_len, min(pre.max_context_len, mb))[0]


def check_split(chunk_lens, contexts, hq, hkv, d=128, bs=16, seed=0, split=True):
    """The call with a workspace (key split when the plan asks for it) and without one,
    both against the oracle; the two agree bit for bit exactly when no split happens."""
    print(f"prefill split chunks={len(chunk_lens)} max_ctx={max(contexts)} Hq={hq} Hkv={hkv} "
          f"D={d} bs={bs} seed={seed}", flush=True)
    pre, kp, vp, nb = W.prefill_only(seed=seed, chunk_lens=chunk_lens, contexts=contexts,
                                     num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs)
    assert expect_split(pre) == split
    got = run_prefill(pre, dev(kp), dev(vp))
    plain = run_prefill(pre, dev(kp), dev(vp), split=False)
    want = O.prefill_chunk(pre.q, pre.cu_q_lens, kp, vp, pre.block_tables, pre.context_lens,
                           pre.scale, "bf16", hkv)
    assert rownorm_err(got, want) <= TOL["bf16"], "with workspace"
    assert rownorm_err(plain, want) <= TOL["bf16"], "without workspace"
    assert np.array_equal(got, plain) != split


def check_small(chunk_lens, contexts, hq, hkv, d=128, bs=16, seed=0, rows=None):
    print(f"prefill chunks={list(chunk_lens)} ctx={list(contexts)} Hq={hq} Hkv={hkv} D={d} bs={bs}",
          flush=True)
    pre, kp, vp, nb = W.prefill_only(seed=seed, chunk_lens=chunk_lens, contexts=contexts,
                                     num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs)
    got = run_prefill(pre, dev(kp), dev(vp))
    want = O.prefill_chunk(pre.q, pre.cu_q_lens, kp, vp, pre.block_tables, pre.context_lens,
                           pre.scale, "bf16", hkv, rows=rows)
    err = rownorm_err(got, want)
    assert err <= TOL["bf16"], f"row-normalised error {err:.3e}"


@pytest.mark.parametrize("g", [1, 2, 3, 4, 5, 6, 7, 8])
def test_groups(g):
    check_small([37, 64], [100, 64], 2 * g, 2, seed=g)


def test_empty_chunks_between_others():
    """Chunks with no queries (their contexts still in the table) between chunks with
    queries, through the call with a workspace (key split when the plan asks for it)
    and without one."""
    pre, kp, vp, nb = W.prefill_only(seed=31, chunk_lens=[37, 0, 200, 0, 5],
                                     contexts=[100, 50, 2600, 300, 900], num_q_heads=8,
                                     num_kv_heads=2, head_dim=128, block_size=16)
    print(f"prefill empty chunks, split planned: {expect_split(pre)}", flush=True)
    want = O.prefill_chunk(pre.q, pre.cu_q_lens, kp, vp, pre.block_tables, pre.context_lens,
                           pre.scale, "bf16", 2)
    for split in (True, False):
        got = run_prefill(pre, dev(kp), dev(vp), split=split)
        assert rownorm_err(got, want) <= TOL["bf16"], f"split={split}"


def test_whole_prompt_and_single_query():
    check_small([1, 130, 5], [1, 130, 300], 8, 2, seed=3)      # n_q == ctx and n_q == 1


@pytest.mark.parametrize("d,bs", [(128, 4), (128, 32), (64, 16), (64, 8)])
def test_shapes(d, bs):
    check_small([70, 33], [333, 33], 8, 2, d=d, bs=bs, seed=4)


def test_ragged_many_tiles():
    check_small([200, 129, 64], [1000, 700, 129], 32, 8, seed=5)


def test_last_row_equals_decode():
    """The last query of a chunk is a decode query over the whole context."""
    pre, kp, vp, nb = W.prefill_only(seed=6, chunk_lens=[48], contexts=[500], num_q_heads=8,
                                     num_kv_heads=2, head_dim=128, block_size=16)
    got = run_prefill(pre, dev(kp), dev(vp))
    out = torch.empty((1, 8, 128), dtype=torch.bfloat16, device="cuda")
    pkv.paged_attention_decode(out, dev(pre.q[-1:]), dev(kp), dev(vp), dev(pre.block_tables),
                               dev(pre.context_lens), 500, pre.scale, partition_tokens=0)
    torch.cuda.synchronize()
    dec = O.widen(host(out), "bf16")
    assert rownorm_err(got[-1:], dec) <= TOL["bf16"]


def test_full_mixed_prefill():
    """The mixed workload's 4 chunks of 512 queries, launched as the benchmark launches
    them (with the key-split workspace): every (query, head) row against the oracle."""
    from tests.oracle_pool import prefill_all
    m = W.mixed()
    b, pre = m.decode, m.prefill
    print("prefill mixed full", flush=True)
    r = DecodeRun(b)
    r.write()                                        # chunk K/V written first
    got = run_prefill(pre, r.k, r.v)
    k = O.kv_write(b.k_pool, b.k_new, b.slot_mapping)
    v = O.kv_write(b.v_pool, b.v_new, b.slot_mapping)
    want = prefill_all(pre.q, pre.cu_q_lens, k, v, pre.block_tables, pre.context_lens, pre.scale,
                       "bf16", pre.num_kv_heads)
    assert not np.isnan(want).any()
    assert rownorm_err(got, want) <= TOL["bf16"]


# ---- balanced key split ---------------------------------------------------------------

def test_split_uneven_chunks():
    """Three chunks of 64 queries over 3000, 300 and 600 keys: 12 items over the resident
    workgroups, so every item is cut into many pieces (merge batches of 16 and more)."""
    check_split([64, 64, 64], [3000, 300, 600], 8, 2, seed=11)


def test_split_one_long_chunk():
    """100 queries over 40000 keys: 8 items, each cut over ~64 workgroups."""
    check_split([100], [40000], 8, 2, seed=12)


@pytest.mark.parametrize("g,d,bs", [(1, 128, 16), (7, 128, 32), (4, 64, 8), (8, 64, 16)])
def test_split_groups_and_shapes(g, d, bs):
    check_split([33, 128, 5], [2500, 700, 9000], 2 * g, 2, d=d, bs=bs, seed=20 + g)


def test_split_many_chunks():
    """70 chunks (past the 64 of one scan pass of the plan) of 1..40 queries over
    40..3000 keys, one kv head."""
    rng = np.random.default_rng(13)
    nq = rng.integers(1, 41, 70)
    ctx = nq + rng.integers(0, 3000, 70)
    check_split(nq.tolist(), ctx.tolist(), 4, 1, seed=13)


def test_even_items_filling_one_round_do_not_split():
    """64 chunks of 16 queries over 300 keys, 64 q / 8 kv heads: 512 equal items of 5
    tiles, one per resident workgroup, so the split would gain nothing."""
    check_split([16] * 64, [300] * 64, 64, 8, seed=14, split=False)


def test_few_items_split_even_when_equal():
    """Two chunks of 128 queries over 2000 keys: 16 equal items would leave most
    workgroups idle, so the keys are split over all of them."""
    check_split([128, 128], [2000, 2000], 8, 2, seed=16)


def test_full_mixed_split_against_unsplit():
    """The mixed workload's prefill at full size splits; every row agrees with the
    unsplit call (the oracle checks sampled rows in test_full_mixed_prefill_sampled)."""
    m = W.mixed()
    b, pre = m.decode, m.prefill
    print("prefill mixed full: split against unsplit", flush=True)
    assert expect_split(pre)
    r = DecodeRun(b)
    r.write()
    got = run_prefill(pre, r.k, r.v)
    plain = run_prefill(pre, r.k, r.v, split=False)
    assert rownorm_err(got, plain) <= TOL["bf16"]
    assert not np.array_equal(got, plain)


def test_split_workspace_too_small():
    pre, kp, vp, nb = W.prefill_only(seed=15, chunk_lens=[16], contexts=[500], num_q_heads=8,
                                     num_kv_heads=2, head_dim=128, block_size=16)
    out = torch.empty(pre.q.shape, dtype=torch.bfloat16, device="cuda")
    need = pkv.paged_attention_prefill_chunk_workspace_bytes(8, 2, 128)
    assert need > 0
    ws = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(pkv.PagedKVError, match="WORKSPACE|workspace"):
        pkv.paged_attention_prefill_chunk(out, dev(pre.q), dev(pre.cu_q_lens), dev(kp), dev(vp),
                                          dev(pre.block_tables), dev(pre.context_lens),
                                          pre.max_q_len, pre.max_context_len, pre.scale,
                                          workspace=ws)


def test_split_at_one_round_of_items():
    """500 chunks of 1..16 queries over 16..600 keys, 4 q / 1 kv head: 500 items (one per
    chunk), just inside one round of 512 workgroups, so the plan scans 8 passes of 64
    chunks and every workgroup locates its range among them."""
    rng = np.random.default_rng(17)
    nq = rng.integers(1, 17, 500)
    ctx = nq + rng.integers(0, 585, 500)
    ctx[::97] = 600                                   # a few long ones make the split pay
    check_split(nq.tolist(), ctx.tolist(), 4, 1, seed=17)
