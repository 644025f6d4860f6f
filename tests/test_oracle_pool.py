"""The process-pool fan-out used by the full-size GPU parity tests returns exactly what
the oracle returns when called directly (same functions, same inputs, split into tasks)."""
import numpy as np

import workloads as W
from oracle import paged as O
from tests.oracle_pool import decode_all, prefill_all


def test_decode_fan_out_equals_direct_call():
    b = W.gqa(num_seqs=9, seed=5)
    k = O.kv_write(b.k_pool, b.k_new, b.slot_mapping)
    v = O.kv_write(b.v_pool, b.v_new, b.slot_mapping)
    want = O.decode(b.q, k, v, b.block_tables, b.context_lens, b.scale, "bf16", b.num_kv_heads)
    got = decode_all(b.q, k, v, b.block_tables, b.context_lens, b.scale, "bf16", b.num_kv_heads,
                     seqs_per_task=2)
    assert np.array_equal(got, want)


def test_prefill_fan_out_equals_direct_call():
    pre, kp, vp, _ = W.prefill_only(seed=3, chunk_lens=[40, 17, 5], contexts=[90, 17, 300],
                                    num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16)
    want = O.prefill_chunk(pre.q, pre.cu_q_lens, kp, vp, pre.block_tables, pre.context_lens,
                           pre.scale, "bf16", pre.num_kv_heads)
    got = prefill_all(pre.q, pre.cu_q_lens, kp, vp, pre.block_tables, pre.context_lens, pre.scale,
                      "bf16", pre.num_kv_heads, rows_per_task=16)
    assert np.array_equal(got, want)
