"""Shared-prefix decode on the GPU: groups of sequences whose block tables start with
the same physical blocks are decoded by the prefix pass (matrix cores, prefix K/V read
once per group) plus the decode of each member's own tokens, merged by log-sum-exp.
The result must be that of plain decode over the same tables: checked against the
oracle's decode (which knows nothing of groups) row by row, and at full size against
the library's plain decode on every row."""
import numpy as np
import pytest
import torch

import paged_kv_cache_79_amd as pkv
import workloads as W
from oracle import paged as O
from tests.gpu_helpers import (TOL, DecodeRun, dev, host, oracle_after_write, oracle_decode,
                               rownorm_err, widen_out)

pytestmark = pytest.mark.gpu


def run_shared(r, seq_prefix, gfirst, gnum, gpre, max_group_seqs=None, max_prefix_len=None,
               ctx=None, max_ctx=None, workspace=None):
    b = r.b
    out = torch.empty_like(r.q)
    mgs = int(gnum.max()) if max_group_seqs is None and gnum.size else (max_group_seqs or 0)
    mpl = int(gpre.max()) if max_prefix_len is None and gpre.size else (max_prefix_len or 0)
    pkv.paged_attention_decode_shared_prefix(
        out, r.q, r.k, r.v, r.tables, r.ctx if ctx is None else ctx,
        b.max_context_len if max_ctx is None else max_ctx, b.scale, dev(seq_prefix), dev(gfirst),
        dev(gnum), dev(gpre), mgs, mpl, workspace=workspace)
    torch.cuda.synchronize()
    return host(out)


def check_groups(pg, seqs=None, **kw):
    b = pg.batch
    print(f"shared prefix S={b.num_seqs} Hq={b.num_q_heads} Hkv={b.num_kv_heads} D={b.head_dim} "
          f"bs={b.block_size} groups={pg.group_num_seqs.tolist()} "
          f"prefix={pg.group_prefix_lens.tolist()} seed={b.seed}", flush=True)
    r = DecodeRun(b)
    r.write()
    got = run_shared(r, pg.seq_prefix_lens, pg.group_first_seq, pg.group_num_seqs,
                     pg.group_prefix_lens, **kw)
    k, v = oracle_after_write(b)
    want = oracle_decode(b, k, v, seqs=seqs)
    err = rownorm_err(widen_out(got, b.dtype), want)
    assert err <= TOL[b.dtype], f"row-normalised error {err:.3e}"
    return r, got


LAYOUTS = {
    # (members, prefix blocks); prefix 0: that many unshared sequences
    "one_group": [(5, 7)],
    "mixed": [(3, 4), (2, 0), (6, 9), (1, 0), (4, 1)],
    "single_member_groups": [(1, 5), (1, 12), (1, 3)],
}


@pytest.mark.parametrize("layout", list(LAYOUTS))
@pytest.mark.parametrize("g", [1, 4, 7, 8])
def test_group_sizes(layout, g):
    check_groups(W.prefix_groups(100 + g, LAYOUTS[layout], num_q_heads=2 * g, num_kv_heads=2))


@pytest.mark.parametrize("bs", [8, 16, 32])
def test_block_sizes_and_head_dim_64(bs):
    check_groups(W.prefix_groups(200 + bs, [(4, 96 // bs * 4), (2, 0), (3, 2)], head_dim=64,
                                 num_q_heads=8, num_kv_heads=4, block_size=bs))


def test_many_row_blocks_and_ragged_splits():
    """70 members at G=4 fill three 32-member row blocks (the last partly); a 1000-token
    prefix at block size 8 is cut into 4 splits of 256 keys, the last one ragged."""
    check_groups(W.prefix_groups(301, [(70, 125), (3, 0), (33, 40)], suffix_range=(1, 130),
                                 block_size=8))


def test_loose_host_bounds():
    """max_group_seqs and max_prefix_len above what the groups need: more splits and row
    blocks are launched and find no work."""
    pg = W.prefix_groups(302, [(4, 6), (2, 0), (3, 20)])
    check_groups(pg, max_group_seqs=100, max_prefix_len=5000)


def test_context_ending_at_the_prefix():
    """A member whose context ends exactly where its prefix ends has no tokens of its
    own: its result is the prefix pass's alone."""
    pg = W.prefix_groups(303, [(4, 5), (1, 0), (3, 8)])
    b = pg.batch
    r = DecodeRun(b)
    r.write()
    ctx = b.context_lens.copy()
    ctx[1] = pg.group_prefix_lens[0]            # member 1 of group 0
    ctx[7] = pg.group_prefix_lens[1]            # last member of group 1
    got = run_shared(r, pg.seq_prefix_lens, pg.group_first_seq, pg.group_num_seqs,
                     pg.group_prefix_lens, ctx=dev(ctx))
    k, v = oracle_after_write(b)
    want = O.decode(b.q, k, v, b.block_tables, ctx, b.scale, b.dtype, b.num_kv_heads)
    err = rownorm_err(widen_out(got, b.dtype), want)
    assert err <= TOL[b.dtype], f"row-normalised error {err:.3e}"


def test_no_groups_is_plain_decode():
    """num_groups == 0: the call is paged_attention_decode, bit for bit."""
    pg = W.prefix_groups(304, [(6, 0)])
    b = pg.batch
    r = DecodeRun(b)
    r.write()
    empty = np.zeros(0, dtype=np.int32)
    got = run_shared(r, np.zeros(b.num_seqs, dtype=np.int32), empty, empty, empty)
    assert np.array_equal(got, r.decode(0))


def test_repeated_calls_reuse_the_workspace():
    """The workspace needs no initialisation: after a call with other groups over the
    same (garbage-filled) workspace, a call gives the same bits as before."""
    pg = W.prefix_groups(305, [(5, 6), (2, 0), (4, 3)])
    b = pg.batch
    r = DecodeRun(b)
    r.write()
    need = pkv.paged_attention_decode_shared_prefix_workspace_bytes(
        b.num_seqs, b.num_q_heads, b.num_kv_heads, b.head_dim, b.max_context_len, 96)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
    full = (pg.seq_prefix_lens, pg.group_first_seq, pg.group_num_seqs, pg.group_prefix_lens)
    first = run_shared(r, *full, workspace=ws)
    # members 0 and 1 of the first group only, everything else unshared
    part = np.zeros(b.num_seqs, dtype=np.int32)
    part[:2] = 96
    other = run_shared(r, part, np.array([0], np.int32), np.array([2], np.int32),
                       np.array([96], np.int32), workspace=ws)
    again = run_shared(r, *full, workspace=ws)
    assert np.array_equal(first, again)
    k, v = oracle_after_write(b)
    want = oracle_decode(b, k, v)
    assert rownorm_err(widen_out(other, b.dtype), want) <= TOL[b.dtype]


def test_prefix_cow_full_size():
    """The 256-sequence copy-on-write batch: after the copy of each sequence's last
    prefix block, 127 blocks (2032 tokens) are still shared by all 256 sequences.
    Sampled rows against the oracle, every row against plain decode."""
    pc = W.prefix_cow()
    b = pc.batch
    print(f"prefix_cow S={b.num_seqs} max_ctx={b.max_context_len}", flush=True)
    r = DecodeRun(b)
    pkv.copy_blocks(r.k, r.v, dev(pc.block_mapping))
    r.write()
    shared_tokens = (len(pc.prefix_blocks) - 1) * b.block_size
    S = b.num_seqs
    seq_prefix = np.full(S, shared_tokens, dtype=np.int32)
    got = run_shared(r, seq_prefix, np.array([0], np.int32), np.array([S], np.int32),
                     np.array([shared_tokens], np.int32))
    plain = r.decode(0)
    assert rownorm_err(widen_out(got, b.dtype), widen_out(plain, b.dtype)) <= TOL[b.dtype]
    k = O.kv_write(O.copy_blocks(b.k_pool, pc.block_mapping), b.k_new, b.slot_mapping)
    v = O.kv_write(O.copy_blocks(b.v_pool, pc.block_mapping), b.v_new, b.slot_mapping)
    rng = np.random.Generator(np.random.PCG64(9))
    seqs = sorted(rng.choice(S, 8, replace=False).tolist())
    want = oracle_decode(b, k, v, seqs=seqs)
    err = rownorm_err(widen_out(got, b.dtype), want)
    assert err <= TOL[b.dtype], f"row-normalised error {err:.3e}"
    # before copy-on-write re-pointed them, all 128 prefix blocks were shared
    r.tables = dev(pc.shared_tables)
    whole = run_shared(r, np.full(S, shared_tokens + b.block_size, dtype=np.int32),
                       np.array([0], np.int32), np.array([S], np.int32),
                       np.array([shared_tokens + b.block_size], np.int32))
    assert rownorm_err(widen_out(whole, b.dtype), want) <= TOL[b.dtype]


def test_many_sequences():
    """470 sequences in three groups and a run of unshared ones: the own-token decode
    counts and locates past the first 256 sequences. Sampled rows against the oracle,
    every row against plain decode."""
    pg = W.prefix_groups(306, [(150, 3), (200, 0), (120, 5)], suffix_range=(1, 150))
    S = pg.batch.num_seqs
    seqs = [0, 149, 150, 255, 256, 349, 350, 469]
    rng = np.random.Generator(np.random.PCG64(307))
    seqs = sorted(set(seqs) | set(rng.choice(S, 12, replace=False).tolist()))
    r, got = check_groups(pg, seqs=seqs)
    b = pg.batch
    assert rownorm_err(widen_out(got, b.dtype), widen_out(r.decode(0), b.dtype)) <= TOL[b.dtype]
