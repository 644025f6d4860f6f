"""Host-side check of the chunked prefill's balanced key split (no GPU).

Replays the split's arithmetic (tests/prefill_plan.py restates it) on random chunk
mixes: every key tile of every work item is attended exactly once, no partial slot
is written twice, and the merge reads exactly the slots written for each cut item,
in key order.  Also checks when the split applies at the mixed workload's shape."""
import numpy as np
import pytest

from tests import prefill_plan as PP


def check(cu, ctx, group, hkv, W, max_q_len):
    split, T, items = PP.plan(cu, ctx, group, hkv, W, max_q_len, 1 << 30)
    if not split:
        return False
    W = PP.ranges(T, W)
    order, starts, pieces = PP.walk(T, W, items, hkv)
    for w in range(W):
        assert PP.begin(T, W, w) < PP.begin(T, W, w + 1)       # no empty range
    covered = {}
    slots = set()
    by_item = {}
    for w, it, k0, k1, slot in pieces:
        for t in range(k0, k1):
            assert (it, t) not in covered
            covered[(it, t)] = w
        if slot >= 0:
            assert slot not in slots and 0 <= slot < 2 * W
            slots.add(slot)
        by_item.setdefault(it, []).append((k0, slot))
    assert len(covered) == T
    for (c, h, qt, n), s in zip(order, starts):
        got = sorted(by_item[(c, h, qt)])
        want = PP.merge_slots(T, W, s, n)
        if want is None:
            assert got == [(0, -1)]
        else:
            assert [sl for _, sl in got] == want
    return True


@pytest.mark.parametrize("seed", range(60))
def test_split_covers_and_merges(seed):
    """Random mixes sized so that the items fit in one round (the only case that
    splits): 1 to 8 kv heads, groups 1..8, up to 300 queries per chunk, up to several
    hundred chunks (past the 64 chunks of one scan pass), contexts with 0..20000 keys
    before the chunk."""
    rng = np.random.default_rng(seed)
    group = int(rng.choice([1, 2, 3, 4, 7, 8]))
    hkv = int(rng.integers(1, 9))
    W = int(rng.choice([8, 64, 512, 1024]))
    maxq = int(rng.integers(1, 300))
    nqt = -(-maxq // (128 // group))
    nc = int(rng.integers(1, max(2, W // (hkv * nqt)) + 1))
    nq = rng.integers(1, maxq + 1, nc)
    nq[0] = maxq
    ctx = nq + rng.integers(0, 20000, nc) * (rng.random(nc) < 0.7)
    cu = np.concatenate([[0], np.cumsum(nq)])
    check(cu, ctx, group, hkv, W, maxq)


def test_random_mixes_exercise_the_split():
    hits = 0
    for seed in range(60):
        rng = np.random.default_rng(seed)
        group = int(rng.choice([1, 2, 3, 4, 7, 8]))
        hkv = int(rng.integers(1, 9))
        W = int(rng.choice([8, 64, 512, 1024]))
        maxq = int(rng.integers(1, 300))
        nqt = -(-maxq // (128 // group))
        nc = int(rng.integers(1, max(2, W // (hkv * nqt)) + 1))
        nq = rng.integers(1, maxq + 1, nc)
        nq[0] = maxq
        ctx = nq + rng.integers(0, 20000, nc) * (rng.random(nc) < 0.7)
        cu = np.concatenate([[0], np.cumsum(nq)])
        hits += PP.plan(cu, ctx, group, hkv, W, maxq, 1 << 30)[0]
    assert hits >= 30


def test_mixed_shape_splits():
    """4 chunks of 512 queries over contexts of 3869..7604 keys (32/8 heads): one round of
    512 workgroups whose longest chunk holds 119 tiles against an even share of 87."""
    ctx = np.array([4992, 7604, 5514, 3869])
    cu = np.array([0, 512, 1024, 1536, 2048])
    assert check(cu, ctx, 4, 8, 512, 512)


def test_even_or_large_batches_do_not_split():
    cu = np.array([0, 2048])
    assert not PP.plan(cu, np.array([32768]), 4, 8, 512, 2048, 1 << 30)[0]   # even items
    cu8 = np.arange(9) * 2048
    assert not PP.plan(cu8, np.full(8, 8192), 4, 8, 512, 2048, 1 << 30)[0]   # 4096 items


def test_one_long_chunk_splits_into_many_pieces():
    """One chunk of 100 queries over 40000 keys: 8 items over 512 workgroups, so each
    row merges ~64 pieces (several batches of the merge)."""
    cu = np.array([0, 100])
    ctx = np.array([40000])
    assert check(cu, ctx, 4, 2, 512, 100)
    split, T, items = PP.plan(cu, ctx, 4, 2, 512, 100, 1 << 30)
    order, starts, _ = PP.walk(T, PP.ranges(T, 512), items, 2)
    assert max(len(PP.merge_slots(T, 512, s, n) or []) for (_, _, _, n), s in zip(order, starts)) > 16


def test_fewer_tiles_than_workgroups():
    """Two chunks of 37 and 64 queries over 100 and 64 keys, 14 q / 2 kv heads: 20 tiles
    for 512 workgroups, so the split uses 20 ranges of one tile (with 512 ranges the
    merge of a 2-tile item would span 26 workgroups, 25 of them with nothing written)."""
    cu = np.array([0, 37, 101])
    ctx = np.array([100, 64])
    assert check(cu, ctx, 7, 2, 512, 64)
    assert PP.plan(cu, ctx, 7, 2, 512, 64, 1 << 30)[1] == 20
