"""The seeded input generator: determinism, allocator invariants, and agreement of its
slot mapping and pool contents with the oracle's translation (no GPU)."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import paged as O


def test_bf16_rounding_matches_torch():
    rng = np.random.Generator(np.random.PCG64(0))
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0, -1.0, 0.0, 3.0e38, 1e-40, 1.00390625, 1.01171875],
                                 dtype=np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(W.f32_to_bf16_bits(x), want)


def test_tiny_contains_worked_example():
    b = W.tiny()
    assert list(b.block_tables[0, :3]) == [7, 2, 5]
    assert list(b.context_lens) == [9, 5, 16]
    # the new (last) token of sequence 0 is position 8 -> slot 20 (physical #5, offset 0)
    assert b.slot_mapping[0] == 20 == O.slot_of(b.block_tables[0], 8, 4)
    used = [int(x) for x in b.block_tables.ravel() if x >= 0]
    assert len(used) == len(set(used)) == 3 + 2 + 4
    assert b.num_blocks == 32 and b.dtype == "f32" and b.scale == 1 / 8


@pytest.mark.parametrize("make", [lambda: W.gqa(num_seqs=8), W.tiny,
                                  lambda: W.long_context(num_seqs=2, ctx_range=(300, 900))])
def test_deterministic(make):
    a, b = make(), make()
    for f in ("context_lens", "block_tables", "q", "k_pool", "v_pool", "slot_mapping", "k_new"):
        assert np.array_equal(getattr(a, f).view(np.uint8), getattr(b, f).view(np.uint8)), f


def test_tables_waste_and_slots():
    b = W.gqa(num_seqs=12)
    bs = b.block_size
    seen = set()
    for s in range(b.num_seqs):
        n = int(b.context_lens[s])
        row = b.block_tables[s]
        valid = row[row >= 0]
        assert len(valid) == O.blocks_needed(n, bs)                 # on-demand paging
        assert 0 <= len(valid) * bs - n <= bs - 1                   # waste < one block
        assert np.all(row[len(valid):] == -1)
        assert not (set(valid.tolist()) & seen)                     # no accidental sharing
        seen |= set(valid.tolist())
        assert b.slot_mapping[s] == O.slot_of(row, n - 1, bs)       # the step's write slot
    assert b.num_blocks == int(np.ceil(1.25 * len(seen)))


def test_history_matches_oracle_gather():
    """The generator scatters history into the pool; the oracle gathers it through the
    table.  Referenced slots are finite, the new token's slot and unreferenced slots NaN."""
    b = W.gqa(num_seqs=3)
    for s in range(b.num_seqs):
        n = int(b.context_lens[s])
        for h in range(b.num_kv_heads):
            g = O.gather_kv(b.k_pool, b.block_tables[s], n, b.block_size, h, "bf16")
            assert np.isfinite(g[:n - 1]).all()
            assert np.isnan(g[n - 1]).all()
    refd = np.zeros(b.num_blocks, bool)
    refd[b.block_tables[b.block_tables >= 0]] = True
    k = O.widen(b.k_pool, "bf16")
    assert np.isnan(k[~refd]).all()


def test_allocator():
    a = W.BlockAllocator(6, np.array([3, 1, 4, 0, 5, 2]))
    x = a.allocate(4)
    assert x == [3, 1, 4, 0] and a.num_free() == 2
    assert a.allocate(3) is None                                    # short: caller preempts
    a.share(x[:2])
    a.release(x)
    assert a.num_free() == 4 and list(a.ref[[3, 1]]) == [1, 1]      # shared ones survive
    a.release(x[:2])
    assert a.num_free() == 6 and a.ref.sum() == 0


def test_prefix_cow_structure():
    p = W.prefix_cow(num_seqs=6)
    b = p.batch
    assert p.prefix_blocks.size == 128
    for s in range(b.num_seqs):
        assert np.array_equal(p.shared_tables[s, :128], p.prefix_blocks)
        assert np.array_equal(b.block_tables[s, :127], p.prefix_blocks[:127])
        assert b.block_tables[s, 127] == p.block_mapping[s, 1] != p.prefix_blocks[127]
        assert p.block_mapping[s, 0] == p.prefix_blocks[127]
    dst = p.block_mapping[:, 1]
    assert len(set(dst.tolist())) == len(dst) and not (set(dst.tolist()) & set(p.prefix_blocks.tolist()))


def test_mixed_structure():
    m = W.mixed(num_chunks=2, chunk_len=64, chunk_ctx=(100, 300), num_decode=4, decode_ctx=(20, 90))
    pre, dec = m.prefill, m.decode
    assert list(pre.cu_q_lens) == [0, 64, 128]
    assert dec.slot_mapping.shape[0] == 4 + 128 == dec.k_new.shape[0]
    for c in range(2):
        n = int(pre.context_lens[c])
        slots = dec.slot_mapping[4 + 64 * c: 4 + 64 * (c + 1)]
        want = [O.slot_of(pre.block_tables[c], t, 16) for t in range(n - 64, n)]
        assert list(slots) == want


def test_contiguous_slabs_hold_the_paged_values():
    """The unpaged layout carries the same values as the pool: history at the same
    positions, the step's new token at ctx - 1, the fill value past the context."""
    b = W.gqa(num_seqs=5, contiguous=True)
    kc = b.extra["k_cache"]
    assert kc.shape == (5, 4096, 8, 128)
    rng = np.random.default_rng(0)
    for s in range(5):
        n = int(b.context_lens[s])
        assert np.array_equal(kc[s, n - 1], b.k_new[s])
        assert np.array_equal(b.extra["v_cache"][s, n - 1], b.v_new[s])
        assert (kc[s, n:] == W.BF16_NAN).all()
        for t in rng.integers(0, n - 1, 20):
            pb, off = b.block_tables[s, t // b.block_size], t % b.block_size
            assert np.array_equal(kc[s, t], b.k_pool[pb, :, off])
    # the same draws as without the slabs
    b0 = W.gqa(num_seqs=5)
    assert np.array_equal(b0.k_pool, b.k_pool) and np.array_equal(b0.q, b.q)
