"""Pins of the CPU oracle to facts outside itself (no GPU).

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
what the pages or mathematics fix: the worked example of the "2.1
PagedAttention" chapter, a library attention routine, closed forms, paging
invariants and the vAttention page's sizing.  ``test_mutants_are_caught``
plants plausible mistakes in the oracle (on the CPU) and checks that at least
one pin fails for each.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import paged as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example_bs4.txt")


# --------------------------------------------------------------------------
# helpers
# --------------------------------------------------------------------------
def load_golden():
    g = {"tokens": [], "growth": []}
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].split()
        if not line:
            continue
        key, vals = line[0], [int(v) for v in line[1:]]
        if key == "block_size":
            g["bs"] = vals[0]
        elif key == "table":
            g["table"] = vals
        elif key == "token":
            g["tokens"].append(vals)
        elif key == "fill":
            g["fill"] = vals
        elif key == "growth":
            g["growth"].append(vals)
        elif key == "needs_new_block":
            g["needs"] = vals
    return g


def rnd(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


def contiguous_case(seed, ctx, hq, hkv, d, bs, dtype="f32"):
    """Pool where sequence s occupies consecutive blocks in logical order (identity tables),
    plus dense float64 histories [S][Hkv][n][D] read straight from the pool's layout."""
    rng = np.random.Generator(np.random.PCG64(seed))
    need = [-(-c // bs) for c in ctx]
    nb = sum(need)
    mb = max(need)
    tables = -np.ones((len(ctx), mb), dtype=np.int64)
    b = 0
    for s, n in enumerate(need):
        tables[s, :n] = np.arange(b, b + n)
        b += n
    k = rng.standard_normal((nb, hkv, bs, d)).astype(np.float32)
    v = rng.standard_normal((nb, hkv, bs, d)).astype(np.float32)
    q = rng.standard_normal((len(ctx), hq, d)).astype(np.float32)
    return q, k, v, tables


def dense_history(pool, tables, ctx, s, bs):
    """With identity tables a sequence's blocks are consecutive, so its history is the
    pool slice [first block, first block + nblocks) with (block, slot) flattened."""
    first = int(tables[s, 0])
    nbk = -(-ctx[s] // bs)
    seg = pool[first:first + nbk]                # [nbk][Hkv][bs][D]
    seg = np.transpose(seg, (1, 0, 2, 3)).reshape(pool.shape[1], nbk * bs, pool.shape[3])
    return seg[:, :ctx[s]].astype(np.float64)    # [Hkv][n][D]


def sdpa(q, k, v, scale, causal=False, mask=None):
    """torch's scaled_dot_product_attention on CPU in float64, grouped heads by the library."""
    qt = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float64))
    kt = torch.from_numpy(np.ascontiguousarray(k, dtype=np.float64))
    vt = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float64))
    return torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=mask, is_causal=causal, scale=scale, enable_gqa=True).numpy()


# --------------------------------------------------------------------------
# pins
# --------------------------------------------------------------------------
def pin_worked_example():
    g = load_golden()
    bs, table = g["bs"], g["table"]
    for pos, lb, pb, off, slot in g["tokens"]:
        assert O.translate(table, pos, bs) == (lb, pb, off), pos
        assert O.slot_of(table, pos, bs) == slot, pos
    fills = [0] * len(table)
    for pos, lb, *_ in g["tokens"]:
        fills[lb] += 1
    assert fills == g["fill"]
    assert O.blocks_needed(len(g["tokens"]), bs) == len(table)
    for pos, slot in g["growth"]:
        assert O.slot_of(table, pos, bs) == slot
    pos, lb = g["needs"]
    with pytest.raises(IndexError):
        O.translate(table, pos, bs)
    assert O.translate(table + [11], pos, bs) == (lb, 11, 0)


def pin_worked_example_write_gather():
    """Writing the example's 9 tokens through their slots and gathering them back through
    the table returns them in logical order; nothing else in the pool changes."""
    g = load_golden()
    bs, table = g["bs"], g["table"]
    hkv, d = 2, 3
    pool = np.full((8, hkv, bs, d), np.nan, dtype=np.float32)
    new = (np.arange(9 * hkv * d, dtype=np.float32).reshape(9, hkv, d) + 1.0)
    slots = [row[4] for row in g["tokens"]]
    out = O.kv_write(pool, new, slots)
    for h in range(hkv):
        np.testing.assert_array_equal(O.gather_kv(out, table, 9, bs, h, "f32"), new[:, h, :])
    # token 8 sits in slot 0 of block #5; the rest of block #5 and blocks 0,1,3,4,6 untouched
    np.testing.assert_array_equal(out[5, :, 0, :], new[8])
    assert np.isnan(out[5, :, 1:, :]).all()
    for b in (0, 1, 3, 4, 6):
        assert np.isnan(out[b]).all()
    # a negative slot writes nothing
    same = O.kv_write(out, new[:1] * 0, [-1])
    assert np.array_equal(same.view(np.uint32), out.view(np.uint32))


def pin_bf16_widening():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0x0001, 0x3EAA, 0x4049], dtype=np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, math.inf, 2.0 ** -133, 0.33203125, 3.140625]
    got = O.widen(bits, "bf16")
    for g_, w in zip(got, want):
        assert g_ == w and math.copysign(1, g_) == math.copysign(1, w)
    assert np.isnan(O.widen(np.array([0x7FC0], dtype=np.uint16), "bf16"))[0]


def pin_decode_vs_library(seed=1, ctx=(1, 7, 13, 32), hq=8, hkv=2, d=16, bs=4):
    q, k, v, tables = contiguous_case(seed, list(ctx), hq, hkv, d, bs)
    scale = 0.37
    got = O.decode(q, k, v, tables, np.array(ctx), scale, "f32", hkv)
    for s, n in enumerate(ctx):
        K = dense_history(k, tables, list(ctx), s, bs)[None]   # [1][Hkv][n][D]
        V = dense_history(v, tables, list(ctx), s, bs)[None]
        want = sdpa(q[s][None, :, None, :].astype(np.float64), K, V, scale)[0, :, 0, :]
        np.testing.assert_allclose(got[s], want, rtol=1e-12, atol=1e-12)


def pin_contiguous_decode(seed=3, ctx=(0, 1, 9, 64, 100), hq=6, hkv=3, d=8, L=128, bs=4):
    """The contiguous-layout decode equals SDPA on each slab, gives a zero row for an
    empty context, and equals the paged decode of a pool cut from the same slabs into
    shuffled blocks of bs tokens."""
    rng = np.random.default_rng(seed)
    S = len(ctx)
    q = rng.standard_normal((S, hq, d)).astype(np.float32)
    kc = rng.standard_normal((S, L, hkv, d)).astype(np.float32)
    vc = rng.standard_normal((S, L, hkv, d)).astype(np.float32)
    got = O.decode_contiguous(q, kc, vc, np.array(ctx), 0.29, "f32", hkv)
    for s, n in enumerate(ctx):
        if n == 0:
            assert np.array_equal(got[s], np.zeros((hq, d)))
            continue
        K = np.transpose(kc[s, :n], (1, 0, 2))[None].astype(np.float64)  # [1][Hkv][n][D]
        V = np.transpose(vc[s, :n], (1, 0, 2))[None].astype(np.float64)
        want = sdpa(q[s][None, :, None, :].astype(np.float64), K, V, 0.29)[0, :, 0, :]
        np.testing.assert_allclose(got[s], want, rtol=1e-12, atol=1e-12)
    # the same slabs cut into blocks of bs tokens at shuffled physical ids
    mb = L // bs
    perm = rng.permutation(S * mb)
    tables = perm.reshape(S, mb).astype(np.int32)
    kp = np.empty((S * mb, hkv, bs, d), np.float32)
    vp = np.empty_like(kp)
    for s in range(S):
        for b in range(mb):
            kp[tables[s, b]] = np.transpose(kc[s, b * bs:(b + 1) * bs], (1, 0, 2))
            vp[tables[s, b]] = np.transpose(vc[s, b * bs:(b + 1) * bs], (1, 0, 2))
    paged = O.decode(q, kp, vp, tables, np.array(ctx), 0.29, "f32", hkv)
    np.testing.assert_allclose(got, paged, rtol=1e-12, atol=1e-12)


def pin_swap_round_trip():
    """Swap-out copies the listed device blocks into host blocks bit for bit; swapping
    them back into other device blocks restores their contents; nothing else changes."""
    rng = np.random.default_rng(8)
    dev_pool = rng.standard_normal((6, 2, 4, 3)).astype(np.float32)
    host_pool = np.full((3, 2, 4, 3), np.nan, np.float32)
    out = O.swap_blocks(host_pool, dev_pool, [[4, 0], [1, 2]])
    assert np.array_equal(out[0].view(np.uint32), dev_pool[4].view(np.uint32))
    assert np.array_equal(out[2].view(np.uint32), dev_pool[1].view(np.uint32))
    assert np.isnan(out[1]).all()
    back = O.swap_blocks(np.zeros_like(dev_pool), out, [[0, 5], [2, 0]])
    assert np.array_equal(back[5], dev_pool[4]) and np.array_equal(back[0], dev_pool[1])
    assert (back[1:5] == 0).all()


def relabel(pool_list, tables, perm):
    """Move physical block b to perm[b] and rewrite the tables to match."""
    outs = []
    for p in pool_list:
        o = np.empty_like(p)
        o[perm] = p
        outs.append(o)
    t = np.where(tables >= 0, perm[np.maximum(tables, 0)], -1)
    return outs, t


def pin_permutation_invariance(seed=2):
    ctx = [5, 16, 9]
    q, k, v, tables = contiguous_case(seed, ctx, 4, 4, 8, 4)
    base = O.decode(q, k, v, tables, np.array(ctx), 0.5, "f32", 4)
    perm = np.random.Generator(np.random.PCG64(seed)).permutation(k.shape[0])
    (k2, v2), t2 = relabel([k, v], tables, perm)
    got = O.decode(q, k2, v2, t2, np.array(ctx), 0.5, "f32", 4)
    assert np.array_equal(got, base)


def pin_closed_forms(seed=3):
    d, bs = 8, 4
    rng = np.random.Generator(np.random.PCG64(seed))
    k = rng.standard_normal((4, 1, bs, d)).astype(np.float32)
    v = rng.standard_normal((4, 1, bs, d)).astype(np.float32)
    table = np.array([[2, 0, 3, 1]])
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    # one token: the output is that token's V row
    out = O.decode(q, k, v, table, np.array([1]), 0.3, "f32", 1)
    assert np.array_equal(out[0, 0], v[2, 0, 0].astype(np.float64))
    # zero query: uniform weights, the mean of the V rows
    out = O.decode(np.zeros_like(q), k, v, table, np.array([11]), 0.3, "f32", 1)
    rows = np.concatenate([v[2, 0], v[0, 0], v[3, 0, :3]]).astype(np.float64)
    np.testing.assert_allclose(out[0, 0], rows.mean(axis=0), rtol=1e-13, atol=1e-14)
    # identical keys: again the mean
    k_eq = np.broadcast_to(k[2, 0, 0], k.shape).copy()
    out = O.decode(q, k_eq, v, table, np.array([11]), 0.3, "f32", 1)
    np.testing.assert_allclose(out[0, 0], rows.mean(axis=0), rtol=1e-13, atol=1e-14)
    # empty context: zeros
    out = O.decode(q, k, v, table, np.array([0]), 0.3, "f32", 1)
    assert np.array_equal(out[0, 0], np.zeros(d))


def pin_one_hot_probe(seed=4):
    """q = 64 e0, the target token's K[0] = +64 and every other K[0] = -64: the score gap
    is 64*64*2*scale, exp underflows to 0 for every other token, and the output is the
    target's V row exactly -- for every target position, including the tail block."""
    d, bs, n = 16, 4, 11
    rng = np.random.Generator(np.random.PCG64(seed))
    table = np.array([[5, 1, 6]])
    v = rng.standard_normal((8, 1, bs, d)).astype(np.float32)
    q = np.zeros((1, 1, d), dtype=np.float32)
    q[0, 0, 0] = 64.0
    for target in range(n):
        k = np.zeros((8, 1, bs, d), dtype=np.float32)
        for t in range(n):
            _, pb, off = O.translate(table[0], t, bs)
            k[pb, 0, off, 0] = 64.0 if t == target else -64.0
        out = O.decode(q, k, v, table, np.array([n]), 1.0 / math.sqrt(d), "f32", 1)
        _, pb, off = O.translate(table[0], target, bs)
        assert np.array_equal(out[0, 0], v[pb, 0, off].astype(np.float64)), target


def pin_nan_poison(seed=5):
    """Slots and blocks outside each sequence's valid length hold NaN: the output is the
    same as with zeros there ("vAttention": the valid length bounds what a kernel sees)."""
    ctx = [6, 9]
    q, k, v, tables = contiguous_case(seed, ctx, 2, 1, 8, 4)
    kz, vz = k.copy(), v.copy()
    extra = np.zeros((3,) + k.shape[1:], dtype=np.float32)
    kz = np.concatenate([kz, extra])
    vz = np.concatenate([vz, extra])
    kn, vn = kz.copy(), vz.copy()
    for s, n in enumerate(ctx):
        for t in range(n, -(-n // 4) * 4):
            _, pb, off = O.translate(tables[s], t, 4)
            kn[pb, :, off] = np.nan
            vn[pb, :, off] = np.nan
    kn[-3:] = np.nan
    vn[-3:] = np.nan
    a = O.decode(q, kz, vz, tables, np.array(ctx), 0.4, "f32", 1)
    b = O.decode(q, kn, vn, tables, np.array(ctx), 0.4, "f32", 1)
    assert np.isfinite(b).all() and np.array_equal(a, b)


def pin_prefix_sharing(seed=6):
    """Two tables pointing at the same prefix blocks give the same output as private
    copies of those blocks ("2.1 PagedAttention", section 6)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    bs, d = 4, 8
    k = rng.standard_normal((10, 2, bs, d)).astype(np.float32)
    v = rng.standard_normal((10, 2, bs, d)).astype(np.float32)
    k[7:9], v[7:9] = k[0:2], v[0:2]                     # private copies of blocks 0, 1
    shared = np.array([[0, 1, 2, -1], [0, 1, 3, 4]])
    private = np.array([[0, 1, 2, -1], [7, 8, 3, 4]])
    q = rng.standard_normal((2, 4, d)).astype(np.float32)
    ctx = np.array([10, 14])
    a = O.decode(q, k, v, shared, ctx, 0.3, "f32", 2)
    b = O.decode(q, k, v, private, ctx, 0.3, "f32", 2)
    assert np.array_equal(a, b)


def pin_cow_divergence():
    """Copy-on-write ("2.1 PagedAttention", section 6): A and B share block #5, which holds
    token 8 (1/4 full).  B must write token 9 there, so #5 is copied to a private block,
    B's table is re-pointed, and the write lands in the copy; A is untouched."""
    bs, d, hkv = 4, 4, 1
    rng = np.random.Generator(np.random.PCG64(7))
    k = np.full((12, hkv, bs, d), np.nan, dtype=np.float32)
    v = np.full((12, hkv, bs, d), np.nan, dtype=np.float32)
    table_a = [7, 2, 5]
    hist_k = rng.standard_normal((9, hkv, d)).astype(np.float32)
    hist_v = rng.standard_normal((9, hkv, d)).astype(np.float32)
    slots = [O.slot_of(table_a, t, bs) for t in range(9)]
    k, v = O.kv_write(k, hist_k, slots), O.kv_write(v, hist_v, slots)
    q = rng.standard_normal((1, 2, d)).astype(np.float32)
    before = O.decode(q, k, v, np.array([table_a]), np.array([9]), 0.5, "f32", 1)
    k2 = O.copy_blocks(k, [[5, 9]])
    v2 = O.copy_blocks(v, [[5, 9]])
    assert np.array_equal(k2[9].view(np.uint32), k[5].view(np.uint32))
    table_b = [7, 2, 9]
    nk = rng.standard_normal((1, hkv, d)).astype(np.float32)
    nv = rng.standard_normal((1, hkv, d)).astype(np.float32)
    s9 = O.slot_of(table_b, 9, bs)
    assert s9 == 37
    k2, v2 = O.kv_write(k2, nk, [s9]), O.kv_write(v2, nv, [s9])
    after_a = O.decode(q, k2, v2, np.array([table_a]), np.array([9]), 0.5, "f32", 1)
    assert np.array_equal(before, after_a)
    gb = O.gather_kv(k2, table_b, 10, bs, 0, "f32")
    np.testing.assert_array_equal(gb[:9], hist_k[:, 0])
    np.testing.assert_array_equal(gb[9], nk[0, 0])
    assert np.isnan(k2[5, :, 1:]).all()               # A's block did not receive token 9


def pin_copy_blocks_snapshot():
    pool = np.arange(6 * 2 * 2 * 3, dtype=np.float32).reshape(6, 2, 2, 3)
    out = O.copy_blocks(pool, [[1, 2], [3, 4]])
    np.testing.assert_array_equal(out[2], pool[1])
    np.testing.assert_array_equal(out[4], pool[3])
    for b in (0, 1, 3, 5):
        np.testing.assert_array_equal(out[b], pool[b])
    # reads see the pool as it was before the call, whatever the pair order
    out = O.copy_blocks(pool, [[2, 5], [0, 2]])
    np.testing.assert_array_equal(out[5], pool[2])
    np.testing.assert_array_equal(out[2], pool[0])


def pin_prefill_vs_library(seed=8):
    """A chunk that is the whole context is ordinary causal self-attention (SDPA is_causal);
    a shorter chunk's row i equals decode on the first ctx - n_q + i + 1 tokens."""
    bs, hq, hkv, d = 4, 6, 2, 8
    ctx = [9, 14]
    q, k, v, tables = contiguous_case(seed, ctx, hq, hkv, d, bs)
    rng = np.random.Generator(np.random.PCG64(seed + 100))
    qc = rng.standard_normal((sum(ctx), hq, d)).astype(np.float32)
    cu = np.array([0, ctx[0], ctx[0] + ctx[1]])
    got = O.prefill_chunk(qc, cu, k, v, tables, np.array(ctx), 0.35, "f32", hkv)
    for c, n in enumerate(ctx):
        K = dense_history(k, tables, ctx, c, bs)[None]
        V = dense_history(v, tables, ctx, c, bs)[None]
        qq = np.transpose(qc[cu[c]:cu[c + 1]], (1, 0, 2))[None].astype(np.float64)
        want = sdpa(qq, K, V, 0.35, causal=True)[0]      # [Hq][n][D]
        np.testing.assert_allclose(got[cu[c]:cu[c + 1]], np.transpose(want, (1, 0, 2)),
                                   rtol=1e-12, atol=1e-12)
    # shorter chunks: 3 queries at the end of each context
    nq = 3
    cu2 = np.array([0, nq, 2 * nq])
    q2 = qc[:2 * nq]
    got2 = O.prefill_chunk(q2, cu2, k, v, tables, np.array(ctx), 0.35, "f32", hkv)
    for c, n in enumerate(ctx):
        for i in range(nq):
            ref = O.decode(q2[cu2[c] + i][None], k, v, tables[c:c + 1], np.array([n - nq + i + 1]),
                           0.35, "f32", hkv)
            np.testing.assert_allclose(got2[cu2[c] + i], ref[0], rtol=1e-13, atol=1e-13)


def pin_lse_merge(seed=9):
    rng = np.random.Generator(np.random.PCG64(seed))
    n, d = 57, 8
    K, V = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    q = rng.standard_normal(d) * 3
    whole = O.attend(q, K, V, 0.7)
    for cuts in ([], [1], [16, 32, 48], sorted(rng.choice(np.arange(1, n), 9, replace=False))):
        edges = [0] + list(cuts) + [n]
        parts = O.partition_partials(q, K, V, 0.7, list(zip(edges[:-1], edges[1:])))
        np.testing.assert_allclose(O.lse_merge(parts), whole, rtol=1e-12, atol=1e-13)


def pin_kv_size_model():
    """vAttention page, Yi-34B FP16 TP=2: 60 layers, 4 local KV heads, D 128, L 200K.
    One layer's K (or V) slot is about 200 MB; 500 slots about 100 GB; K and V of all
    60 layers about 12 TB of virtual space."""
    per_slot_k = O.kv_size_bytes(1, 200_000, 4, 128, 2) // 2
    assert per_slot_k == 204_800_000
    assert abs(per_slot_k / 1e6 - 200) / 200 < 0.05
    assert abs(500 * per_slot_k / 1e9 - 100) / 100 < 0.05
    total = 500 * O.kv_size_bytes(60, 200_000, 4, 128, 2)
    assert abs(total / 1e12 - 12) / 12 < 0.05


def pin_waste_bound():
    for bs in (4, 8, 16, 32):
        for n in range(1, 200):
            w = O.tail_waste(n, bs)
            assert 0 <= w <= bs - 1
            assert O.blocks_needed(n, bs) * bs - n == w
    assert O.tail_waste(9, 4) == 3          # the worked example's 3 free slots in #5


PINS = [pin_worked_example, pin_worked_example_write_gather, pin_bf16_widening,
        pin_decode_vs_library, pin_permutation_invariance, pin_closed_forms, pin_one_hot_probe,
        pin_nan_poison, pin_prefix_sharing, pin_cow_divergence, pin_copy_blocks_snapshot,
        pin_prefill_vs_library, pin_lse_merge, pin_kv_size_model, pin_waste_bound,
        pin_contiguous_decode, pin_swap_round_trip]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# --------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail
# --------------------------------------------------------------------------
def _mut_offset(table_row, t, block_size):
    lb = t // block_size
    if lb >= len(table_row) or table_row[lb] < 0:
        raise IndexError
    return lb, int(table_row[lb]), (t + 1) % block_size


def _mut_gather_transposed(pool, table_row, n, block_size, kv_head, dtype):
    t = np.arange(n)
    pb = np.asarray(table_row)[t // block_size]
    return O.widen(pool[pb, kv_head, (block_size - 1 - t % block_size), :], dtype)


def _mut_heads(hq, num_q_heads, num_kv_heads):
    return hq % num_kv_heads


def _mut_attend_noscale(q, K, V, scale):
    s = K @ np.asarray(q, dtype=np.float64)
    w = np.exp(s - s.max()) if len(s) else s
    return (w @ V) / w.sum() if len(s) else np.zeros(V.shape[1])


def _mut_attend_sign(q, K, V, scale):
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    s = -scale * (K @ np.asarray(q, dtype=np.float64))
    w = np.exp(s - s.max())
    return (w @ V) / w.sum()


def _mut_attend_drop_last(q, K, V, scale):
    if K.shape[0] <= 1:
        return np.zeros(V.shape[1]) if K.shape[0] == 0 else V[0].copy()
    s = scale * (K[:-1] @ np.asarray(q, dtype=np.float64))
    w = np.exp(s - s.max())
    return (w @ V[:-1]) / w.sum()


def _mut_lse(parts):
    M = max(m for m, _, _ in parts)
    num = sum(np.exp(m - M) * o for m, _, o in parts)
    den = sum(l for m, l, _ in parts)
    return num / den


def _mut_widen(a, dtype):
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
        return bits.view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


_orig_kv_write = O.kv_write


def _mut_kv_write(pool, new, slot_mapping):
    return _orig_kv_write(pool, new, [s + 1 if s >= 0 else s for s in slot_mapping])


_orig_copy = O.copy_blocks


def _mut_copy(pool, block_mapping):
    m = np.asarray(block_mapping).reshape(-1, 2)[:, ::-1]
    return _orig_copy(pool, m)


_orig_prefill = O.prefill_chunk


def _mut_prefill_exclusive(q, cu_q_lens, k_pool, v_pool, block_tables, context_lens, scale,
                           dtype, num_kv_heads, rows=None):
    # sees one key less than it should (t < p instead of t <= p)
    shifted = np.maximum(np.asarray(context_lens) - 0, 0)
    out = np.full(q.shape, np.nan)
    for c in range(len(context_lens)):
        q0, q1 = int(cu_q_lens[c]), int(cu_q_lens[c + 1])
        nq, n = q1 - q0, int(shifted[c])
        for i in range(nq):
            pos = n - nq + i
            for hq in range(q.shape[1]):
                h = O.kv_head_of(hq, q.shape[1], num_kv_heads)
                K = O.gather_kv(k_pool, block_tables[c], n, k_pool.shape[2], h, dtype)
                V = O.gather_kv(v_pool, block_tables[c], n, v_pool.shape[2], h, dtype)
                out[q0 + i, hq] = O.attend(O.widen(q[q0 + i, hq], dtype), K[:max(pos, 1)],
                                           V[:max(pos, 1)], scale)
    return out


def _mut_contiguous_heads(q, k_cache, v_cache, context_lens, scale, dtype, num_kv_heads,
                          seqs=None, heads=None):
    """Interleaved instead of consecutive query-head groups on the contiguous layout."""
    S, Hq, D = q.shape
    out = np.full((S, Hq, D), np.nan)
    for s in range(S):
        n = int(context_lens[s])
        for hq in range(Hq):
            h = hq % num_kv_heads
            out[s, hq] = O.attend(O.widen(q[s, hq], dtype), O.widen(k_cache[s, :n, h], dtype),
                                  O.widen(v_cache[s, :n, h], dtype), scale)
    return out


def _mut_size(layers, length, kv_heads, head_dim, elem_bytes):
    return layers * length * kv_heads * head_dim * elem_bytes


MUTANTS = {
    "translate_offset": ("translate", _mut_offset),
    "gather_reversed_slots": ("gather_kv", _mut_gather_transposed),
    "gqa_interleaved": ("kv_head_of", _mut_heads),
    "attend_no_scale": ("attend", _mut_attend_noscale),
    "attend_wrong_sign": ("attend", _mut_attend_sign),
    "attend_drops_last_token": ("attend", _mut_attend_drop_last),
    "lse_unweighted_denominator": ("lse_merge", _mut_lse),
    "widen_wrong_shift": ("widen", _mut_widen),
    "kv_write_off_by_one": ("kv_write", _mut_kv_write),
    "copy_reversed_pairs": ("copy_blocks", _mut_copy),
    "prefill_exclusive_causal": ("prefill_chunk", _mut_prefill_exclusive),
    "size_model_missing_factor_2": ("kv_size_bytes", _mut_size),
    "contiguous_interleaved_heads": ("decode_contiguous", _mut_contiguous_heads),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutants_are_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, IndexError, ValueError, pytest.fail.Exception):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name!r}"
