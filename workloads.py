"""Seeded synthetic inputs for the paged KV-cache attention path.

This module plays the role the serving engine's scheduler and block allocator
play around the kernels: it picks context lengths, hands out physical blocks
from a shuffled free pool, fills the cache with the history K/V that earlier
forward passes would have written, and produces the slot mapping and new-token
K/V of the current step. It holds none of the attention arithmetic.

Both the CPU oracle (``oracle/``) and the HIP library are fed from the arrays
built here; neither imports the other.

Conventions (all stated readings of the pages):
  * pool layout ``[num_blocks][num_kv_heads][block_size][head_dim]`` for K and
    for V separately;
  * a context length counts the token(s) written in the current step
    (the step's target length is "computed + scheduled"), so a decode query
    sits at position ``ctx - 1`` and its K/V are written through
    ``slot_mapping`` before attention;
  * ``slot = physical_block * block_size + offset`` (int64), negative = skip;
  * block-table padding beyond ``ceil(ctx / block_size)`` is -1;
  * bf16 tensors are carried as uint16 bit patterns, rounded from fp32
    ``standard_normal`` draws to nearest-even;
  * slots that no sequence references hold NaN in parity runs (``poison``)
    and zeros in benchmark runs, so an out-of-bounds read shows up.

Recipe (draw order per workload, one ``numpy.random.Generator(PCG64(seed))``):
context lengths -> free-pool permutation -> q -> history K/V (sequence by
sequence, logical order, K then V) -> new-token K/V.  Seeds are
``79000 + k`` for the five named workloads k = 1..5.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BF16 = "bf16"
F32 = "f32"

BF16_NAN = np.uint16(0x7FC0)


# --------------------------------------------------------------------------
# element encoding
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def _encode(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == BF16 else np.ascontiguousarray(x, dtype=np.float32)


def _storage(dtype: str):
    return np.uint16 if dtype == BF16 else np.float32


def _fill_value(dtype: str, poison: bool):
    if not poison:
        return 0
    return BF16_NAN if dtype == BF16 else np.float32(np.nan)


def element_bytes(dtype: str) -> int:
    return 2 if dtype == BF16 else 4


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


# --------------------------------------------------------------------------
# host-side block allocator (the scheduler's job, emulated)
# --------------------------------------------------------------------------
class BlockAllocator:
    """Hands out physical block ids from a shuffled free list.

    A request gets ``ceil(tokens / block_size)`` blocks, taken from the head of
    the free list, and ``allocate`` returns None when the pool is short (the
    caller would preempt). Blocks carry a reference count so a prefix can be
    shared by several block tables and released only when the last user frees
    it.
    """

    def __init__(self, num_blocks: int, order: np.ndarray):
        assert sorted(order.tolist()) == list(range(num_blocks))
        self.num_blocks = num_blocks
        self.free = [int(b) for b in order]
        self.ref = np.zeros(num_blocks, dtype=np.int64)

    def num_free(self) -> int:
        return len(self.free)

    def allocate(self, n: int) -> Optional[list]:
        if n > len(self.free):
            return None
        got, self.free = self.free[:n], self.free[n:]
        for b in got:
            assert self.ref[b] == 0, "a newly handed-out block must be unreferenced"
            self.ref[b] += 1
        return got

    def share(self, blocks) -> None:
        for b in blocks:
            assert self.ref[b] > 0
            self.ref[b] += 1

    def release(self, blocks) -> None:
        # reverse order: tail blocks go back first
        for b in reversed(list(blocks)):
            assert self.ref[b] > 0
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(int(b))


def slots_for_positions(table_row: np.ndarray, positions: np.ndarray, block_size: int) -> np.ndarray:
    """Slot ids the scheduler hands to the cache write for the given positions."""
    positions = np.asarray(positions, dtype=np.int64)
    return table_row[positions // block_size].astype(np.int64) * block_size + positions % block_size


# --------------------------------------------------------------------------
# containers
# --------------------------------------------------------------------------
@dataclass
class DecodeBatch:
    """One decode step over ``num_seqs`` sequences (plus the step's cache write)."""
    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    context_lens: np.ndarray          # int32 [S], includes the token written this step
    block_tables: np.ndarray          # int32 [S][MB], -1 padded
    q: np.ndarray                     # [S][Hq][D]
    k_pool: np.ndarray                # [NB][Hkv][bs][D]  (before the step's write)
    v_pool: np.ndarray
    slot_mapping: np.ndarray          # int64 [T]
    k_new: np.ndarray                 # [T][Hkv][D]
    v_new: np.ndarray
    seed: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.context_lens.size else 0


@dataclass
class PrefillBatch:
    """Query chunks of chunked prefill, each the last ``n_q`` positions of its context."""
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    scale: float
    cu_q_lens: np.ndarray             # int32 [chunks + 1]
    context_lens: np.ndarray          # int32 [chunks], includes the chunk
    block_tables: np.ndarray          # int32 [chunks][MB]
    q: np.ndarray                     # [sum n_q][Hq][D]

    @property
    def num_chunks(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_q_len(self) -> int:
        return int(np.diff(self.cu_q_lens).max()) if self.num_chunks else 0

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_chunks else 0


# --------------------------------------------------------------------------
# generic builder
# --------------------------------------------------------------------------
def _fill_history(rng, pool_k, pool_v, table_row, n_hist, block_size, dtype, hkv, d,
                  slab_k=None, slab_v=None):
    """Write positions [0, n_hist) of one sequence, as earlier steps would have (and,
    when slabs [L][Hkv][D] are given, the same values at the same positions there)."""
    if n_hist <= 0:
        return
    # bounded chunks keep peak host memory modest for 200K-token contexts
    step = 1 << 15
    for p0 in range(0, n_hist, step):
        p1 = min(n_hist, p0 + step)
        pos = np.arange(p0, p1, dtype=np.int64)
        pb = table_row[pos // block_size]
        off = pos % block_size
        kv = rng.standard_normal((2, p1 - p0, hkv, d), dtype=np.float32)
        pool_k[pb, :, off, :] = _encode(kv[0], dtype)
        pool_v[pb, :, off, :] = _encode(kv[1], dtype)
        if slab_k is not None:
            slab_k[p0:p1] = _encode(kv[0], dtype)
            slab_v[p0:p1] = _encode(kv[1], dtype)


def build_decode_batch(*, name, dtype, context_lens, num_q_heads, num_kv_heads, head_dim,
                       block_size, seed, pool_factor=1.25, poison=True, fixed_tables=None,
                       num_blocks=None, scale=None, rng=None, contiguous=False) -> DecodeBatch:
    """Decode step: history K/V in the pool, one new token per sequence to write.

    contiguous=True also keeps the same values in the unpaged layout: extra["k_cache"],
    extra["v_cache"] [S][L][Hkv][D] with L the longest context rounded up to 64, holding
    each sequence's history and its new token at position ctx - 1 (the state after the
    step's write); positions past a context hold the fill value."""
    rng = rng if rng is not None else np.random.Generator(np.random.PCG64(seed))
    ctx = np.asarray(context_lens, dtype=np.int64)
    S = int(ctx.shape[0])
    hq, hkv, d, bs = num_q_heads, num_kv_heads, head_dim, block_size
    need = [cdiv(int(c), bs) for c in ctx]
    mb = max(1, max(need) if need else 1)
    if num_blocks is None:
        num_blocks = max(1, math.ceil(pool_factor * sum(need)))
    tables = np.full((S, mb), -1, dtype=np.int32)
    if fixed_tables is not None:
        for s, row in enumerate(fixed_tables):
            tables[s, :len(row)] = row
    else:
        alloc = BlockAllocator(num_blocks, rng.permutation(num_blocks))
        for s in range(S):
            got = alloc.allocate(need[s])
            assert got is not None, "pool too small"
            tables[s, :need[s]] = got
    st = _storage(dtype)
    q = _encode(rng.standard_normal((S, hq, d), dtype=np.float32), dtype)
    fill = _fill_value(dtype, poison)
    k_pool = np.full((num_blocks, hkv, bs, d), fill, dtype=st)
    v_pool = np.full((num_blocks, hkv, bs, d), fill, dtype=st)
    extra = {}
    if contiguous:
        L = max(64, cdiv(int(ctx.max()) if S else 1, 64) * 64)
        extra["k_cache"] = np.full((S, L, hkv, d), fill, dtype=st)
        extra["v_cache"] = np.full((S, L, hkv, d), fill, dtype=st)
    for s in range(S):
        _fill_history(rng, k_pool, v_pool, tables[s], int(ctx[s]) - 1, bs, dtype, hkv, d,
                      extra["k_cache"][s] if contiguous else None,
                      extra["v_cache"][s] if contiguous else None)
    new = rng.standard_normal((2, S, hkv, d), dtype=np.float32)
    if contiguous:
        for s in range(S):
            if ctx[s] > 0:
                extra["k_cache"][s, int(ctx[s]) - 1] = _encode(new[0, s], dtype)
                extra["v_cache"][s, int(ctx[s]) - 1] = _encode(new[1, s], dtype)
    slots = np.array([slots_for_positions(tables[s], [int(ctx[s]) - 1], bs)[0] if ctx[s] > 0 else -1
                      for s in range(S)], dtype=np.int64)
    return DecodeBatch(
        name=name, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs,
        num_blocks=num_blocks, scale=float(scale if scale is not None else 1.0 / math.sqrt(d)),
        context_lens=ctx.astype(np.int32), block_tables=tables, q=q, k_pool=k_pool, v_pool=v_pool,
        slot_mapping=slots, k_new=_encode(new[0], dtype), v_new=_encode(new[1], dtype), seed=seed,
        extra=extra)


# --------------------------------------------------------------------------
# the five named workloads
# --------------------------------------------------------------------------
SEED_BASE = 79000


def tiny(poison=True) -> DecodeBatch:
    """fp32; 3 sequences of 9, 5 and 16 tokens; block_size 4; 4 q = 4 kv heads; D 64;
    a pool of 32 blocks.  Sequence 0 is the guide's worked example: 9 tokens on
    physical blocks #7, #2, #5 (4/4, 4/4, 1/4 filled); the other two draw distinct
    ids from the remaining 29."""
    seed = SEED_BASE + 1
    rng = np.random.Generator(np.random.PCG64(seed))
    ctx = [9, 5, 16]
    rest = np.array([b for b in range(32) if b not in (7, 2, 5)])
    picks = rng.permutation(rest)[:2 + 4]
    tables = [[7, 2, 5], picks[:2].tolist(), picks[2:6].tolist()]
    return build_decode_batch(name="tiny_fp32_bs4", dtype=F32, context_lens=ctx, num_q_heads=4,
                              num_kv_heads=4, head_dim=64, block_size=4, seed=seed, poison=poison,
                              fixed_tables=tables, num_blocks=32, scale=1.0 / 8.0, rng=rng)


def gqa(poison=True, seed=None, num_seqs=64, block_size=16, contiguous=False) -> DecodeBatch:
    """bf16 Llama-style GQA decode: 64 sequences, ctx ~ U[128, 4096], 32 q / 8 kv heads,
    D 128, block_size 16, shuffled blocks from a pool of 1.25x the blocks needed."""
    seed = SEED_BASE + 2 if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    ctx = rng.integers(128, 4096, size=num_seqs, endpoint=True)
    return build_decode_batch(name="gqa_decode_bf16", dtype=BF16, context_lens=ctx, num_q_heads=32,
                              num_kv_heads=8, head_dim=128, block_size=block_size, seed=seed,
                              poison=poison, rng=rng, contiguous=contiguous)


def long_context(poison=True, seed=None, num_seqs=8, ctx_range=(32768, 200000), block_size=16,
                 contiguous=False) -> DecodeBatch:
    """bf16 long-context decode shaped like one TP=2 shard of the vAttention page's Yi-34B
    example: 8 sequences, ctx ~ U[32768, 200000], 28 q / 4 kv heads, D 128, block_size 16."""
    seed = SEED_BASE + 3 if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    ctx = rng.integers(ctx_range[0], ctx_range[1], size=num_seqs, endpoint=True)
    return build_decode_batch(name="long_decode_bf16", dtype=BF16, context_lens=ctx, num_q_heads=28,
                              num_kv_heads=4, head_dim=128, block_size=block_size, seed=seed,
                              poison=poison, rng=rng, contiguous=contiguous)


@dataclass
class PrefixCowBatch:
    """Prefix sharing plus copy-on-write of the last shared block."""
    batch: DecodeBatch                # tables already re-pointed to the private copies
    shared_tables: np.ndarray         # tables before the copy (every row on the shared blocks)
    block_mapping: np.ndarray         # int64 [n][2] (src, dst)
    prefix_blocks: np.ndarray         # the shared physical ids


def prefix_cow(poison=True, seed=None, num_seqs=256, prefix_tokens=2048,
               suffix_range=(64, 512)) -> PrefixCowBatch:
    """bf16: 256 sequences whose tables all start with the same 128 physical blocks
    (a 2048-token prefix at block_size 16) followed by private suffixes of U[64, 512]
    tokens; 32 q / 8 kv heads, D 128.  Before decode, every sequence gets a private
    copy of its last shared block (copy-on-write) and its table is re-pointed to it;
    then one token per sequence is written and decoded."""
    seed = SEED_BASE + 4 if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    bs, hq, hkv, d = 16, 32, 8, 128
    n_prefix = cdiv(prefix_tokens, bs)
    suffix = rng.integers(suffix_range[0], suffix_range[1], size=num_seqs, endpoint=True)
    ctx = prefix_tokens + suffix
    need_tot = [cdiv(int(c), bs) for c in ctx]
    unique = n_prefix + num_seqs + sum(n - n_prefix for n in need_tot)
    num_blocks = math.ceil(1.25 * unique)
    alloc = BlockAllocator(num_blocks, rng.permutation(num_blocks))
    prefix = np.array(alloc.allocate(n_prefix), dtype=np.int32)
    mb = max(need_tot)
    shared = np.full((num_seqs, mb), -1, dtype=np.int32)
    private = np.full((num_seqs, mb), -1, dtype=np.int32)
    mapping = np.zeros((num_seqs, 2), dtype=np.int64)
    for s in range(num_seqs):
        alloc.share(prefix)
        tail = alloc.allocate(need_tot[s] - n_prefix)
        cow = alloc.allocate(1)
        shared[s, :n_prefix] = prefix
        shared[s, n_prefix:need_tot[s]] = tail
        private[s] = shared[s]
        private[s, n_prefix - 1] = cow[0]
        mapping[s] = (prefix[-1], cow[0])
    st = _storage(BF16)
    q = _encode(rng.standard_normal((num_seqs, hq, d), dtype=np.float32), BF16)
    fill = _fill_value(BF16, poison)
    k_pool = np.full((num_blocks, hkv, bs, d), fill, dtype=st)
    v_pool = np.full((num_blocks, hkv, bs, d), fill, dtype=st)
    # shared prefix written once
    _fill_history(rng, k_pool, v_pool, shared[0], prefix_tokens, bs, BF16, hkv, d)
    for s in range(num_seqs):
        # suffix history (positions prefix_tokens .. ctx-2), logical order
        n_hist = int(ctx[s]) - 1
        p0 = prefix_tokens
        if n_hist > p0:
            pos = np.arange(p0, n_hist, dtype=np.int64)
            pb = shared[s][pos // bs]
            off = pos % bs
            kv = rng.standard_normal((2, pos.size, hkv, d), dtype=np.float32)
            k_pool[pb, :, off, :] = _encode(kv[0], BF16)
            v_pool[pb, :, off, :] = _encode(kv[1], BF16)
    new = rng.standard_normal((2, num_seqs, hkv, d), dtype=np.float32)
    slots = np.array([slots_for_positions(private[s], [int(ctx[s]) - 1], bs)[0]
                      for s in range(num_seqs)], dtype=np.int64)
    batch = DecodeBatch(name="prefix_cow_bf16", dtype=BF16, num_q_heads=hq, num_kv_heads=hkv,
                        head_dim=d, block_size=bs, num_blocks=num_blocks, scale=1.0 / math.sqrt(d),
                        context_lens=ctx.astype(np.int32), block_tables=private, q=q,
                        k_pool=k_pool, v_pool=v_pool, slot_mapping=slots,
                        k_new=_encode(new[0], BF16), v_new=_encode(new[1], BF16), seed=seed)
    return PrefixCowBatch(batch=batch, shared_tables=shared, block_mapping=mapping,
                          prefix_blocks=prefix)


@dataclass
class MixedBatch:
    """Chunked prefill and decode sharing one pool."""
    decode: DecodeBatch               # pool, decode tables, and every token written this step
    prefill: PrefillBatch             # chunk queries; their K/V are among decode.k_new rows
    num_decode_tokens: int            # the first rows of slot_mapping belong to decode


def mixed(poison=True, seed=None, num_chunks=4, chunk_len=512, chunk_ctx=(2048, 8192),
          num_decode=128, decode_ctx=(256, 8192)) -> MixedBatch:
    """bf16: 4 prefill chunks of 512 queries (causal) over paged contexts of U[2048, 8192]
    tokens that include the chunk, plus 128 decode sequences of U[256, 8192] tokens;
    32 q / 8 kv heads, D 128, block_size 16, shuffled blocks, one pool of 1.25x.
    The step writes the chunk tokens' K/V and each decode sequence's new token."""
    seed = SEED_BASE + 5 if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    bs, hq, hkv, d = 16, 32, 8, 128
    cctx = rng.integers(chunk_ctx[0], chunk_ctx[1], size=num_chunks, endpoint=True)
    dctx = rng.integers(decode_ctx[0], decode_ctx[1], size=num_decode, endpoint=True)
    need_c = [cdiv(int(c), bs) for c in cctx]
    need_d = [cdiv(int(c), bs) for c in dctx]
    num_blocks = math.ceil(1.25 * (sum(need_c) + sum(need_d)))
    alloc = BlockAllocator(num_blocks, rng.permutation(num_blocks))
    mb = max(need_c + need_d)
    ctab = np.full((num_chunks, mb), -1, dtype=np.int32)
    dtab = np.full((num_decode, mb), -1, dtype=np.int32)
    for c in range(num_chunks):
        ctab[c, :need_c[c]] = alloc.allocate(need_c[c])
    for s in range(num_decode):
        dtab[s, :need_d[s]] = alloc.allocate(need_d[s])
    st = _storage(BF16)
    qd = _encode(rng.standard_normal((num_decode, hq, d), dtype=np.float32), BF16)
    qc = _encode(rng.standard_normal((num_chunks * chunk_len, hq, d), dtype=np.float32), BF16)
    fill = _fill_value(BF16, poison)
    k_pool = np.full((num_blocks, hkv, bs, d), fill, dtype=st)
    v_pool = np.full((num_blocks, hkv, bs, d), fill, dtype=st)
    for c in range(num_chunks):
        _fill_history(rng, k_pool, v_pool, ctab[c], int(cctx[c]) - chunk_len, bs, BF16, hkv, d)
    for s in range(num_decode):
        _fill_history(rng, k_pool, v_pool, dtab[s], int(dctx[s]) - 1, bs, BF16, hkv, d)
    newd = rng.standard_normal((2, num_decode, hkv, d), dtype=np.float32)
    newc = rng.standard_normal((2, num_chunks * chunk_len, hkv, d), dtype=np.float32)
    slots_d = np.array([slots_for_positions(dtab[s], [int(dctx[s]) - 1], bs)[0]
                        for s in range(num_decode)], dtype=np.int64)
    slots_c = np.concatenate([slots_for_positions(ctab[c], np.arange(int(cctx[c]) - chunk_len,
                                                                     int(cctx[c])), bs)
                              for c in range(num_chunks)]).astype(np.int64)
    k_new = np.concatenate([_encode(newd[0], BF16), _encode(newc[0], BF16)])
    v_new = np.concatenate([_encode(newd[1], BF16), _encode(newc[1], BF16)])
    dec = DecodeBatch(name="mixed_bf16", dtype=BF16, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                      block_size=bs, num_blocks=num_blocks, scale=1.0 / math.sqrt(d),
                      context_lens=dctx.astype(np.int32), block_tables=dtab, q=qd,
                      k_pool=k_pool, v_pool=v_pool,
                      slot_mapping=np.concatenate([slots_d, slots_c]),
                      k_new=k_new, v_new=v_new, seed=seed)
    pre = PrefillBatch(dtype=BF16, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs,
                       scale=1.0 / math.sqrt(d),
                       cu_q_lens=np.arange(num_chunks + 1, dtype=np.int32) * chunk_len,
                       context_lens=cctx.astype(np.int32), block_tables=ctab, q=qc)
    return MixedBatch(decode=dec, prefill=pre, num_decode_tokens=num_decode)


@dataclass
class PrefixGroups:
    """Decode batch whose sequences come in groups sharing the physical blocks of a prefix."""
    batch: DecodeBatch
    group_first_seq: np.ndarray       # int32 [G]
    group_num_seqs: np.ndarray        # int32 [G]
    group_prefix_lens: np.ndarray     # int32 [G], whole blocks
    seq_prefix_lens: np.ndarray       # int32 [S], 0 outside every group


def prefix_groups(seed, layout, suffix_range=(1, 200), num_q_heads=8, num_kv_heads=2,
                  head_dim=128, block_size=16, poison=True) -> PrefixGroups:
    """bf16 decode batch laid out by ``layout``: a list of (members, prefix_blocks);
    prefix_blocks 0 makes one unshared sequence per member.  Members of a group share
    their first prefix_blocks physical blocks (written once) and own a suffix of
    U[suffix_range] tokens, the step's new token included."""
    rng = np.random.Generator(np.random.PCG64(seed))
    hq, hkv, d, bs = num_q_heads, num_kv_heads, head_dim, block_size
    seqs = []                                  # (group index or -1, prefix tokens)
    for gi, (members, pblocks) in enumerate(layout):
        seqs += [(gi if pblocks else -1, pblocks * bs)] * members
    S = len(seqs)
    suffix = rng.integers(suffix_range[0], suffix_range[1], size=S, endpoint=True)
    ctx = np.array([p + int(x) for (_, p), x in zip(seqs, suffix)], dtype=np.int64)
    need = [cdiv(int(c), bs) for c in ctx]
    shared_blocks = sum(p for m, p in layout if p)
    num_blocks = math.ceil(1.25 * (shared_blocks + sum(n - p // bs for n, (_, p) in zip(need, seqs))))
    alloc = BlockAllocator(num_blocks, rng.permutation(num_blocks))
    mb = max(need)
    tab = np.full((S, mb), -1, dtype=np.int32)
    st = _storage(BF16)
    fill = _fill_value(BF16, poison)
    k_pool = np.full((num_blocks, hkv, bs, d), fill, dtype=st)
    v_pool = np.full((num_blocks, hkv, bs, d), fill, dtype=st)
    q = _encode(rng.standard_normal((S, hq, d), dtype=np.float32), BF16)
    gfirst, gnum, gpre = [], [], []
    s = 0
    for gi, (members, pblocks) in enumerate(layout):
        if pblocks:
            prefix = np.array(alloc.allocate(pblocks), dtype=np.int32)
            for j in range(1, members):
                alloc.share(prefix)
            _fill_history(rng, k_pool, v_pool, prefix, pblocks * bs, bs, BF16, hkv, d)
            gfirst.append(s)
            gnum.append(members)
            gpre.append(pblocks * bs)
        for j in range(members):
            p = pblocks * bs
            if pblocks:
                tab[s, :pblocks] = prefix
            tail = alloc.allocate(need[s] - pblocks)
            tab[s, pblocks:need[s]] = tail
            # the member's own history: positions p .. ctx-2
            n_hist = int(ctx[s]) - 1
            if n_hist > p:
                pos = np.arange(p, n_hist, dtype=np.int64)
                kv = rng.standard_normal((2, pos.size, hkv, d), dtype=np.float32)
                k_pool[tab[s][pos // bs], :, pos % bs, :] = _encode(kv[0], BF16)
                v_pool[tab[s][pos // bs], :, pos % bs, :] = _encode(kv[1], BF16)
            s += 1
    new = rng.standard_normal((2, S, hkv, d), dtype=np.float32)
    slots = np.array([slots_for_positions(tab[i], [int(ctx[i]) - 1], bs)[0] for i in range(S)],
                     dtype=np.int64)
    batch = DecodeBatch(name="prefix_groups_bf16", dtype=BF16, num_q_heads=hq, num_kv_heads=hkv,
                        head_dim=d, block_size=bs, num_blocks=num_blocks,
                        scale=1.0 / math.sqrt(d), context_lens=ctx.astype(np.int32),
                        block_tables=tab, q=q, k_pool=k_pool, v_pool=v_pool, slot_mapping=slots,
                        k_new=_encode(new[0], BF16), v_new=_encode(new[1], BF16), seed=seed)
    return PrefixGroups(batch=batch, group_first_seq=np.array(gfirst, dtype=np.int32),
                        group_num_seqs=np.array(gnum, dtype=np.int32),
                        group_prefix_lens=np.array(gpre, dtype=np.int32),
                        seq_prefix_lens=np.array([p if g >= 0 else 0 for g, p in seqs],
                                                 dtype=np.int32))


@dataclass
class SpecDecodeBatch:
    """Multi-token decode (speculative verification): every sequence writes its k + 1
    newest tokens (the last accepted one and k draft tokens) and attends with k + 1
    queries at the last k + 1 positions of its context, causally."""
    prefill: PrefillBatch             # queries [S (k + 1)][Hq][D]; cu_q_lens = (k + 1) * arange
    k_pool: np.ndarray
    v_pool: np.ndarray
    slot_mapping: np.ndarray          # int64 [S (k + 1)]: slots of positions ctx-k-1 .. ctx-1
    k_new: np.ndarray                 # [S (k + 1)][Hkv][D]
    v_new: np.ndarray
    num_blocks: int
    draft: int                        # k


def spec_decode(poison=True, seed=None, num_seqs=64, draft=3, ctx_range=(128, 4096),
                num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16) -> SpecDecodeBatch:
    """bf16 speculative-decode verification step shaped like the GQA decode batch:
    64 sequences with contexts U[128, 4096] that include k = 3 draft tokens (4 queries
    per sequence), 32 q / 8 kv heads, D 128, block_size 16, shuffled blocks from a pool
    of 1.25x the blocks needed.  Blocks are reserved for the whole context, draft
    slots included, before the step writes the k + 1 new tokens."""
    seed = SEED_BASE + 6 if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    hq, hkv, d, bs, nq = num_q_heads, num_kv_heads, head_dim, block_size, draft + 1
    ctx = rng.integers(max(ctx_range[0], nq), ctx_range[1], size=num_seqs, endpoint=True)
    need = [cdiv(int(c), bs) for c in ctx]
    num_blocks = math.ceil(1.25 * sum(need))
    alloc = BlockAllocator(num_blocks, rng.permutation(num_blocks))
    mb = max(need)
    tab = np.full((num_seqs, mb), -1, dtype=np.int32)
    for s in range(num_seqs):
        tab[s, :need[s]] = alloc.allocate(need[s])
    st = _storage(BF16)
    q = _encode(rng.standard_normal((num_seqs * nq, hq, d), dtype=np.float32), BF16)
    fill = _fill_value(BF16, poison)
    k_pool = np.full((num_blocks, hkv, bs, d), fill, dtype=st)
    v_pool = np.full((num_blocks, hkv, bs, d), fill, dtype=st)
    for s in range(num_seqs):
        _fill_history(rng, k_pool, v_pool, tab[s], int(ctx[s]) - nq, bs, BF16, hkv, d)
    new = rng.standard_normal((2, num_seqs * nq, hkv, d), dtype=np.float32)
    slots = np.concatenate([slots_for_positions(tab[s], np.arange(int(ctx[s]) - nq, int(ctx[s])), bs)
                            for s in range(num_seqs)]).astype(np.int64)
    pre = PrefillBatch(dtype=BF16, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs,
                       scale=1.0 / math.sqrt(d),
                       cu_q_lens=(np.arange(num_seqs + 1) * nq).astype(np.int32),
                       context_lens=ctx.astype(np.int32), block_tables=tab, q=q)
    return SpecDecodeBatch(prefill=pre, k_pool=k_pool, v_pool=v_pool, slot_mapping=slots,
                           k_new=_encode(new[0], BF16), v_new=_encode(new[1], BF16),
                           num_blocks=num_blocks, draft=draft)


def prefill_only(*, seed, dtype=BF16, chunk_lens, contexts, num_q_heads, num_kv_heads, head_dim,
                 block_size, poison=True, pool_factor=1.25):
    """Small chunked-prefill case for tests: every context fully written (chunk included)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ctx = np.asarray(contexts, dtype=np.int64)
    nq = np.asarray(chunk_lens, dtype=np.int64)
    assert np.all(nq <= ctx)
    C = ctx.shape[0]
    bs = block_size
    need = [cdiv(int(c), bs) for c in ctx]
    num_blocks = max(1, math.ceil(pool_factor * sum(need)))
    alloc = BlockAllocator(num_blocks, rng.permutation(num_blocks))
    mb = max(1, max(need))
    tab = np.full((C, mb), -1, dtype=np.int32)
    for c in range(C):
        tab[c, :need[c]] = alloc.allocate(need[c])
    st = _storage(dtype)
    q = _encode(rng.standard_normal((int(nq.sum()), num_q_heads, head_dim), dtype=np.float32), dtype)
    fill = _fill_value(dtype, poison)
    k_pool = np.full((num_blocks, num_kv_heads, bs, head_dim), fill, dtype=st)
    v_pool = np.full((num_blocks, num_kv_heads, bs, head_dim), fill, dtype=st)
    for c in range(C):
        _fill_history(rng, k_pool, v_pool, tab[c], int(ctx[c]), bs, dtype, num_kv_heads, head_dim)
    cu = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    pre = PrefillBatch(dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                       head_dim=head_dim, block_size=bs, scale=1.0 / math.sqrt(head_dim),
                       cu_q_lens=cu, context_lens=ctx.astype(np.int32), block_tables=tab, q=q)
    return pre, k_pool, v_pool, num_blocks


WORKLOADS = {
    "tiny": tiny,
    "gqa": gqa,
    "long": long_context,
    "prefix_cow": prefix_cow,
    "mixed": mixed,
    "spec": spec_decode,
}
