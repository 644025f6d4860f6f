"""numpy float64 oracle for paged KV-cache attention.  TEST INFRASTRUCTURE ONLY.

Paged attention reaches exactly the result of ordinary softmax attention over
each sequence's logically contiguous history: paging only changes where the
bytes live ("2.1 PagedAttention", section 5: scattered physical blocks are
read as one logically contiguous context).  So this oracle reads every token
through the block table into a contiguous float64 array and runs the plain
definition of attention on it.

Storage conventions (readings of the pages, shared with the workload builder
only by agreement, never by code):
  * K and V pools are ``[num_blocks][num_kv_heads][block_size][head_dim]``;
  * bf16 values arrive as uint16 bit patterns, fp32 values as float32;
  * query head ``hq`` reads KV head ``hq // (Hq / Hkv)``;
  * a context length counts every token visible to the step's queries; a
    decode query is the last position, a prefill chunk the last ``n_q``.
"""
from __future__ import annotations

import numpy as np

BF16 = "bf16"
F32 = "f32"


# --------------------------------------------------------------------------
# element widening
# --------------------------------------------------------------------------
def widen(a, dtype: str) -> np.ndarray:
    """Exact float64 value of stored elements.

    A bfloat16 number is the upper half of a float32, so its bits shifted left
    by 16 are that float32, which float64 holds exactly."""
    if dtype == BF16:
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == F32:
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------
# block-table translation  ("2.1 PagedAttention", sections 3 and 5)
# --------------------------------------------------------------------------
def translate(table_row, t: int, block_size: int):
    """Logical position t of a request -> (logical block, physical block, offset).

    Section 3 of the chapter: a request's tokens fill logical blocks of
    block_size tokens in order, so token t lives in logical block
    t // block_size; the block table maps that logical block to a physical
    block number; section 5 names the slot inside it the physical block
    offset, t mod block_size.  A position whose logical block has no table
    entry has not been allocated yet (section 3: the next block is requested
    only when the last one is full) and raises IndexError."""
    if t < 0:
        raise IndexError("negative position")
    lb = t // block_size
    off = t - lb * block_size
    if lb >= len(table_row) or int(table_row[lb]) < 0:
        raise IndexError(f"position {t} needs logical block {lb}, which has no physical block")
    return lb, int(table_row[lb]), off


def slot_of(table_row, t: int, block_size: int) -> int:
    """Flat slot id of position t: physical block * block_size + offset."""
    _, pb, off = translate(table_row, t, block_size)
    return pb * block_size + off


def blocks_needed(n_tokens: int, block_size: int) -> int:
    """Blocks a request of n tokens holds under on-demand paging: ceil(n / block_size)."""
    return -(-int(n_tokens) // block_size)


def tail_waste(n_tokens: int, block_size: int) -> int:
    """Unused slots in the last block ("2.1 PagedAttention", section 4: under one block)."""
    return blocks_needed(n_tokens, block_size) * block_size - int(n_tokens)


def gather_kv(pool, table_row, n: int, block_size: int, kv_head: int, dtype: str) -> np.ndarray:
    """[n, head_dim] float64 K (or V) of the first n logical positions of one request
    for one KV head, each read at (physical block, kv head, offset) of the pool."""
    num_blocks = pool.shape[0]
    out = np.empty((n, pool.shape[-1]), dtype=np.float64)
    if n == 0:
        return out
    t = np.arange(n)
    lb = t // block_size
    off = t % block_size
    if lb[-1] >= len(table_row):
        raise IndexError("context longer than the block table")
    pb = np.asarray(table_row, dtype=np.int64)[lb]
    if np.any(pb < 0) or np.any(pb >= num_blocks):
        raise IndexError("block table entry outside the pool")
    out[:] = widen(pool[pb, kv_head, off, :], dtype)
    return out


def kv_head_of(hq: int, num_q_heads: int, num_kv_heads: int) -> int:
    """Grouped-query attention: consecutive groups of Hq/Hkv query heads share one KV head."""
    if num_q_heads % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    return hq // (num_q_heads // num_kv_heads)


# --------------------------------------------------------------------------
# attention over a contiguous history
# --------------------------------------------------------------------------
def attend(q, K, V, scale: float) -> np.ndarray:
    """softmax(scale * K q) V in float64 for one query vector.

    The result does not depend on which constant is subtracted before exp;
    the maximum is used so large scores cannot overflow.  An empty history
    gives a zero vector."""
    q = np.asarray(q, dtype=np.float64)
    n = K.shape[0]
    if n == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    s = scale * (K @ q)
    w = np.exp(s - s.max())
    return (w @ V) / w.sum()


def decode(q, k_pool, v_pool, block_tables, context_lens, scale: float, dtype: str,
           num_kv_heads: int, seqs=None, heads=None) -> np.ndarray:
    """Decode attention: every query head of sequence s attends to the sequence's
    context_lens[s] tokens, gathered through its block table row.

    Returns float64 [S][Hq][D] (rows outside ``seqs``/``heads`` stay NaN)."""
    S, Hq, D = q.shape
    out = np.full((S, Hq, D), np.nan)
    seqs = range(S) if seqs is None else seqs
    heads = range(Hq) if heads is None else heads
    for s in seqs:
        n = int(context_lens[s])
        cache = {}
        for hq in heads:
            h = kv_head_of(hq, Hq, num_kv_heads)
            if h not in cache:
                cache[h] = (gather_kv(k_pool, block_tables[s], n, k_pool.shape[2], h, dtype),
                            gather_kv(v_pool, block_tables[s], n, v_pool.shape[2], h, dtype))
            K, V = cache[h]
            out[s, hq] = attend(widen(q[s, hq], dtype), K, V, scale)
    return out


def decode_contiguous(q, k_cache, v_cache, context_lens, scale: float, dtype: str,
                      num_kv_heads: int, seqs=None, heads=None) -> np.ndarray:
    """Decode attention over K/V kept contiguous per request -- the layout of
    "vAttention 完全拆解" (section on its core abstraction: each request's KV cache
    is one virtually contiguous range, and the kernel indexes K[t, h, d] linearly;
    the comparison with PagedAttention keeps that index unchanged).  Token t of
    sequence s, kv head h is k_cache[s, t, h].  The attention itself is decode()'s:
    every query head of sequence s attends to its context_lens[s] tokens.

    Returns float64 [S][Hq][D] (rows outside ``seqs``/``heads`` stay NaN)."""
    S, Hq, D = q.shape
    out = np.full((S, Hq, D), np.nan)
    seqs = range(S) if seqs is None else seqs
    heads = range(Hq) if heads is None else heads
    for s in seqs:
        n = int(context_lens[s])
        for hq in heads:
            h = kv_head_of(hq, Hq, num_kv_heads)
            K = widen(k_cache[s, :n, h, :], dtype)
            V = widen(v_cache[s, :n, h, :], dtype)
            out[s, hq] = attend(widen(q[s, hq], dtype), K, V, scale)
    return out


def prefill_chunk(q, cu_q_lens, k_pool, v_pool, block_tables, context_lens, scale: float,
                  dtype: str, num_kv_heads: int, rows=None) -> np.ndarray:
    """Causal attention of a prefill chunk over its paged context.

    "Inside vLLM, part 2" (chunked prefill): a long prompt is processed a
    chunk of tokens at a time, and each chunk attends to everything computed
    before it plus itself.  Chunk c holds n_q = cu[c+1]-cu[c] queries, the last
    n_q positions of its context of context_lens[c] tokens; query i sits at
    position p = ctx - n_q + i and sees keys t <= p.

    ``rows`` optionally restricts the computation to (query row, q head) pairs.
    Returns float64 [sum n_q][Hq][D] (rows not computed stay NaN)."""
    Tq, Hq, D = q.shape
    out = np.full((Tq, Hq, D), np.nan)
    want = None if rows is None else set((int(r), int(h)) for r, h in rows)
    for c in range(len(context_lens)):
        q0, q1 = int(cu_q_lens[c]), int(cu_q_lens[c + 1])
        nq, n = q1 - q0, int(context_lens[c])
        if nq > n:
            raise ValueError("a chunk cannot be longer than its context")
        cache = {}
        for i in range(nq):
            pos = n - nq + i
            for hq in range(Hq):
                if want is not None and (q0 + i, hq) not in want:
                    continue
                h = kv_head_of(hq, Hq, num_kv_heads)
                if h not in cache:
                    cache[h] = (gather_kv(k_pool, block_tables[c], n, k_pool.shape[2], h, dtype),
                                gather_kv(v_pool, block_tables[c], n, v_pool.shape[2], h, dtype))
                K, V = cache[h]
                out[q0 + i, hq] = attend(widen(q[q0 + i, hq], dtype), K[:pos + 1], V[:pos + 1], scale)
    return out


# --------------------------------------------------------------------------
# split context: partial softmax states and their log-sum-exp merge
# --------------------------------------------------------------------------
def partition_partials(q, K, V, scale: float, bounds):
    """Softmax state of each token range [a, b): (max score m, sum of exp(s - m),
    unnormalised sum of exp(s - m) * v).  Empty ranges are skipped."""
    q = np.asarray(q, dtype=np.float64)
    parts = []
    for a, b in bounds:
        if b <= a:
            continue
        s = scale * (K[a:b] @ q)
        m = s.max()
        w = np.exp(s - m)
        parts.append((m, w.sum(), w @ V[a:b]))
    return parts


def lse_merge(parts) -> np.ndarray:
    """Combine partial states: with M the largest partial max, each part is weighted
    by exp(m_p - M); the output is sum_p w_p o_p / sum_p w_p l_p."""
    if not parts:
        raise ValueError("nothing to merge")
    M = max(m for m, _, _ in parts)
    num = sum(np.exp(m - M) * o for m, _, o in parts)
    den = sum(np.exp(m - M) * l for m, l, _ in parts)
    return num / den


# --------------------------------------------------------------------------
# cache writes and block copies (bit-pattern assignments)
# --------------------------------------------------------------------------
def _bits(a):
    a = np.asarray(a)
    return a.view(np.uint16) if a.dtype.itemsize == 2 else a.view(np.uint32)


def kv_write(pool, new, slot_mapping):
    """Write each new token's [Hkv][D] K (or V) into its slot.

    "2.1 PagedAttention", section 3: each new token fills the next free slot of
    its request's current block; the scheduler names that slot as
    physical block * block_size + offset.  Slot < 0 marks padding and writes
    nothing.  Bits are copied as they are, NaN payloads included."""
    out = np.array(pool, copy=True)
    ob, nb = _bits(out), _bits(new)
    bs = pool.shape[2]
    for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0:
            continue
        pb, off = int(slot) // bs, int(slot) % bs
        if pb >= pool.shape[0]:
            raise IndexError("slot outside the pool")
        ob[pb, :, off, :] = nb[i]
    return out


def copy_blocks(pool, block_mapping):
    """Copy-on-write block copies ("2.1 PagedAttention", section 6): for each (src, dst)
    pair the whole physical block (all KV heads, all slots) is duplicated.  All
    pairs read the pool as it was before the call."""
    out = np.array(pool, copy=True)
    m = np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2)
    if m.size == 0:
        return out
    ob, ib = _bits(out), _bits(np.asarray(pool))
    snap = ib[m[:, 0]].copy()
    ob[m[:, 1]] = snap
    return out


# --------------------------------------------------------------------------
# KV size model (vAttention page, opening section)
# --------------------------------------------------------------------------
def swap_blocks(dst_pool, src_pool, block_mapping):
    """Swapping ("2.1 PagedAttention", section 7: a preempted request's KV blocks are
    copied from GPU memory to CPU memory and copied back on resume): for each (src, dst)
    pair, block dst of the destination pool becomes a bit copy of block src of the source
    pool.  Returns the new destination pool; the source is unchanged."""
    out = np.array(dst_pool, copy=True)
    src = np.asarray(src_pool)
    for s, d in np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2):
        _bits(out[d])[...] = _bits(src[s])
    return out


def kv_size_bytes(layers: int, length: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """M_KV = 2 N L H D P: K and V for N layers, L tokens, H KV heads of D elements of
    P bytes each."""
    return 2 * layers * length * kv_heads * head_dim * elem_bytes
