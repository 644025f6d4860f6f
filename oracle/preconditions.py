"""Plain model of the device-content preconditions of the paged KV-cache calls.
TEST INFRASTRUCTURE ONLY.

The kernels trust what lies in device memory; these are the rules that trust rests on:

  * "2.1 PagedAttention" (sections 3 and 5): token t of a sequence lives in physical
    block block_tables[s][t // block_size], so every table entry a context reaches
    must name a block of the pool, and a context cannot reach past the table's
    max_blocks_per_seq * block_size tokens;
  * the same chapter (section 3): a write puts token i at slot slot_mapping[i] =
    block * block_size + offset, so a slot must lie inside the pool, and two tokens of
    one write cannot share a slot (negative slots are padding, skipped);
  * the same chapter (section 6): copy-on-write copies whole blocks, src -> dst, all
    at once, so every id must name a block, no block may be written twice, and no
    block may be both written and read in one call;
  * "Inside vLLM, part 2" (chunked prefill): a chunk's queries are the last positions
    of its context, so a chunk cannot hold more queries than its context, and the
    chunks' queries are packed one after another from row 0.

validate() counts the violations of each rule the way the device check does: each
offending table entry, sequence, token or pair once.
"""
from __future__ import annotations

import numpy as np


def bad_table_entries(num_blocks, block_size, block_tables, context_lens) -> int:
    """Entries j < min(ceil(ctx / block_size), max_blocks_per_seq) outside [0, num_blocks)."""
    tab = np.asarray(block_tables)
    mb = tab.shape[1] if tab.ndim == 2 else 0
    bad = 0
    for s, c in enumerate(np.asarray(context_lens)):
        reach = min(-(-max(int(c), 0) // block_size), mb)
        for j in range(reach):
            if not 0 <= int(tab[s, j]) < num_blocks:
                bad += 1
    return bad


def bad_context_lens(block_size, max_blocks_per_seq, context_lens) -> int:
    """Sequences whose context is negative or longer than the table can hold."""
    cap = max_blocks_per_seq * block_size
    return sum(1 for c in np.asarray(context_lens) if not 0 <= int(c) <= cap)


def bad_slots(num_blocks, block_size, slot_mapping) -> int:
    """Tokens whose slot lies past the pool, or repeats the slot of an earlier token
    (negative slots are padding and never counted)."""
    seen = set()
    bad = 0
    for x in np.asarray(slot_mapping):
        x = int(x)
        if x < 0:
            continue
        if x >= num_blocks * block_size or x in seen:
            bad += 1
        seen.add(x)
    return bad


def bad_copy_pairs(num_blocks, block_mapping) -> int:
    """Pairs with an id outside the pool, a destination written by an earlier pair, or
    a destination that some pair reads."""
    m = np.asarray(block_mapping).reshape(-1, 2)
    srcs = {int(x) for x in m[:, 0]}
    bad = 0
    dsts = set()
    for src, dst in m:
        src, dst = int(src), int(dst)
        if not (0 <= src < num_blocks and 0 <= dst < num_blocks) or dst in dsts or dst in srcs:
            bad += 1
        dsts.add(dst)
    return bad


def validate(num_blocks, block_size, block_tables, context_lens, slot_mapping=(),
             block_mapping=()) -> np.ndarray:
    """[bad table entries, bad context lengths, bad slots, bad copy pairs] (int32)."""
    tab = np.asarray(block_tables)
    mb = tab.shape[1] if tab.ndim == 2 else 0
    return np.array([bad_table_entries(num_blocks, block_size, tab, context_lens),
                     bad_context_lens(block_size, mb, context_lens),
                     bad_slots(num_blocks, block_size, slot_mapping),
                     bad_copy_pairs(num_blocks, block_mapping)], dtype=np.int32)


def bad_chunks(cu_q_lens, context_lens, total_q=-1) -> int:
    """Chunks whose query range runs backwards, whose context is negative or shorter than
    its queries, or whose queries end past total_q rows (total_q >= 0); chunk 0 also
    when the packing does not start at row 0."""
    cu = [int(x) for x in np.asarray(cu_q_lens)]
    bad = 0
    for c, ctx in enumerate(np.asarray(context_lens)):
        ctx = int(ctx)
        q0, q1 = cu[c], cu[c + 1]
        if (c == 0 and q0 != 0) or q1 < q0 or ctx < 0 or q1 - q0 > ctx or \
                (total_q >= 0 and q1 > total_q):
            bad += 1
    return bad
