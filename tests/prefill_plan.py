"""Host replica of the balanced key split of the chunked prefill (test support).

Work items are the query tiles of QP = 128 // G positions of every (chunk, kv head),
in (chunk, kv head, query tile) order; query tile qt of a chunk with n_q queries and
context ctx reads ceil((ctx - n_q + min(n_q, (qt + 1) QP)) / 64) key tiles.  The
split applies when a workspace is given, the items fit in one round of W resident
workgroups, and the largest item exceeds 5/4 of an even share ceil(T / W).  Then
workgroup w takes tiles [w T / W, (w + 1) T / W) of the batch order (chunk, kv head,
query tile, tile), with W replaced by min(W, T) so that no range is empty; an item
inside one range is finished in place, a cut one leaves
a piece in slot 2w + 1 (the piece that starts the item) or 2w (a piece that
continues it), and the merge takes the first covering workgroup's slot 2w + 1 and
slot 2w of every later one."""
from __future__ import annotations


def chunk_items(cu_q_lens, context_lens, qp, num_q_tiles, max_ctx):
    """Per chunk: the tile counts of its query tiles (empty for a malformed chunk)."""
    out = []
    for c in range(len(context_lens)):
        nq = int(cu_q_lens[c + 1]) - int(cu_q_lens[c])
        ctx = max(0, min(int(context_lens[c]), max_ctx))
        if nq <= 0 or nq > ctx:
            out.append([])
            continue
        nqt = min(-(-nq // qp), num_q_tiles)
        out.append([-(-(ctx - nq + min(nq, (qt + 1) * qp)) // 64) for qt in range(nqt)])
    return out


def plan(cu_q_lens, context_lens, group, hkv, W, max_q_len, max_ctx):
    """(split?, T, per-chunk item tile lists)."""
    qp = 128 // group
    nqt = -(-max_q_len // qp)
    items = chunk_items(cu_q_lens, context_lens, qp, nqt, max_ctx)
    T = hkv * sum(sum(t) for t in items)
    n_items = hkv * sum(len(t) for t in items)
    maxn = max([max(t) for t in items if t] or [0])
    host_ok = len(context_lens) * hkv * nqt <= W
    split = host_ok and T > 0 and n_items <= W and 4 * maxn > 5 * (-(-T // W))
    return split, T, items


def begin(T, W, w):
    return w * T // W


def owner(T, W, u):
    return ((u + 1) * W - 1) // T


def ranges(T, W):
    """Ranges of the split: one per workgroup, never more than tiles."""
    return min(W, T)


def walk(T, W, items, hkv):
    """Every workgroup's pieces: (w, (c, h, qt), k0, k1, slot or -1); W ranges."""
    order = [(c, h, qt, n) for c, t in enumerate(items) for h in range(hkv)
             for qt, n in enumerate(t)]
    starts, u = [], 0
    for it in order:
        starts.append(u)
        u += it[3]
    pieces = []
    for w in range(W):
        b, e = begin(T, W, w), begin(T, W, w + 1)
        for (c, h, qt, n), s in zip(order, starts):
            lo, hi = max(b, s), min(e, s + n)
            if lo >= hi:
                continue
            k0, k1 = lo - s, hi - s
            slot = -1 if (k0 == 0 and k1 == n) else 2 * w + (1 if k0 == 0 else 0)
            pieces.append((w, (c, h, qt), k0, k1, slot))
    return order, starts, pieces


def merge_slots(T, W, start, n):
    """Slots the merge reads for an item starting at tile `start` with n tiles (None:
    finished in place); W ranges."""
    w0, w1 = owner(T, W, start), owner(T, W, start + n - 1)
    if w0 == w1:
        return None
    return [2 * w0 + 1] + [2 * w for w in range(w0 + 1, w1 + 1)]
