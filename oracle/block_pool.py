"""Plain model of the host block manager.  TEST INFRASTRUCTURE ONLY.

Follows the block pool of "2.1 PagedAttention" (the walk-through of the V1
engine: section 9.2 on why the free blocks sit in a doubly linked queue, 9.3 on
reference counts and the order of release) and the prefix caching of "Inside
vLLM, part 2" (block hashes chained over the previous block's hash and the
block's tokens; a cached block keeps its hash until the free queue hands it out
again).  Copy-on-write follows "2.1 PagedAttention", section 6.

The free queue is a Python list (index 0 = head); every operation is the plain
list operation the pages describe, so the model can be checked by eye.
Readings where the pages leave a choice open:
  * the initial queue holds blocks 0..n-1 in ascending order;
  * free() applies the ids in the order given (a request passes its blocks tail
    first), so unhashed blocks freed together end up at the head in reverse of
    that order, hashed ones at the tail in that order;
  * cache_blocks() leaves a block that already has a hash, and a hash already
    held by another block, unchanged (first one wins);
  * cow() on a block whose count is 1 writes in place (no copy).
"""
from __future__ import annotations

FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3
MASK64 = (1 << 64) - 1


def fnv1a_64(data: bytes, h: int = FNV_OFFSET) -> int:
    """64-bit FNV-1a (Fowler/Noll/Vo): per byte, xor then multiply by the prime."""
    for byte in data:
        h ^= byte
        h = (h * FNV_PRIME) & MASK64
    return h


def block_hash(parent: int, tokens) -> int:
    """Hash of a full block chained over its parent's hash ("Inside vLLM, part 2",
    prefix caching: each full block's hash combines the previous block's hash and
    its tokens).  Bytes: the parent as 8 little-endian bytes, then each token id as
    4 little-endian bytes (two's complement)."""
    data = (parent & MASK64).to_bytes(8, "little")
    data += b"".join(int(t).to_bytes(4, "little", signed=True) for t in tokens)
    return fnv1a_64(data)


class BlockPoolModel:
    """Reference counts, free queue, hash index ("2.1 PagedAttention", 9.2-9.3)."""

    def __init__(self, num_blocks: int):
        assert num_blocks > 0
        self.ref = [0] * num_blocks
        self.queue = list(range(num_blocks))      # head first
        self.hash = [None] * num_blocks
        self.cached = {}                          # hash -> block

    @property
    def num_free(self) -> int:
        return len(self.queue)

    def allocate(self, n: int):
        """Take n blocks from the head (None, nothing taken, if fewer are free).  A block
        that still carries a hash loses it: its contents are about to be replaced."""
        if n > len(self.queue):
            return None
        out = self.queue[:n]
        del self.queue[:n]
        for b in out:
            assert self.ref[b] == 0
            h = self.hash[b]
            if h is not None:
                if self.cached.get(h) == b:
                    del self.cached[h]
                self.hash[b] = None
            self.ref[b] = 1
        return out

    def free(self, ids) -> None:
        """Drop one reference per id, in order; a block reaching zero keeps its contents
        and returns to the queue: the tail if it has a hash, the head otherwise."""
        for b in set(ids):
            if list(ids).count(b) > self.ref[b]:
                raise ValueError("freed more often than referenced")
        for b in ids:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                if self.hash[b] is not None:
                    self.queue.append(b)
                else:
                    self.queue.insert(0, b)

    def touch(self, ids) -> None:
        """A prefix-cache hit: a free block leaves the queue from wherever it sits."""
        for b in ids:
            if self.ref[b] == 0 and b in self.queue:
                self.queue.remove(b)
            self.ref[b] += 1

    def cache_blocks(self, ids, hashes) -> None:
        for b, h in zip(ids, hashes):
            h &= MASK64
            if self.hash[b] is not None or h in self.cached:
                continue
            self.hash[b] = h
            self.cached[h] = b

    def longest_hit(self, hashes):
        """Blocks of the longest cached prefix (a linear scan that stops at the first miss)."""
        out = []
        for h in hashes:
            b = self.cached.get(h & MASK64)
            if b is None:
                break
            out.append(b)
        return out

    def cow(self, b: int):
        """Before writing into block b: (b, False) if the writer is its only user, else a
        fresh block and True (the writer's reference moves to the copy); None if no block
        is free."""
        assert self.ref[b] > 0
        if self.ref[b] == 1:
            return b, False
        fresh = self.allocate(1)
        if fresh is None:
            return None
        self.ref[b] -= 1
        return fresh[0], True
