"""Host block manager: the oracle's plain model pinned to the pages' rules and to the
published FNV-1a test vectors, then the library's C++ pool (pkv_pool_*) checked
against the model operation by operation on random streams (bit-exact: same blocks,
same free-queue order, same counts)."""
import numpy as np
import pytest

import paged_kv_cache_79_amd as pkv
from oracle import block_pool as BP


# --------------------------------------------------------------------------
# pins of the model
# --------------------------------------------------------------------------
def pin_fnv_vectors():
    # published FNV-1a 64-bit test vectors
    assert BP.fnv1a_64(b"") == 0xCBF29CE484222325
    assert BP.fnv1a_64(b"a") == 0xAF63DC4C8601EC8C
    assert BP.fnv1a_64(b"foobar") == 0x85944171F73967E8


def pin_hash_chain():
    """The same tokens under another parent hash differently; each block hash depends
    on every earlier block ("Inside vLLM, part 2", prefix caching)."""
    toks = list(range(16))
    a = BP.block_hash(0, toks)
    b = BP.block_hash(a, toks)
    assert a != b and BP.block_hash(0, toks) == a
    assert BP.block_hash(a, toks[:-1] + [99]) != b
    # byte layout: parent LE (8 bytes) then tokens LE (4 bytes each)
    assert BP.block_hash(0x61, []) == BP.fnv1a_64(b"a" + bytes(7))


def pin_allocation_from_head():
    p = BP.BlockPoolModel(6)
    assert p.allocate(4) == [0, 1, 2, 3]
    assert p.allocate(3) is None and p.num_free == 2      # nothing taken when short
    assert p.ref[:4] == [1, 1, 1, 1]


def pin_release_order():
    """Freed unhashed blocks go to the head (reused first), hashed ones to the tail
    (kept longer); a request frees tail first ("2.1 PagedAttention", 9.1 and 9.3)."""
    p = BP.BlockPoolModel(6)
    req = p.allocate(3)                                     # [0, 1, 2]
    p.free(list(reversed(req)))
    assert p.queue == [0, 1, 2, 3, 4, 5]
    req = p.allocate(3)
    p.cache_blocks(req, [11, 12, 13])
    p.free(list(reversed(req)))                             # hashed: to the tail, 2 first
    assert p.queue == [3, 4, 5, 2, 1, 0]


def pin_touch_revives_from_middle():
    p = BP.BlockPoolModel(6)
    req = p.allocate(3)
    p.cache_blocks(req, [21, 22, 23])
    p.free(list(reversed(req)))                             # queue [3, 4, 5, 2, 1, 0]
    hit = p.longest_hit([21, 22, 99, 23])                   # stops at the first miss
    assert hit == [0, 1]
    p.touch(hit)
    assert p.queue == [3, 4, 5, 2] and p.ref[0] == p.ref[1] == 1


def pin_reallocation_drops_hash():
    p = BP.BlockPoolModel(3)
    req = p.allocate(3)
    p.cache_blocks(req, [31, 32, 33])
    p.free([2, 1, 0])
    assert p.allocate(1) == [2]                             # the oldest cached block goes
    assert p.longest_hit([33]) == [] and p.longest_hit([31, 32]) == [0, 1]


def pin_copy_on_write():
    """A block two requests share is copied before either writes into it; a block
    with one user is written in place ("2.1 PagedAttention", section 6)."""
    p = BP.BlockPoolModel(4)
    a = p.allocate(2)                                       # request A: [0, 1]
    p.touch([0, 1])                                         # request B shares them
    assert p.cow(1) == (2, True) and p.ref[1] == 1 and p.ref[2] == 1
    assert p.cow(1) == (1, False)                           # now A is its only user
    p.allocate(1)
    assert p.cow(0) is None                                 # no block left for a copy


PINS = [pin_fnv_vectors, pin_hash_chain, pin_allocation_from_head, pin_release_order,
        pin_touch_revives_from_middle, pin_reallocation_drops_hash, pin_copy_on_write]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_model_pin(pin):
    pin()


class _HashedToHead(BP.BlockPoolModel):
    def free(self, ids):
        for b in ids:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.queue.insert(0, b)


class _TouchLeavesQueue(BP.BlockPoolModel):
    def touch(self, ids):
        for b in ids:
            self.ref[b] += 1


class _KeepsHashOnReuse(BP.BlockPoolModel):
    def allocate(self, n):
        if n > len(self.queue):
            return None
        out = self.queue[:n]
        del self.queue[:n]
        for b in out:
            self.ref[b] = 1
        return out


class _CowWithoutRelease(BP.BlockPoolModel):
    def cow(self, b):
        if self.ref[b] == 1:
            return b, False
        fresh = self.allocate(1)
        return (fresh[0], True) if fresh else None


@pytest.mark.parametrize("mutant", [_HashedToHead, _TouchLeavesQueue, _KeepsHashOnReuse,
                                    _CowWithoutRelease], ids=lambda c: c.__name__)
def test_model_mutants_are_caught(mutant, monkeypatch):
    monkeypatch.setattr(BP, "BlockPoolModel", mutant)
    caught = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, TypeError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches {mutant.__name__}"


# --------------------------------------------------------------------------
# the C++ pool against the model
# --------------------------------------------------------------------------
def test_block_hash_matches_model():
    rng = np.random.default_rng(5)
    for _ in range(200):
        parent = int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2))
        toks = rng.integers(-2**31, 2**31, int(rng.integers(0, 40))).tolist()
        assert pkv.block_hash(parent, toks) == BP.block_hash(parent, toks)


@pytest.mark.parametrize("seed", range(12))
def test_pool_matches_model(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(4, 64))
    lib, ref = pkv.BlockPool(n), BP.BlockPoolModel(n)
    live = []                       # requests: lists of blocks they hold
    hashes = {}                     # block -> hash given to it (to re-find later)
    next_hash = 1000
    for step in range(400):
        op = rng.choice(["alloc", "free", "cache", "hit", "cow", "share"])
        if op == "alloc":
            k = int(rng.integers(1, max(2, n // 3)))
            got, want = lib.allocate(k), ref.allocate(k)
            assert got == want, (step, op)
            if got is not None:
                live.append(list(got))
        elif op == "free" and live:
            req = live.pop(int(rng.integers(len(live))))
            lib.free(list(reversed(req)))
            ref.free(list(reversed(req)))
        elif op == "cache" and live:
            req = live[int(rng.integers(len(live)))]
            hs = []
            for b in req:
                hashes.setdefault(b, next_hash)
                hs.append(hashes[b])
                next_hash += 1
            lib.cache_blocks(req, hs)
            ref.cache_blocks(req, hs)
        elif op == "hit" and hashes:
            keys = list(hashes.values())
            q = [keys[int(i)] for i in rng.integers(0, len(keys), int(rng.integers(1, 6)))]
            got, want = lib.longest_hit(q), ref.longest_hit(q)
            assert got == want, (step, op)
            if got:
                lib.touch(got)
                ref.touch(got)
                live.append(list(got))
        elif op == "cow" and live:
            req = live[int(rng.integers(len(live)))]
            j = int(rng.integers(len(req)))
            got, want = lib.cow(req[j]), ref.cow(req[j])
            assert got == want, (step, op)
            if got is not None:
                req[j] = got[0]
        elif op == "share" and live:
            req = live[int(rng.integers(len(live)))]
            lib.touch(req)
            ref.touch(req)
            live.append(list(req))
        assert lib.free_queue() == ref.queue, (step, op)
        assert lib.num_free == ref.num_free
        assert [lib.ref_count(b) for b in range(n)] == ref.ref, (step, op)


def test_pool_rejects_bad_frees_without_changing_anything():
    p = pkv.BlockPool(4)
    got = p.allocate(2)
    before = (p.free_queue(), [p.ref_count(b) for b in range(4)])
    with pytest.raises(pkv.PagedKVError):
        p.free([got[0], got[0]])                # listed twice, referenced once
    with pytest.raises(pkv.PagedKVError):
        p.free([7])                             # out of range
    assert (p.free_queue(), [p.ref_count(b) for b in range(4)]) == before
    assert p.cow(got[1]) == (got[1], False)
