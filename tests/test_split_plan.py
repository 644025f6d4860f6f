"""Host-side check of the balanced decode split (no GPU).

The device code divides the T = Hkv * sum_s ceil(ctx_s / 64) tiles of a batch over
W' = min(W, T) waves into contiguous ranges.  When the grid fills every wave slot
(W' = W), W is a multiple of 16 and T >= 2W, wave w gets a share proportional to a
class weight -- lead share f (in 1/1024) for the first half of the grid, 1024 - f for
the second -- times the weight of the XCD it runs on (w mod 8, the table kXcdWeight of
pkv_split.h, read from the header here); otherwise the T tiles are shared evenly.  Range
w starts at floor(T P(w) / P(W)) with P the prefix sum of the weights.  Each wave walks
its range in (sequence, kv head, tile) order, finishes a (sequence, head) that lies
inside its range, and otherwise leaves one partial: in slot 1 if the piece starts the
(sequence, head) (only a wave's last segment can), in slot 0 if it starts inside it
(only a wave's first segment can); the merge takes the first covering wave's slot 1 and
every later covering wave's slot 0, locating the owner of a tile by the same split.  This
test replays that arithmetic on random mixes of lengths and checks that every tile is
processed exactly once and that the merge reads exactly the slots that were written
for that (sequence, head)."""
import os
import re

import numpy as np
import pytest

_HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "paged_kv_cache_79_amd", "csrc", "pkv_split.h")
XCD_WEIGHT = [int(x) for x in re.search(r"kXcdWeight\[8\] = \{([^}]*)\}", open(_HDR).read())
              .group(1).split(",")]


def xcd_prefix(n):
    return (n // 8) * sum(XCD_WEIGHT) + sum(XCD_WEIGHT[:n % 8])


def split(T, Weff, W, lead_q10):
    """(Wl, lw, gw, Ptot): Wl = 0 is the even split."""
    if Weff == W and W % 16 == 0 and 0 < lead_q10 < 1024:
        lw, gw = lead_q10, 1024 - lead_q10
        Ptot = (lw + gw) * xcd_prefix(W // 2)
        if T * min(lw, gw) * min(XCD_WEIGHT) >= Ptot:     # the lightest share >= 1 tile
            return W // 2, lw, gw, Ptot
    return 0, 1, 1, Weff


def prefix(sp, w):
    Wl, lw, gw, _ = sp
    if Wl == 0:
        return w
    return lw * xcd_prefix(w) if w <= Wl else lw * xcd_prefix(Wl) + gw * xcd_prefix(w - Wl)


def begin(T, Weff, sp, w):
    return T * prefix(sp, w) // sp[3]


def owner(T, Weff, sp, u):
    lo, hi = 0, Weff - 1
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if begin(T, Weff, sp, mid) <= u:
            lo = mid
        else:
            hi = mid - 1
    return lo


def plan(ctx, hkv, W, lead_q10):
    nt = [-(-int(c) // 64) for c in ctx]
    T = hkv * sum(nt)
    Weff = min(W, T)
    sp = split(T, Weff, W, lead_q10)
    written = {}       # (wave, slot) -> (s, h)
    finished = {}      # (s, h) -> wave
    seen = []
    for w in range(Weff):
        b, e = begin(T, Weff, sp, w), begin(T, Weff, sp, w + 1)
        assert b < e
        before = 0
        s = 0
        while hkv * (before + nt[s]) <= b:
            before += nt[s]
            s += 1
        rel = b - before * hkv
        h, tile = rel // nt[s], rel % nt[s]
        rem, first = e - b, True
        while rem > 0:
            seg = min(nt[s] - tile, rem)
            last = seg == rem
            seen += [(s, h, t) for t in range(tile, tile + seg)]
            if tile == 0 and seg == nt[s]:
                assert (s, h) not in finished
                finished[(s, h)] = w
            else:
                slot = 1 if tile == 0 else 0
                assert (w, slot) not in written
                assert (slot == 1 and last) or (slot == 0 and first)
                written[(w, slot)] = (s, h)
            rem -= seg
            first = False
            if rem > 0:
                tile = 0
                h += 1
                if h == hkv:
                    h = 0
                    s += 1
                    while nt[s] == 0:
                        s += 1
    if T:
        assert begin(T, Weff, sp, Weff) == T
    return nt, T, Weff, sp, written, finished, seen


def check(ctx, hkv, nt, T, Weff, sp, written, finished, seen):
    S = len(ctx)
    assert sorted(seen) == [(s, h, t) for s in range(S) for h in range(hkv) for t in range(nt[s])]
    before = np.concatenate([[0], np.cumsum(nt)])
    for s in range(S):
        for h in range(hkv):
            if nt[s] == 0:
                assert (s, h) not in finished
                continue
            u0 = before[s] * hkv + h * nt[s]
            w0 = owner(T, Weff, sp, u0)
            w1 = owner(T, Weff, sp, u0 + nt[s] - 1)
            if w0 == w1:
                assert finished.get((s, h)) == w0
            else:
                assert (s, h) not in finished
                assert written[(w0, 1)] == (s, h)
                for w in range(w0 + 1, w1 + 1):
                    assert written[(w, 0)] == (s, h)


@pytest.mark.parametrize("seed", range(60))
def test_balanced_split_covers_and_merges(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    S = int(rng.integers(1, 40))
    hkv = int(rng.choice([1, 2, 4, 8]))
    kind = seed % 4
    if kind == 0:
        ctx = rng.integers(0, 300, S)                    # short, some empty
    elif kind == 1:
        ctx = rng.integers(1, 20000, S)                  # long
    elif kind == 2:
        ctx = np.where(rng.random(S) < 0.5, 0, rng.integers(1, 5000, S))
    else:
        ctx = rng.integers(60, 70, S)                    # around one tile
    W = int(rng.choice([1, 3, 7, 16, 64, 1024, 2048]))
    lead = int(rng.choice([512, 584, 624, 656, 700, 1000]))
    nt, T, Weff, sp, written, finished, seen = plan(ctx, hkv, W, lead)
    check(ctx, hkv, nt, T, Weff, sp, written, finished, seen)


@pytest.mark.parametrize("shape", ["gqa", "long"])
def test_skewed_split_at_benchmark_shapes(shape):
    """The split the bf16 kernels take on a 256-CU device: 2048 waves, lead share 656."""
    rng = np.random.Generator(np.random.PCG64(7))
    if shape == "gqa":
        ctx, hkv = rng.integers(128, 4096, 64, endpoint=True), 8
    else:
        ctx, hkv = rng.integers(32768, 200000, 8, endpoint=True), 4
    nt, T, Weff, sp, written, finished, seen = plan(ctx, hkv, 2048, 656)
    assert sp[0] == 1024                                 # the weighted path is taken
    check(ctx, hkv, nt, T, Weff, sp, written, finished, seen)
    sizes = np.diff([begin(T, Weff, sp, w) for w in range(Weff + 1)])
    # lead waves hold ~656/368 = 1.78x the tiles of the others; within a class, even XCDs more
    lead, lag = sizes[:1024].mean(), sizes[1024:].mean()
    assert 1.75 < lead / lag < 1.81
    even, odd = sizes[0::2].mean(), sizes[1::2].mean()
    assert 1.02 < even / odd < 1.06
    assert sizes.min() >= 1


def test_weighted_split_never_leaves_a_range_empty():
    """From the smallest T the weighted split takes, for uneven lead shares."""
    for W in (16, 1024, 2048):
        for lead in (512, 656, 1000):
            for T in range(W, 40 * W, max(1, W // 3)):
                sp = split(T, W, W, lead)
                if sp[0] == 0:
                    continue
                b = [begin(T, W, sp, w) for w in range(W + 1)] if W <= 16 or T % 7 == 0 else \
                    [begin(T, W, sp, w) for w in (0, W // 2 - 1, W // 2, W // 2 + 1, W - 1, W)]
                assert b[0] == 0 and b[-1] == T and min(np.diff(b)) >= 1, (W, lead, T)
    assert split(2 * 2048, 2048, 2048, 656)[0] == 1024   # the benchmark grids are weighted
