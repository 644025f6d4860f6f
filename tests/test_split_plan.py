"""Host-side check of the balanced decode split (no GPU).

The device code divides the T = Hkv * sum_s ceil(ctx_s / 64) tiles of a batch into
W' = min(W, T) ranges [floor(wT/W'), floor((w+1)T/W')), walks each range in
(sequence, kv head, tile) order, finishes a (sequence, head) that lies inside one
range, and otherwise leaves a partial in slot 0 (first segment of a wave) and/or
slot 1 (last segment); the merge takes the first covering wave's slot 1 and every
later covering wave's slot 0, with owner(u) = ((u + 1) W' - 1) // T.  This test
replays that arithmetic on random mixes of lengths and checks that every tile is
processed exactly once and that the merge reads exactly the slots that were written
for that (sequence, head)."""
import numpy as np
import pytest


def plan(ctx, hkv, W):
    nt = [-(-int(c) // 64) for c in ctx]
    T = hkv * sum(nt)
    Weff = min(W, T)
    written = {}       # (wave, slot) -> (s, h)
    finished = {}      # (s, h) -> wave
    seen = []
    for w in range(Weff):
        b, e = w * T // Weff, (w + 1) * T // Weff
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
                if first:
                    written[(w, 0)] = (s, h)
                if last:
                    written[(w, 1)] = (s, h)
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
    return nt, T, Weff, written, finished, seen


@pytest.mark.parametrize("seed", range(40))
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
    W = int(rng.choice([1, 3, 7, 64, 2048]))
    nt, T, Weff, written, finished, seen = plan(ctx, hkv, W)
    # every tile exactly once
    want = [(s, h, t) for s in range(S) for h in range(hkv) for t in range(nt[s])]
    assert sorted(seen) == want
    # merge view
    before = np.concatenate([[0], np.cumsum(nt)])
    for s in range(S):
        for h in range(hkv):
            if nt[s] == 0:
                assert (s, h) not in finished
                continue
            u0 = before[s] * hkv + h * nt[s]
            w0 = ((u0 + 1) * Weff - 1) // T
            w1 = ((u0 + nt[s]) * Weff - 1) // T
            if w0 == w1:
                assert finished.get((s, h)) == w0
            else:
                assert (s, h) not in finished
                assert written[(w0, 1)] == (s, h)
                for w in range(w0 + 1, w1 + 1):
                    assert written[(w, 0)] == (s, h)
