"""Host-side check of the balanced decode split (no GPU).

The device code divides the T = Hkv * sum_s ceil(ctx_s / 64) tiles of a batch over
W' = min(W, T) waves: with a lead share f (in 1/1024) and W' = W even, the first
W'/2 waves share the first F = floor(T f / 1024) tiles evenly and the others the
remaining T - F (when both classes get at least one tile per wave), otherwise all
W' waves share the T tiles evenly.  Each wave walks its range in (sequence, kv
head, tile) order, finishes a (sequence, head) that lies inside its range, and
otherwise leaves one partial: in slot 1 if the piece starts the (sequence, head)
(only a wave's last segment can), in slot 0 if it starts inside it (only a wave's
first segment can); the merge takes the first covering wave's slot 1 and every
later covering wave's slot 0, locating the owner of a tile by the same split.  This test
replays that arithmetic on random mixes of lengths and checks that every tile is
processed exactly once and that the merge reads exactly the slots that were written
for that (sequence, head)."""
import numpy as np
import pytest


def split(T, Weff, W, lead_q10):
    """(F, Wl): the first Wl waves take the first F tiles."""
    if Weff == W and W % 2 == 0:
        F, Wl = T * lead_q10 // 1024, W // 2
        if F >= Wl and T - F >= W - Wl:
            return F, Wl
    return T, Weff


def begin(T, Weff, F, Wl, w):
    return w * F // Wl if w <= Wl else F + (w - Wl) * (T - F) // (Weff - Wl)


def owner(T, Weff, F, Wl, u):
    if u < F:
        return ((u + 1) * Wl - 1) // F
    return Wl + ((u - F + 1) * (Weff - Wl) - 1) // (T - F)


def plan(ctx, hkv, W, lead_q10):
    nt = [-(-int(c) // 64) for c in ctx]
    T = hkv * sum(nt)
    Weff = min(W, T)
    F, Wl = split(T, Weff, W, lead_q10)
    written = {}       # (wave, slot) -> (s, h)
    finished = {}      # (s, h) -> wave
    seen = []
    for w in range(Weff):
        b, e = begin(T, Weff, F, Wl, w), begin(T, Weff, F, Wl, w + 1)
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
        assert begin(T, Weff, F, Wl, Weff) == T
    return nt, T, Weff, (F, Wl), written, finished, seen


def check(ctx, hkv, nt, T, Weff, F, Wl, written, finished, seen):
    S = len(ctx)
    assert sorted(seen) == [(s, h, t) for s in range(S) for h in range(hkv) for t in range(nt[s])]
    before = np.concatenate([[0], np.cumsum(nt)])
    for s in range(S):
        for h in range(hkv):
            if nt[s] == 0:
                assert (s, h) not in finished
                continue
            u0 = before[s] * hkv + h * nt[s]
            w0 = owner(T, Weff, F, Wl, u0)
            w1 = owner(T, Weff, F, Wl, u0 + nt[s] - 1)
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
    W = int(rng.choice([1, 3, 7, 64, 2048]))
    lead = int(rng.choice([512, 584, 624, 700, 1000]))
    nt, T, Weff, (F, Wl), written, finished, seen = plan(ctx, hkv, W, lead)
    check(ctx, hkv, nt, T, Weff, F, Wl, written, finished, seen)


@pytest.mark.parametrize("shape", ["gqa", "long"])
def test_skewed_split_at_benchmark_shapes(shape):
    """The split the bf16 kernels take on a 256-CU device: 2048 waves, lead share 624."""
    rng = np.random.Generator(np.random.PCG64(7))
    if shape == "gqa":
        ctx, hkv = rng.integers(128, 4096, 64, endpoint=True), 8
    else:
        ctx, hkv = rng.integers(32768, 200000, 8, endpoint=True), 4
    nt, T, Weff, (F, Wl), written, finished, seen = plan(ctx, hkv, 2048, 624)
    assert Wl == 1024 and F == T * 624 // 1024          # the skewed path is taken
    check(ctx, hkv, nt, T, Weff, F, Wl, written, finished, seen)
    # lead waves hold ~1.56x the tiles of the others
    assert 1.53 < (F / Wl) / ((T - F) / (Weff - Wl)) < 1.59
