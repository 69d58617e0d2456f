"""Host check of the rule by which the top-k finish's fallback rescores only
some chunks ("DeepSeek V4.1 Flash : 890 octets de cache KV par token",
section "L'architecture : trois leviers contre le cache": a Full layer keeps
the top-512 by score).

The score pass leaves, per chunk of 1024 positions, a list of every key whose
20-bit prefix reaches the chunk's cutoff (at most 256 of them, in position
order; more sets an overflow flag). When fewer than k keys reach the highest
cutoff, the finish looks for a level lam among the cutoffs, from the highest
down, that at least k listed keys reach with at most 8 chunks above it
(overflowed lists count as above); it rescores those chunks, takes the other
chunks' listed keys, and selects over that set. This test models the lists
and the rule on the CPU and checks, over randomized sequences with clustered,
tied and overflowing chunks, that the selection over the set equals the
oracle's top-k over every score. The GPU tests check the kernel itself.
"""
import numpy as np
import pytest

from oracle import indexer as OI

CHUNK, CAP, LEVELS, MAX_RESCORED = 1024, 256, 8, 8


def keys_of(s):
    """Order-preserving u32 keys of float32 scores (-0 maps like +0)."""
    b = (s.astype(np.float32) + np.float32(0)).view(np.uint32).astype(np.uint64)
    neg = (b >> 31) == 1
    return np.where(neg, (~b) & 0xFFFFFFFF, b | 0x80000000).astype(np.uint64)


def chunk_lists(s, k):
    """(cutoff prefix, overflow, listed positions) per chunk; the cutoff is the
    prefix of the chunk's budget-th largest key (0 when it has fewer keys)."""
    n = s.size
    key = keys_of(s)
    p20 = key >> 12
    share = -(-k * CHUNK // n)
    budget = 2 * share + 16
    out = []
    for c0 in range(0, n, CHUNK):
        pc = p20[c0:c0 + CHUNK]
        cut = int(np.sort(pc)[::-1][budget - 1]) if pc.size >= budget else 0
        listed = np.nonzero(pc >= cut)[0] + c0
        out.append((cut, listed.size > CAP, listed[:CAP]))
    return out, p20


def partial_selection(s, k):
    """The rule: returns the top-k over the candidate set, or None when no
    level qualifies (the whole sequence would be rescored)."""
    lists, p20 = chunk_lists(s, k)
    cuts = sorted({c for c, _, _ in lists}, reverse=True)
    for lam in cuts[1:1 + LEVELS]:
        above = [i for i, (c, ovf, _) in enumerate(lists) if ovf or c > lam]
        n_listed = sum(int((p20[l] >= lam).sum()) for c, ovf, l in lists if not ovf)
        if len(above) <= MAX_RESCORED and n_listed >= k:
            pos = []
            for i, (c, ovf, l) in enumerate(lists):
                pos.append(np.arange(i * CHUNK, min((i + 1) * CHUNK, s.size)) if i in above else l)
            pos = np.concatenate(pos)
            return OI.topk(s[pos], pos, k), len(above)
    return None, None


def sequence(rng, n, hot, tie_chunks, high_ties=()):
    s = rng.standard_normal(n).astype(np.float32)
    for c in hot:                      # clustered: a run of large scores in chunk c
        a = c * CHUNK + int(rng.integers(0, 200))
        s[a:a + 300] = s[a:a + 300] * 8 + 20
    for c in tie_chunks:               # tied: a chunk of exact zeros
        s[c * CHUNK:(c + 1) * CHUNK] = 0.0
    for c in high_ties:                # 600 equal scores above everything else: the list overflows
        s[c * CHUNK:c * CHUNK + 600] = 100.0
    return s


@pytest.mark.parametrize("seed", range(40))
def test_partial_rescore_selects_the_top_k(seed):
    rng = np.random.default_rng(1000 + seed)
    n = int(rng.integers(20000, 70000))
    nch = -(-n // CHUNK)
    hot = rng.choice(nch, size=int(rng.integers(1, 12)), replace=False)
    ties = rng.choice(nch, size=int(rng.integers(0, 3)), replace=False)
    high = rng.choice(nch, size=1, replace=False) if seed % 4 == 0 else ()
    s = sequence(rng, n, hot, ties, high)
    k = 512
    got, rescored = partial_selection(s, k)
    want = OI.topk(s, np.arange(n), k)
    if got is not None:
        assert rescored <= MAX_RESCORED
        assert np.array_equal(got, want)


def test_one_hot_chunk_rescores_only_it():
    """One chunk holds far larger scores than the rest: the first level below
    its cutoff already qualifies, and only that chunk is rescored."""
    rng = np.random.default_rng(5)
    s = sequence(rng, 65536, [63], [])
    got, rescored = partial_selection(s, 512)
    assert rescored == 1
    assert np.array_equal(got, OI.topk(s, np.arange(s.size), 512))


def test_overflowed_chunk_is_rescored():
    """600 equal scores above all others in one chunk: its list overflows
    (256 kept) yet 512 of them are among the best; the overflowed chunk is
    rescored with the clustered one, and the tie goes to the lowest positions."""
    rng = np.random.default_rng(9)
    s = sequence(rng, 60000, [40], [], [3])
    lists, _ = chunk_lists(s, 512)
    assert lists[3][1], "the tied chunk's list overflows"
    got, rescored = partial_selection(s, 512)
    assert got is not None and rescored == 2
    want = OI.topk(s, np.arange(s.size), 512)
    assert np.array_equal(got, want)
    assert np.array_equal(want, np.arange(3 * CHUNK, 3 * CHUNK + 512))


def test_overflowed_chunk_below_the_level_is_rescored():
    """A chunk whose list overflows at a cutoff no higher than the chosen
    level: 800 equal scores fill its list (256 kept, all ties), and its 30
    best keys, above everything, lie after them. Its list misses them, so it
    must be rescored although its cutoff is not above the level."""
    rng = np.random.default_rng(13)
    n = 60000
    s = rng.standard_normal(n).astype(np.float32)
    x = 7 * CHUNK
    s[x:x + 800] = 10.0
    s[x + 900:x + 930] = 50.0
    for c in range(20, 40):                       # chunks with 30 keys just above the tie value
        s[c * CHUNK:c * CHUNK + 30] = 12.0 + rng.random(30, dtype=np.float32)
    for c in (50, 52, 54):                        # clustered chunks above them
        s[c * CHUNK:c * CHUNK + 300] = 20.0 + 8.0 * np.abs(rng.standard_normal(300)).astype(np.float32)
    lists, p20 = chunk_lists(s, 512)
    assert lists[7][1], "the tied chunk's list overflows"
    got, rescored = partial_selection(s, 512)
    want = OI.topk(s, np.arange(n), 512)
    assert np.all(np.isin(np.arange(x + 900, x + 930), want))
    assert got is not None and rescored == 4
    assert np.array_equal(got, want)


def test_all_tied_has_no_level():
    """Every score equal: every list overflows, no level qualifies."""
    s = np.zeros(65536, np.float32)
    got, _ = partial_selection(s, 512)
    assert got is None
