"""Invariants of the host model of the balanced decode plan (tests/plan_model.py),
which the GPU test compares with the planning kernel's words: every visible
tile of every sequence lies in exactly one segment, each work-group's tiles
plus the sequence starts in its range cost at most one chunk plus one start,
the segments of a sequence are consecutive and in work-group order, and the
work-groups' segment lists tile the segment slots in order."""
import random

import numpy as np
import pytest

import synth
from plan_model import MIN_CHUNK, SEGMENT_COST, n_words, plan_words, unpack, visible_tiles


def brute_tiles(n, window, max_len):
    """Tiles of [max(0, n - W), n) by walking 32-row tiles (full windows of a
    multiple of 32 keys start at n - W)."""
    n = min(max(n, 0), max_len)
    lo = max(0, n - window) if window > 0 else 0
    if n <= lo:
        return 0
    org = lo if (window > 0 and window % 32 == 0 and n >= window) else 0
    return len({(r - org) // 32 for r in range(lo, n)})


@pytest.mark.parametrize("window", [0, 1, 31, 32, 100, 1024])
def test_visible_tiles_against_a_walk(window):
    for n in list(range(0, 140)) + [1023, 1024, 1025, 2047, 5000]:
        assert visible_tiles(n, window, 4096) == brute_tiles(n, window, 4096), (n, window)
    assert visible_tiles(5000, 0, 1500) == 47   # clamped to max_len


def check(lens, window, max_len, G):
    B = len(lens)
    words, S = plan_words(lens, window, max_len, G)
    assert len(words) == n_words(G, B)
    (chunk, T, S_h, used), wg, segs, seqs = unpack(words, G, B)
    tiles = [visible_tiles(int(n), window, max_len) for n in lens]
    assert T == sum(tiles) and S_h == S and S <= G + B
    assert chunk >= MIN_CHUNK and used <= G
    owner = {}
    order = []
    for j in range(G):
        first, n = wg[j]
        assert n >= 0 and (n > 0) == (first >= 0)
        cost = 0
        for s in range(first, first + n):
            b, lo, ln, length = segs[s]
            assert ln > 0 and 0 <= lo and lo + ln <= tiles[b]
            for x in range(lo, lo + ln):
                assert (b, x) not in owner
                owner[(b, x)] = j
            cost += ln + (SEGMENT_COST if lo == 0 else 0)
            order.append(s)
        assert cost <= chunk + SEGMENT_COST
    assert order == list(range(S))
    for b, t in enumerate(tiles):
        first, n = seqs[b]
        js = [owner[(b, x)] for x in range(t)]
        assert len(js) == t
        if t:
            assert sorted(set(js)) == list(range(min(js), max(js) + 1)) and len(set(js)) == n
            assert all(segs[first + k][0] == b for k in range(n))
            assert [segs[first + k][1] for k in range(n)] == sorted(segs[first + k][1] for k in range(n))
            assert all(segs[first + k][3] == min(max(int(lens[b]), 0), max_len) for k in range(n))
        else:
            assert n == 0


def test_random_batches():
    rnd = random.Random(5)
    for _ in range(300):
        B = rnd.choice([1, 2, 3, 17, 128, 300])
        hi = rnd.choice([3, 100, 40000])
        lens = [rnd.choice([0, rnd.randint(0, hi)]) for _ in range(B)]
        check(lens, rnd.choice([0, 0, 64, 1024, 100]), max(1, hi), rnd.choice([1, 2, 8, 256]))


def test_hybrid_global_layer():
    lens = synth.HYBRID.lens()
    check(list(lens), 0, int(lens.max()), 256)


def test_sequence_starts_shift_work_off_busy_ranges():
    """Ranges that start several short sequences get fewer tiles: the cost of
    a range (tiles plus 40 per sequence start) stays within one chunk of the
    others'."""
    lens = [32 * 300] * 10 + [32 * 20] * 30 + [32 * 300] * 10
    B, G = len(lens), 16
    words, _ = plan_words(lens, 0, 32 * 300, G)
    (chunk, *_), wg, segs, _ = unpack(words, G, B)
    tiles = np.array([sum(segs[s][2] for s in range(f, f + n)) for f, n in wg])
    starts = np.array([sum(segs[s][1] == 0 for s in range(f, f + n)) for f, n in wg])
    assert starts.max() >= 3 and tiles[starts.argmax()] <= tiles.max() - 2 * SEGMENT_COST
    assert np.all(tiles + SEGMENT_COST * starts <= chunk + SEGMENT_COST)
