"""Host model of the balanced decode plan that mqa_decode_ragged's planning
kernel writes at the start of its workspace (layout documented beside the
kernel): the visible 32-key tiles of all sequences, each sequence preceded
by a fixed start cost, laid end to end and cut into G ranges of equal cost.

Integer bookkeeping only (no attention arithmetic): the GPU test compares the
kernel's plan words with this model exactly, and the CPU tests check the
model's own invariants (every tile in exactly one segment, no range costing
more than its chunk plus one start, segments and slots in order)."""
from __future__ import annotations

import numpy as np

SEGMENT_COST = 40   # cost of a sequence start, in tiles
MIN_CHUNK = 8       # at least one tile per wave of a work-group
TILE = 32


def visible_tiles(n: int, window: int, max_len: int) -> int:
    """Tiles the attention kernel computes for a sequence of n keys (full
    windows whose length is a multiple of 32 are tiled from their first key,
    other ranges from 32-aligned rows)."""
    n = min(max(n, 0), max_len)
    lo = max(0, n - window) if window > 0 else 0
    if window > 0 and window % TILE == 0 and n >= window:
        return window // TILE
    b = lo // TILE
    end = (n + TILE - 1) // TILE if n > lo else b
    return end - b


def plan_words(seq_lens, window: int, max_len: int, G: int) -> np.ndarray:
    """The plan as int32 words: header {chunk, T, segments, ranges used};
    per work-group {first segment, segments} ({-1, 0} without tiles); per
    segment slot (G + B of them, unused ones left as they were: zero here)
    {sequence, first tile, tiles, the sequence's length clamped to
    [0, max_len]}; per sequence {first segment, segments}."""
    B = len(seq_lens)
    tiles = [visible_tiles(int(n), window, max_len) for n in seq_lens]
    cost = [t + SEGMENT_COST if t > 0 else 0 for t in tiles]
    C, T = sum(cost), sum(tiles)
    chunk = max(MIN_CHUNK, -(-C // G))
    wg = np.zeros((G, 2), np.int64)
    wg[:, 0] = -1
    segs = np.zeros((G + B, 4), np.int64)
    seqs = np.zeros((B, 2), np.int64)
    Q = S = 0
    for b, t in enumerate(tiles):
        A = Q + SEGMENT_COST                      # unit of the sequence's first tile
        n = (A + t - 1) // chunk - A // chunk + 1 if t > 0 else 0
        seqs[b] = (S, n)
        for k in range(n):
            j = A // chunk + k
            lo, hi = max(j * chunk, A), min((j + 1) * chunk, A + t)
            segs[S + k] = (b, lo - A, hi - lo, min(max(int(seq_lens[b]), 0), max_len))
            # first segment of range j: a range that opens inside this sequence,
            # or one where no earlier sequence has a tile
            if k > 0 or Q == 0 or (Q - 1) // chunk != j:
                wg[j, 0] = S + k
        Q += cost[b]
        S += n
    firsts = [j for j in range(G) if wg[j, 0] >= 0]
    for i, j in enumerate(firsts):
        nxt = wg[firsts[i + 1], 0] if i + 1 < len(firsts) else S
        wg[j, 1] = nxt - wg[j, 0]
    header = np.array([chunk, T, S, -(-C // chunk)], np.int64)
    return np.concatenate([header, wg.ravel(), segs.ravel(), seqs.ravel()]).astype(np.int32), S


def unpack(words: np.ndarray, G: int, B: int):
    w = np.asarray(words, np.int64)
    header = w[:4]
    wg = w[4:4 + 2 * G].reshape(G, 2)
    segs = w[4 + 2 * G:4 + 2 * G + 4 * (G + B)].reshape(G + B, 4)
    seqs = w[4 + 2 * G + 4 * (G + B):4 + 2 * G + 4 * (G + B) + 2 * B].reshape(B, 2)
    return header, wg, segs, seqs


def n_words(G: int, B: int) -> int:
    return 4 + 2 * G + 4 * (G + B) + 2 * B
