"""Algorithmic work of the hot path (what the method must move or compute).

Counted: one shared KV head per token, int8 K and V plus one fp32 scale each
(2*D + 8 bytes per visible key), visible keys only, and 4*D*Hq flops per
visible (query token, key) pair (QK^T and PV, 2 flops per multiply-add).
Excluded: masked keys, partial-state traffic, re-reads, padding.
"""
from __future__ import annotations


def kv_bytes_per_key(D: int) -> int:
    return 2 * D + 8


def decode_visible(n: int, window: int) -> int:
    return min(n, window) if window > 0 else n


def decode_kv_bytes(seq_lens, window: int, D: int) -> int:
    return sum(decode_visible(int(n), window) for n in seq_lens) * kv_bytes_per_key(D)


def decode_flops(seq_lens, window: int, Hq: int, D: int) -> int:
    return sum(decode_visible(int(n), window) for n in seq_lens) * 4 * D * Hq


def prefill_pairs(prefix_lens, C: int, window: int) -> int:
    tot = 0
    for P in prefix_lens:
        P = int(P)
        if window > 0:
            # query at position P+i sees min(W, P+i+1) keys
            for i in range(C):
                tot += min(window, P + i + 1)
        else:
            tot += C * P + C * (C + 1) // 2
    return tot


def prefill_flops(prefix_lens, C: int, window: int, Hq: int, D: int) -> int:
    return prefill_pairs(prefix_lens, C, window) * 4 * D * Hq


def prefill_kv_bytes(prefix_lens, C: int, window: int, D: int) -> int:
    """Distinct cache rows a chunk must read at least once."""
    tot = 0
    for P in prefix_lens:
        lo = max(0, int(P) - window + 1) if window > 0 else 0
        tot += int(P) + C - lo
    return tot * kv_bytes_per_key(D)
