"""The host prefix cache's control plane (CPU, through the C ABI) against the
plain policy model in oracle/prefix_cache_ref.py, on synthetic multi-turn
conversation streams (growing histories, regenerated replies that share a
partial prefix, many conversations competing for a small cache)."""
import numpy as np
import pytest

import synth
from oracle.prefix_cache_ref import PrefixCacheRef


def conversation_stream(seed, n_conv, n_events, vocab=50):
    """Events (conversation id, tokens requested, tokens kept after the turn)."""
    g = synth.rng(980, 1, seed)
    hist = [list(g.integers(0, vocab, size=int(g.integers(5, 40)))) for _ in range(n_conv)]
    for _ in range(n_events):
        c = int(g.integers(0, n_conv))
        user = list(g.integers(0, vocab, size=int(g.integers(1, 30))))
        reply = list(g.integers(0, vocab, size=int(g.integers(1, 30))))
        request = hist[c] + user
        if g.random() < 0.2 and len(hist[c]) > 8:
            # regenerate: the last reply is replaced, only part of the history is shared
            cut = int(g.integers(len(hist[c]) // 2, len(hist[c])))
            request = hist[c][:cut] + user
            hist[c] = hist[c][:cut]
        hist[c] = request + reply
        yield c, request, hist[c]


@pytest.mark.parametrize("bs,cap,n_conv", [(4, 40, 6), (8, 25, 10), (16, 200, 4), (4, 3, 3)])
def test_policy_matches_model(bs, cap, n_conv):
    import mqa_attention_int8_amd as m
    cache = m.PrefixCache(bs, cap)
    ref = PrefixCacheRef(bs, cap)
    for i, (c, request, kept) in enumerate(conversation_stream(bs * 100 + cap, n_conv, 300)):
        got, slots = cache.match(request)
        want = ref.match(request)
        assert got == want, (i, got, want)
        assert len(slots) == got // bs and len(set(slots.tolist())) == len(slots)
        slots2, first, n = cache.insert(kept)
        rf, rn = ref.insert(kept)
        assert (first, n) == (rf, rn), (i, first, n, rf, rn)
        assert len(set(slots2.tolist())) == len(slots2)
        assert np.all((slots2 >= 0) & (slots2 < cap))
        st = cache.stats()
        assert st["used_blocks"] == ref.cached_blocks() <= cap
        assert st["evicted_blocks"] == ref.evicted
    cache.close()


def test_slots_are_stable_while_cached():
    import mqa_attention_int8_amd as m
    cache = m.PrefixCache(4, 100)
    a = list(range(40))
    slots, first, n = cache.insert(a)
    assert first == 0 and n == 10
    b = a[:22] + [99, 98, 97, 96, 95, 94]        # shares 5 full blocks and 2 tokens of the 6th
    got, s = cache.match(b)
    assert got == 20 and np.array_equal(s, slots[:5])
    s2, first2, n2 = cache.insert(b)
    assert first2 == 5 and n2 == 7 and np.array_equal(s2[:5], slots[:5])
    assert not set(s2[5:].tolist()) & set(slots.tolist())


def test_hit_rate_of_a_long_conversation():
    """A conversation of many turns finds its whole history (up to the last
    partial block) cached at every turn once the cache holds it."""
    import mqa_attention_int8_amd as m
    bs = 16
    cache = m.PrefixCache(bs, 10_000)
    g = synth.rng(981, 1)
    hist = []
    for turn in range(60):
        request = hist + list(g.integers(0, 1000, size=int(g.integers(5, 60))))
        got, _ = cache.match(request)
        assert got == (len(hist) // bs) * bs
        hist = request + list(g.integers(0, 1000, size=int(g.integers(5, 60))))
        cache.insert(hist)
    st = cache.stats()
    assert st["matched_tokens"] / st["lookup_tokens"] > 0.8


def _golden_cases():
    from _golden import prefix_cache_cases
    return prefix_cache_cases()


@pytest.mark.parametrize("ci", [0, 1])
def test_model_follows_hand_worked_sequence(ci):
    """The policy model against a sequence worked out by hand: a partial
    match, evictions of the least recently used leaf (not the oldest block),
    a cascade where a parent becomes the next leaf, and an insert that stops
    instead of evicting its own chain."""
    bs, cap, ops = _golden_cases()[ci]
    ref = PrefixCacheRef(bs, cap)
    for i, (op, toks, want) in enumerate(ops):
        if op == "match":
            assert ref.match(toks) == want[0], (i, op, toks)
        elif op == "insert":
            assert list(ref.insert(toks)) == want, (i, op, toks)
        elif op == "state":
            assert sorted(ref.last_use) == want, i
        else:
            assert ref.evicted == want, i


@pytest.mark.parametrize("ci", [0, 1])
def test_library_follows_hand_worked_sequence(ci):
    import mqa_attention_int8_amd as m
    bs, cap, ops = _golden_cases()[ci]
    cache = m.PrefixCache(bs, cap)
    for i, (op, toks, want) in enumerate(ops):
        if op == "match":
            got, _ = cache.match(toks)
            assert got == want[0], (i, op, toks)
        elif op == "insert":
            _, first, n = cache.insert(toks)
            assert [first, n] == want, (i, op, toks)
        elif op == "state":
            assert cache.stats()["used_blocks"] == len(want), i
        else:
            assert cache.stats()["evicted_blocks"] == want, i
    cache.close()
