"""Pins for the oracle's paged KV mapping (CPU only).

The mapping is checked against constructions that do not use it: block-wise
copies of a contiguous cache, the contiguous layout it must reduce to, and a
simulated ring of appends. The residency rule the library validates is
checked by brute force over small rings.
"""
import numpy as np
import pytest

import oracle
import synth


from gpu_util import block_copy_pool  # whole-block copies, no use of the mapping under test


@pytest.mark.parametrize("bs", [32, 64])
def test_identity_table_is_contiguous_layout(bs):
    B, TL, D = 3, 5, 8
    pool = synth.rng(900, 1).integers(-127, 128, size=(B * TL, bs, D)).astype(np.int8)
    table = np.arange(B * TL, dtype=np.int32).reshape(B, TL)
    got = oracle.paged_gather(pool, table, bs, TL * bs)
    assert np.array_equal(got, pool.reshape(B, TL * bs, D))


@pytest.mark.parametrize("bs", [32, 128])
def test_shuffled_blocks_gather_back(bs):
    B, TL, D = 4, 6, 16
    num_blocks = 40
    cont = synth.rng(901, 1).integers(-127, 128, size=(B, TL * bs, D)).astype(np.int8)
    table = synth.block_table(synth.rng(901, 2), B, TL, num_blocks)
    pool = block_copy_pool(cont, table, bs, num_blocks)
    assert np.array_equal(oracle.paged_gather(pool, table, bs, TL * bs), cont)
    # scales travel the same way (a pool of one value per row)
    sc = synth.rng(901, 3).random((B, TL * bs)).astype(np.float32)
    assert np.array_equal(oracle.paged_gather(block_copy_pool(sc, table, bs, num_blocks), table, bs, TL * bs), sc)


def test_scatter_matches_block_copy():
    B, TL, bs, D = 2, 4, 32, 4
    num_blocks = 11
    cont = synth.rng(902, 1).integers(-127, 128, size=(B, TL * bs, D)).astype(np.int8)
    table = synth.block_table(synth.rng(902, 2), B, TL, num_blocks)
    pool = np.zeros((num_blocks, bs, D), np.int8)
    # written in three uneven pieces, as appends would arrive
    for lo, hi in ((0, 5), (5, 70), (70, TL * bs)):
        oracle.paged_scatter(pool, table, bs, cont[:, lo:hi], [lo] * B)
    assert np.array_equal(pool, block_copy_pool(cont, table, bs, num_blocks))


def test_distinct_positions_distinct_rows():
    B, TL, bs = 3, 7, 32
    table = synth.block_table(synth.rng(903, 1), B, TL, 30)
    rows = np.concatenate([oracle.paged_rows(table, bs, b, np.arange(TL * bs)) for b in range(B)])
    assert len(np.unique(rows)) == len(rows)


@pytest.mark.parametrize("bs,TL", [(32, 2), (32, 5), (64, 3)])
def test_ring_keeps_recent_positions(bs, TL):
    """Append positions one at a time through a wrapping table; after each
    append the last TL * bs positions read back and the one before them has
    been overwritten."""
    table = np.array([[7, 2, 9, 4, 0][:TL]], np.int32)
    pool = np.full((10, bs, 1), -1, np.int64)
    n_total = 5 * TL * bs + 3
    keep = TL * bs
    for n in range(1, n_total + 1):
        oracle.paged_scatter(pool, table, bs, np.array([[[n - 1]]], np.int64), [n - 1])
        lo = max(0, n - keep)
        view = oracle.paged_gather(pool, table, bs, n)[0, :, 0]
        assert np.array_equal(view[lo:n], np.arange(lo, n)), n
        if n > keep:
            assert view[n - keep - 1] == n - 1  # its row now holds the newest position


def test_residency_rule_brute_force():
    """paged_window_resident(window, TL, bs) holds exactly when every window
    of the last `window` positions survives a long run of appends."""
    bs = 32
    for TL in (1, 2, 3):
        for window in (1, 2, bs - 1, bs, bs + 1, 2 * bs, 2 * bs + 1, 3 * bs, 3 * bs + 1):
            table = np.arange(TL, dtype=np.int32)[None]
            pool = np.full((TL, bs, 1), -1, np.int64)
            ok = True
            for n in range(1, 4 * TL * bs + 5):
                oracle.paged_scatter(pool, table, bs, np.array([[[n - 1]]], np.int64), [n - 1])
                lo = max(0, n - window)
                ok &= bool(np.array_equal(oracle.paged_gather(pool, table, bs, n)[0, lo:n, 0], np.arange(lo, n)))
            assert ok == oracle.paged_window_resident(window, TL, bs), (TL, window)


def test_paged_decode_equals_contiguous_decode():
    """Attention through the paged view of a shuffled pool equals attention on
    the contiguous cache it was built from (same numbers, no rounding)."""
    B, Hq, D, bs, TL = 2, 4, 16, 32, 3
    L = TL * bs
    g = synth.rng(905, 1)
    q = synth.q_bf16(g, (B, Hq, D))
    kq, ks = oracle.quantize_rows(synth.normal_f32(synth.rng(905, 2), (B, L, D)))
    vq, vs = oracle.quantize_rows(synth.normal_f32(synth.rng(905, 3), (B, L, D)))
    lens = np.array([L, 50], np.int32)
    table = synth.block_table(synth.rng(905, 4), B, TL, 9)
    P = lambda a: oracle.paged_gather(block_copy_pool(a, table, bs, 9), table, bs, L)
    for window in (0, 40):
        ref = oracle.decode_ref(q, kq, ks, vq, vs, lens, window)
        got = oracle.decode_ref(q, P(kq), P(ks), P(vq), P(vs), lens, window)
        assert np.array_equal(ref, got)
