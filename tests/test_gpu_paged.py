"""Paged KV buffers on the GPU: kv_quantize_int8_paged, mqa_decode_paged,
mqa_decode_append_paged and mqa_prefill_chunk_paged against the oracle.

Pools are built from seeded contiguous caches by whole-block copies through
shuffled block tables, so the paged result must equal the contiguous one (up
to summation order, 1e-6) and the oracle (decode 1e-4; prefill
5e-3 + 1e-2 |ref|). Ring buffers (tables shorter than the sequence) are
filled by appending every position in order through kv_quantize_int8_paged;
the oracle sees the whole sequence, so the check also covers that the ring
still holds every key the window reads.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (HostKV, assert_decode_close, assert_prefill_close, block_copy_pool, dev, log,
                      paged_from_host, q_bits, q_dev)

pytestmark = pytest.mark.gpu

WID = 60


def shuffled_table(seed, B, TL, spare=5):
    nb = B * TL + spare
    return synth.block_table(synth.rng(WID, 50, seed), B, TL, nb), nb


@pytest.mark.parametrize("D,bs,TL,T,start", [(128, 32, 6, 37, [0, 50, 150]), (64, 64, 3, 40, [5, 100, 130]),
                                              (128, 32, 2, 40, [100, 7, 0])])
def test_quantize_paged_exact(D, bs, TL, T, start):
    import mqa_attention_int8_amd as m
    B = 3
    log(f"quantize paged: D={D} bs={bs} TL={TL} T={T} start={start}")
    table, nb = shuffled_table(1, B, TL)
    k = synth.normal_f32(synth.rng(WID, synth.T_K, 1), (B, T, D))
    v = synth.normal_f32(synth.rng(WID, synth.T_V, 1), (B, T, D))
    kq, ks = oracle.quantize_rows(k)
    vq, vs = oracle.quantize_rows(v)
    sentinel_q, sentinel_s = np.int8(90), np.float32(-7.0)
    exp = [np.full((nb, bs, D), sentinel_q, np.int8), np.full((nb, bs), sentinel_s, np.float32),
           np.full((nb, bs, D), sentinel_q, np.int8), np.full((nb, bs), sentinel_s, np.float32)]
    for arr, rows in zip(exp, (kq, ks, vq, vs)):
        oracle.paged_scatter(arr, table, bs, rows, start)
    kv = m.PagedKV(dev(np.full((nb, bs, D), sentinel_q, np.int8)), dev(np.full((nb, bs, D), sentinel_q, np.int8)),
                   dev(np.full((nb, bs), sentinel_s, np.float32)), dev(np.full((nb, bs), sentinel_s, np.float32)),
                   dev(table))
    m.kv_quantize_int8_paged(dev(k), dev(v), kv, dev(np.asarray(start, np.int32)))
    torch.cuda.synchronize()
    for name, got, want in (("k", kv.k, exp[0]), ("k_scale", kv.k_scale, exp[1]), ("v", kv.v, exp[2]),
                            ("v_scale", kv.v_scale, exp[3])):
        assert got.cpu().numpy().tobytes() == want.tobytes(), f"pool {name} differs from the oracle's scatter"


@pytest.mark.parametrize("D,Hq,bs,W", [(128, 32, 32, 0), (128, 32, 128, 256), (64, 8, 64, 0), (128, 64, 32, 100),
                                       (64, 16, 32, 1024)])
def test_decode_paged_matches_oracle(D, Hq, bs, W):
    import mqa_attention_int8_amd as m
    B, L = 4, 600
    TL = -(-L // bs)
    log(f"decode paged: D={D} Hq={Hq} bs={bs} W={W}")
    hk = HostKV.seeded(WID, 2, B, TL * bs, D)
    lens = synth.ragged_lens(synth.rng(WID, synth.T_LENS, 2), B, 1, L).astype(np.int32)
    lens[0] = L
    table, nb = shuffled_table(2, B, TL)
    qb = q_bits(WID, (B, Hq, D), 2)
    ref = oracle.decode_ref(qb, *hk.arrays(), lens, W)
    kvp = paged_from_host(hk, table, bs, nb)
    q, seq = q_dev(qb), dev(lens)
    out = m.mqa_decode_paged(q, kvp, seq, int(lens.max()), W)
    cont = m.mqa_decode(q, hk.to_device(), seq, int(lens.max()), W)
    torch.cuda.synchronize()
    assert float((out - cont).abs().max()) <= 1e-6, "paged and contiguous decode differ"
    assert_decode_close(out, ref, 1e-4, f"paged D={D} Hq={Hq} bs={bs} W={W}")


def fill_ring(m, kvp, table, k, v, lens, chunk):
    """Append positions 0 .. lens[b]-1 of each sequence, in order, `chunk`
    positions per kv_quantize_int8_paged call (one sequence per call)."""
    from mqa_attention_int8_amd import PagedKV
    for b in range(k.shape[0]):
        row = PagedKV(kvp.k, kvp.v, kvp.k_scale, kvp.v_scale, kvp.block_table[b:b + 1].contiguous())
        for lo in range(0, int(lens[b]), chunk):
            hi = min(int(lens[b]), lo + chunk)
            m.kv_quantize_int8_paged(dev(k[b:b + 1, lo:hi]), dev(v[b:b + 1, lo:hi]), row,
                                     dev(np.array([lo], np.int32)))


@pytest.mark.parametrize("D,bs,TL,W", [(128, 32, 8, 256), (64, 64, 5, 300)])
def test_decode_paged_ring(D, bs, TL, W):
    import mqa_attention_int8_amd as m
    B, Hq = 3, 32
    lens = np.array([1500, 777, 2100], np.int32)
    L = int(lens.max())
    assert oracle.paged_window_resident(W, TL, bs)
    log(f"decode ring: D={D} bs={bs} TL={TL} (ring {TL * bs}) W={W} lens={lens.tolist()}")
    k = synth.normal_f32(synth.rng(WID, synth.T_K, 3), (B, L, D))
    v = synth.normal_f32(synth.rng(WID, synth.T_V, 3), (B, L, D))
    kq, ks = oracle.quantize_rows(k)
    vq, vs = oracle.quantize_rows(v)
    table, nb = shuffled_table(3, B, TL)
    kvp = m.PagedKV.empty(nb, bs, D, dev(table))
    fill_ring(m, kvp, table, k, v, lens, chunk=96)
    qb = q_bits(WID, (B, Hq, D), 3)
    out = m.mqa_decode_paged(q_dev(qb), kvp, dev(lens), L, W)
    torch.cuda.synchronize()
    ref = oracle.decode_ref(qb, kq, ks, vq, vs, lens, W)
    assert_decode_close(out, ref, 1e-4, f"ring D={D} bs={bs} W={W}")


@pytest.mark.parametrize("bs,W", [(64, 0), (32, 100)])
def test_decode_append_paged(bs, W):
    import mqa_attention_int8_amd as m
    B, Hq, D, L = 4, 32, 128, 700
    TL = -(-L // bs)
    log(f"append paged: bs={bs} W={W}")
    hk = HostKV.seeded(WID, 4, B, TL * bs, D)
    lens = synth.ragged_lens(synth.rng(WID, synth.T_LENS, 4), B, 1, L).astype(np.int32)
    table, nb = shuffled_table(4, B, TL)
    knew = synth.normal_f32(synth.rng(WID, synth.T_KNEW, 4), (B, D))
    vnew = synth.normal_f32(synth.rng(WID, synth.T_VNEW, 4), (B, D))
    kqn, ksn = oracle.quantize_rows(knew)
    vqn, vsn = oracle.quantize_rows(vnew)
    exp = [a.copy() for a in hk.arrays()]
    for b in range(B):
        n = int(lens[b])
        exp[0][b, n - 1], exp[1][b, n - 1], exp[2][b, n - 1], exp[3][b, n - 1] = kqn[b], ksn[b], vqn[b], vsn[b]
    qb = q_bits(WID, (B, Hq, D), 4)
    ref = oracle.decode_ref(qb, *exp, lens, W)
    kv_a = paged_from_host(hk, table, bs, nb)
    kv_b = paged_from_host(hk, table, bs, nb)
    q, seq, kn, vn = q_dev(qb), dev(lens), dev(knew), dev(vnew)
    out_a = m.mqa_decode_append_paged(q, kv_a, kn, vn, seq, int(lens.max()), W)
    m.kv_quantize_int8_paged(kn.view(B, 1, D), vn.view(B, 1, D), kv_b, dev(lens - 1))
    out_b = m.mqa_decode_paged(q, kv_b, seq, int(lens.max()), W)
    torch.cuda.synchronize()
    want = [block_copy_pool(a, table, bs, nb) for a in exp]
    for name, got, w in (("k", kv_a.k, want[0]), ("k_scale", kv_a.k_scale, want[1]), ("v", kv_a.v, want[2]),
                         ("v_scale", kv_a.v_scale, want[3])):
        assert got.cpu().numpy().tobytes() == w.tobytes(), f"pool {name} differs from the oracle encoding"
    assert float((out_a - out_b).abs().max()) <= 1e-6
    assert_decode_close(out_a, ref, 1e-4, f"append paged bs={bs} W={W}")


@pytest.mark.parametrize("bs,W", [(32, 0), (128, 256)])
def test_prefill_paged_matches_oracle(bs, W):
    import mqa_attention_int8_amd as m
    B, Hq, D, C = 2, 32, 128, 128
    P = np.array([300, 700], np.int32)
    L = int((P + C).max())
    TL = -(-L // bs)
    log(f"prefill paged: bs={bs} W={W}")
    hk = HostKV.seeded(WID, 5, B, TL * bs, D)
    table, nb = shuffled_table(5, B, TL)
    qb = q_bits(WID, (B, C, Hq, D), 5)
    ref = oracle.prefill_ref(qb, *hk.arrays(), P, W)
    kvp = paged_from_host(hk, table, bs, nb)
    q, pre = q_dev(qb), dev(P)
    out = m.mqa_prefill_chunk_paged(q, kvp, pre, int(P.max()), W)
    cont = m.mqa_prefill_chunk(q, hk.to_device(), pre, int(P.max()), W)
    torch.cuda.synchronize()
    assert float((out - cont).abs().max()) <= 1e-6, "paged and contiguous prefill differ"
    assert_prefill_close(out, ref, what=f"prefill paged bs={bs} W={W}")


def test_prefill_paged_ring():
    import mqa_attention_int8_amd as m
    B, Hq, D, C, W, bs, TL = 2, 16, 64, 64, 256, 32, 10
    P = np.array([900, 1301], np.int32)
    assert W + C - 1 <= TL * bs
    L = int((P + C).max())
    log(f"prefill ring: ring {TL * bs} W={W} C={C} P={P.tolist()}")
    k = synth.normal_f32(synth.rng(WID, synth.T_K, 6), (B, L, D))
    v = synth.normal_f32(synth.rng(WID, synth.T_V, 6), (B, L, D))
    kq, ks = oracle.quantize_rows(k)
    vq, vs = oracle.quantize_rows(v)
    table, nb = shuffled_table(6, B, TL)
    kvp = m.PagedKV.empty(nb, bs, D, dev(table))
    fill_ring(m, kvp, table, k, v, P + C, chunk=64)
    qb = q_bits(WID, (B, C, Hq, D), 6)
    out = m.mqa_prefill_chunk_paged(q_dev(qb), kvp, dev(P), int(P.max()), W)
    torch.cuda.synchronize()
    ref = oracle.prefill_ref(qb, kq, ks, vq, vs, P, W)
    assert_prefill_close(out, ref, what="prefill ring")
