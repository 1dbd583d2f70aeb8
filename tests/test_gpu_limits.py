"""The largest batch the ABI accepts (65535 sequences: one grid dimension of
the decode, merge and prefill staging launches) on the GPU, with short
ragged sequences, against the oracle on sampled sequences (every sequence
is independent, so any sample is a full check of the ones it holds), and the
first batch size past the limit rejected before any launch.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_decode_close, assert_prefill_close, dev, log, pad_rows, q_bits, q_dev

pytestmark = pytest.mark.gpu

BMAX = 65535


def cache(wid, B, L, D, cap=32):
    """int8 cache with `cap` rows per sequence (a multiple of 32), the first L
    of them filled: one quantizer call for all rows."""
    kq, ks = oracle.quantize_rows(synth.normal_f32(synth.rng(wid, synth.T_K), (B * L, D)))
    vq, vs = oracle.quantize_rows(synth.normal_f32(synth.rng(wid, synth.T_V), (B * L, D)))
    return tuple(pad_rows(a, cap) for a in (kq.reshape(B, L, D), ks.reshape(B, L), vq.reshape(B, L, D),
                                            vs.reshape(B, L)))


def sample(B, n, seed):
    g = synth.rng(seed, 9)
    return np.unique(np.concatenate([[0, 1, B // 2, B - 2, B - 1], g.integers(0, B, size=n)])).astype(np.int64)


@pytest.mark.parametrize("window", [0, 3])
def test_decode_at_the_largest_batch(window):
    import mqa_attention_int8_amd as m
    B, Hq, D, L = BMAX, 8, 64, 8
    lens = synth.ragged_lens(synth.rng(61, synth.T_LENS), B, 0, L)
    log(f"decode B={B} Hq={Hq} D={D} lens 0..{L} W={window}")
    arrs = cache(61, B, L, D)
    qb = q_bits(61, (B, Hq, D))
    kv = m.KVView(dev(arrs[0]), dev(arrs[2]), dev(arrs[1]), dev(arrs[3]))
    out = m.mqa_decode(q_dev(qb), kv, dev(lens), L, window)
    torch.cuda.synchronize()
    bs = sample(B, 200, 62)
    picks = [(int(b), h) for b in bs for h in range(Hq)]
    ref = oracle.decode_ref_rows(qb, *arrs, lens, window, picks).reshape(len(bs), Hq, D)
    assert_decode_close(out[torch.from_numpy(bs).cuda()], ref, 1e-4, f"{len(bs)} sampled sequences")
    with pytest.raises(m.MQAError) as err:
        m.mqa_decode(q_dev(q_bits(61, (B + 1, Hq, D))), m.KVView.empty(B + 1, 32, D), dev(np.zeros(B + 1, np.int32)),
                     L, window)
    assert err.value.code == 2  # MQA_ERR_SHAPE, before any launch


@pytest.mark.parametrize("window", [0, 2])
def test_prefill_at_the_largest_batch(window):
    import mqa_attention_int8_amd as m
    B, C, Hq, D = BMAX, 2, 8, 64
    plens = synth.ragged_lens(synth.rng(63, synth.T_LENS), B, 0, 5)
    L = 8
    log(f"prefill B={B} C={C} Hq={Hq} D={D} prefixes 0..5 W={window}")
    arrs = cache(63, B, L, D)
    qb = q_bits(63, (B, C, Hq, D))
    kv = m.KVView(dev(arrs[0]), dev(arrs[2]), dev(arrs[1]), dev(arrs[3]))
    out = m.mqa_prefill_chunk(q_dev(qb), kv, dev(plens), 5, window)
    torch.cuda.synchronize()
    bs = sample(B, 100, 64)
    ref = oracle.prefill_ref(qb[bs], *(a[bs] for a in arrs), plens[bs], window)
    assert_prefill_close(out[torch.from_numpy(bs).cuda()], ref, what=f"{len(bs)} sampled sequences")
