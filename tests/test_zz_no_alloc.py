"""mqa_decode_noalloc (partition states in the library's static device array,
no workspace) against mqa_decode (the same kernels, states in a caller
workspace) and the oracle, on two calls in a row: the first with many
partitions per sequence, the second smaller, so the second reuses the array
the first left behind."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import HostKV, assert_decode_close, dev, log, q_bits, q_dev

pytestmark = pytest.mark.gpu


def one_call(wid, B, L, Hq, D, lens, window, what):
    import mqa_attention_int8_amd as m
    lens = np.asarray(lens, np.int32)
    need = m.mqa_decode_workspace_bytes(B, Hq, D, int(lens.max()), window)
    log(f"noalloc {what}: B={B} L={L} Hq={Hq} D={D} W={window}, partition states {need} B")
    hk = HostKV.seeded(wid, 0, B, L, D)
    kv = hk.to_device()
    qb = q_bits(wid, (B, Hq, D))
    q, seq = q_dev(qb), dev(lens)
    out_n = torch.full((B, Hq, D), float("nan"), device="cuda")
    m.mqa_decode_noalloc(q, kv, seq, int(lens.max()), window, out=out_n)
    out_w = m.mqa_decode(q, kv, seq, int(lens.max()), window)
    torch.cuda.synchronize()
    ref = oracle.decode_ref(qb, *hk.arrays(), lens, window)
    # same kernels; tiles are handed to waves dynamically, so sums may be ordered differently
    assert_decode_close(out_n, out_w.cpu().numpy().astype(np.float64), 1e-4, f"{what}: noalloc vs mqa_decode")
    assert_decode_close(out_n, ref, 1e-4, f"{what}: noalloc vs oracle")
    return need


def test_noalloc_two_calls_second_smaller():
    first = one_call(95, 16, 16384, 32, 128, synth.ragged_lens(synth.rng(95, synth.T_LENS), 16, 9000, 16384), 0,
                     "call 1")
    second = one_call(96, 4, 2048, 32, 128, [2048, 1500, 700, 1], 0, "call 2")
    assert first > second > 0
