"""Full-size workloads in the launch configuration the benchmark uses.

Hybrid 6-layer block (ragged 1024..32768 keys, 3 shared buffers), long-context
decode (131072 keys, many partitions + merge) and prefill of a 512-token chunk
over an 8192-token prefix. Decode outputs are compared in full; prefill
outputs on sampled chunk positions the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import HostKV, assert_decode_close, assert_prefill_close, dev, log, q_bits, q_dev

pytestmark = pytest.mark.gpu


def test_hybrid_block_full():
    from mqa_attention_int8_amd import mqa_decode
    w = synth.HYBRID
    B, Hq, D = w.B, w.Hq, w.D
    lens = w.lens()
    L = int(lens.max())
    L_cap = (L + 31) // 32 * 32          # capacity: a multiple of 32 rows
    log(f"hybrid block: B={B} lens {lens.min()}..{lens.max()}")
    # global buffer: every visible row; window buffers: only their last 1024 rows
    bufs = {"G": HostKV.seeded(w.wid, 0, B, L_cap, D, rows=[(b, 0, int(n)) for b, n in enumerate(lens)])}
    for bid, name in ((1, "A"), (2, "Bf")):
        bufs[name] = HostKV.seeded(w.wid, bid, B, L_cap, D,
                                   rows=[(b, max(0, int(n) - 1024), int(n)) for b, n in enumerate(lens)])
    dv = {k: v.to_device() for k, v in bufs.items()}
    lens_d = dev(lens)
    for li, (name, window) in enumerate(w.layers):
        qb = q_bits(w.wid, (B, Hq, D), li)
        out = mqa_decode(q_dev(qb), dv[name], lens_d, L, window)
        torch.cuda.synchronize()
        ref = oracle.decode_ref(qb, *bufs[name].arrays(), lens, window)
        assert_decode_close(out, ref, 1e-4, f"layer {li} ({name}, W={window})")


def test_long_context_full():
    from mqa_attention_int8_amd import mqa_decode, mqa_decode_workspace_bytes
    w = synth.LONG
    B, Hq, D = w.B, w.Hq, w.D
    lens = w.lens()
    L = int(lens.max())
    log(f"long decode: B={B} L={L}; workspace {mqa_decode_workspace_bytes(B, Hq, D, L, 0)} B")
    hk = HostKV.seeded(w.wid, 0, B, L, D)
    qb = q_bits(w.wid, (B, Hq, D))
    out = mqa_decode(q_dev(qb), hk.to_device(), dev(lens), L, 0)
    torch.cuda.synchronize()
    ref = oracle.decode_ref(qb, *hk.arrays(), lens, 0)
    assert_decode_close(out, ref, 1e-4, "long context")


@pytest.mark.parametrize("window", [0, 1024])
def test_prefill_full_sampled(window):
    """Every chunk position of two sequences, and sampled positions of all
    the others (the full-size launch: 16 sequences, XCD-grouped order)."""
    from mqa_attention_int8_amd import mqa_prefill_chunk
    w = synth.PREFILL
    B, C, P, Hq, D = w.B, w.C, w.prefix, w.Hq, w.D
    L = P + C
    log(f"prefill full: B={B} C={C} prefix={P} W={window}")
    hk = HostKV.seeded(w.wid, 0, B, L, D)
    qb = q_bits(w.wid, (B, C, Hq, D))
    plens = np.full(B, P, np.int32)
    out = mqa_prefill_chunk(q_dev(qb), hk.to_device(), dev(plens), P, window)
    torch.cuda.synchronize()
    full = [0, 9]
    ref = oracle.prefill_ref(qb[full], *(a[full] for a in hk.arrays()), plens[full], window)
    assert_prefill_close(out[full], ref, what=f"sequences {full}, every position, W={window}")
    rest = [b for b in range(B) if b not in full]
    picks = [0, 1, 63, 64, 255, 256, 300, 510, 511]
    sub = oracle.prefill_ref(qb[rest], *(a[rest] for a in hk.arrays()), plens[rest], window,
                             positions=picks)
    assert_prefill_close(out[rest][:, picks], sub[:, picks], what=f"other sequences, sampled positions W={window}")
