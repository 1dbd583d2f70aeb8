"""mqa_prefill_chunk on the GPU against the oracle (|gpu-ref| <= 5e-3 + 1e-2|ref|)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import HostKV, assert_prefill_close, assert_decode_close, dev, log, q_bits, q_dev

pytestmark = pytest.mark.gpu


def run_prefill(q, kv, plens, max_p, window, scale=None):
    from mqa_attention_int8_amd import mqa_prefill_chunk
    o = mqa_prefill_chunk(q, kv, dev(np.asarray(plens, np.int32)), max_p, window, scale)
    torch.cuda.synchronize()
    return o


def case(wid, B, C, Hq, D, plens, window, L=None, what=""):
    plens = np.asarray(plens, np.int32)
    L = int(plens.max()) + C if L is None else L
    log(f"prefill {what}: B={B} C={C} Hq={Hq} D={D} prefix={plens.tolist()} W={window}")
    hk = HostKV.seeded(wid, 0, B, L, D)
    qb = q_bits(wid, (B, C, Hq, D))
    out = run_prefill(q_dev(qb), hk.to_device(), plens, int(plens.max()), window)
    ref = oracle.prefill_ref(qb, *hk.arrays(), plens, window)
    return assert_prefill_close(out, ref, what=what)


@pytest.mark.parametrize("window", [0, 64, 1024])
def test_small_ragged(window):
    case(80, 3, 100, 32, 128, [0, 37, 300], window, what=f"small W{window}")


@pytest.mark.parametrize("Hq,D", [(8, 64), (1, 128), (20, 128), (64, 64)])
def test_head_counts(Hq, D):
    case(81, 2, 77, Hq, D, [5, 130], 0, what=f"Hq{Hq} D{D}")
    case(81, 2, 77, Hq, D, [5, 130], 16, what=f"Hq{Hq} D{D} W16")


@pytest.mark.parametrize("window", [1, 2, 63, 65])
def test_tiny_windows(window):
    case(82, 2, 70, 32, 128, [3, 200], window, what=f"W{window}")


def test_chunk_of_one_matches_decode():
    from mqa_attention_int8_amd import mqa_decode
    B, L, Hq, D = 4, 700, 32, 128
    hk = HostKV.seeded(83, 0, B, L, D)
    kv = hk.to_device()
    lens = np.array([700, 1, 64, 333], np.int32)
    qb = q_bits(83, (B, Hq, D))
    for W in (0, 100):
        pre = run_prefill(q_dev(qb[:, None]), kv, lens - 1, int(lens.max()) - 1, W)
        dec = mqa_decode(q_dev(qb), kv, dev(lens), int(lens.max()), W)
        ref = oracle.decode_ref(qb, *hk.arrays(), lens, W)
        assert_decode_close(dec, ref, 1e-4, f"decode W{W}")
        assert_prefill_close(pre[:, 0], ref, what=f"prefill C=1 W{W}")


def test_causality_on_gpu():
    B, C, Hq, D, P = 1, 96, 32, 128, 40
    L = P + C
    hk = HostKV.seeded(84, 0, B, L, D)
    qb = q_bits(84, (B, C, Hq, D))
    a = run_prefill(q_dev(qb), hk.to_device(), [P], P, 0).cpu()
    hk.kq[0, P + 50:] = -hk.kq[0, P + 50:]
    hk.vq[0, P + 50:] = 127
    b = run_prefill(q_dev(qb), hk.to_device(), [P], P, 0).cpu()
    assert torch.equal(a[0, :50], b[0, :50])
    assert not torch.equal(a[0, 50:], b[0, 50:])
