"""mqa_decode_append (fused append of the new token + decode) on the GPU.

Checks, on the same seeded inputs: the cache rows it writes are bit-identical
to the oracle quantizer's encoding of k_new / v_new (and to kv_quantize_int8's),
the rest of the cache is untouched, the output equals that of the separate
kv_quantize_int8 x 2 + mqa_decode sequence up to summation order (1e-6), and
it matches the oracle (decode on the cache with the oracle-encoded new row)
within 1e-4.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import HostKV, assert_decode_close, dev, log, q_bits, q_dev

pytestmark = pytest.mark.gpu

T_KNEW, T_VNEW = synth.T_KNEW, synth.T_VNEW


def clone(kv):
    from mqa_attention_int8_amd import KVView
    return KVView(kv.k.clone(), kv.v.clone(), kv.k_scale.clone(), kv.v_scale.clone())


def run_case(wid, B, L, Hq, D, lens, window, what):
    import mqa_attention_int8_amd as m
    lens = np.asarray(lens, np.int32)
    log(f"append {what}: B={B} L={L} Hq={Hq} D={D} W={window}")
    # cache rows before the new token: oracle-encoded N(0,1); the slot of the new row holds other bytes
    hk = HostKV.seeded(wid, 0, B, L, D)
    knew = synth.normal_f32(synth.rng(wid, T_KNEW, 0), (B, D))
    vnew = synth.normal_f32(synth.rng(wid, T_VNEW, 0), (B, D))
    qb = q_bits(wid, (B, Hq, D))
    # expected cache: row n - 1 replaced by the oracle encoding of the new rows
    kq_new, ks_new = oracle.quantize_rows(knew)
    vq_new, vs_new = oracle.quantize_rows(vnew)
    exp = [a.copy() for a in hk.arrays()]
    for b in range(B):
        n = int(lens[b])
        if n > 0:
            exp[0][b, n - 1], exp[1][b, n - 1] = kq_new[b], ks_new[b]
            exp[2][b, n - 1], exp[3][b, n - 1] = vq_new[b], vs_new[b]
    ref = oracle.decode_ref(qb, *exp, lens, window)

    kv_a = hk.to_device()
    kv_b = clone(kv_a)
    q = q_dev(qb)
    seq = dev(lens)
    kn, vn = dev(knew), dev(vnew)
    out_a = m.mqa_decode_append(q, kv_a, kn, vn, seq, int(lens.max()), window)
    # the same step as separate calls: quantize K, quantize V, decode
    start = dev(np.maximum(lens - 1, 0).astype(np.int32))
    has = lens > 0
    if has.all():
        m.kv_quantize_int8(kn.view(B, 1, D), kv_b.k, kv_b.k_scale, start)
        m.kv_quantize_int8(vn.view(B, 1, D), kv_b.v, kv_b.v_scale, start)
    else:  # sequences without a token get no row: quantize only the others
        for b in np.nonzero(has)[0]:
            sb = start[b:b + 1]
            m.kv_quantize_int8(kn[b:b + 1].view(1, 1, D), kv_b.k[b:b + 1], kv_b.k_scale[b:b + 1], sb)
            m.kv_quantize_int8(vn[b:b + 1].view(1, 1, D), kv_b.v[b:b + 1], kv_b.v_scale[b:b + 1], sb)
    out_b = m.mqa_decode(q, kv_b, seq, int(lens.max()), window)
    torch.cuda.synchronize()
    for name, got, want in (("k", kv_a.k, exp[0]), ("k_scale", kv_a.k_scale, exp[1]),
                            ("v", kv_a.v, exp[2]), ("v_scale", kv_a.v_scale, exp[3])):
        g = got.cpu().numpy()
        assert g.view(np.uint8).tobytes() == np.ascontiguousarray(want).view(np.uint8).tobytes(), \
            f"{what}: cache {name} differs from the oracle encoding"
    for name in ("k", "v", "k_scale", "v_scale"):
        assert torch.equal(getattr(kv_a, name), getattr(kv_b, name)), f"{what}: cache {name} differs from kv_quantize_int8"
    # same arithmetic; tiles are handed out to waves dynamically, so sums may be ordered differently
    assert float((out_a - out_b).abs().max()) <= 1e-6, f"{what}: fused output differs from the separate calls"
    assert_decode_close(out_a, ref, 1e-4, what)


@pytest.mark.parametrize("window", [0, 100, 64, 1024])
def test_append_ragged(window):
    lens = [1, 2, 31, 32, 33, 500, 999, 1000]
    run_case(90, 8, 1000, 32, 128, lens, window, f"ragged W{window}")


@pytest.mark.parametrize("Hq,D", [(8, 64), (48, 128), (64, 128)])
def test_append_heads(Hq, D):
    run_case(91, 4, 300, Hq, D, [300, 299, 64, 65], 0, f"Hq{Hq} D{D}")


def test_append_empty_sequences():
    run_case(92, 4, 128, 32, 128, [0, 5, 0, 128], 0, "with empty sequences")


@pytest.mark.parametrize("window", [0, 1024])
def test_append_decode_config(window):
    # 64 sequences x 4096 keys (the new token is key 4095), 32 heads, D = 128
    run_case(93, 64, 4096, 32, 128, [4096] * 64, window, f"B64 L4096 W{window}")
