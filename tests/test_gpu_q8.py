"""mqa_decode_q8 / mqa_decode_append_q8 (int8 queries, int8 MFMA for Q K^T)
on the GPU against the oracle's int8-query decode (max abs error <= 1e-4).

The int8 queries are the oracle quantizer's encoding of the seeded bf16
queries; kv_quantize_int8 applied to the same fp32 query rows must give those
codes bit for bit (the documented way to make the input).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import HostKV, assert_decode_close, dev, log, q_bits

pytestmark = pytest.mark.gpu

WID = 61


def q8_case(seed, B, Hq, D):
    qb = q_bits(WID, (B, Hq, D), seed)
    qf = oracle.bf16_bits_to_f64(qb).astype(np.float32)
    q8, qs = oracle.quantize_rows(qf)
    return qf, q8, qs


@pytest.mark.parametrize("D,Hq,W", [(128, 32, 0), (128, 32, 1024), (128, 8, 100), (64, 16, 0), (128, 64, 0),
                                    (64, 48, 256)])
def test_decode_q8_matches_oracle(D, Hq, W):
    import mqa_attention_int8_amd as m
    B, L = 4, 1500
    log(f"decode q8: D={D} Hq={Hq} W={W}")
    hk = HostKV.seeded(WID, 1, B, L, D)
    lens = synth.ragged_lens(synth.rng(WID, synth.T_LENS, 1), B, 1, L).astype(np.int32)
    lens[0] = L
    qf, q8, qs = q8_case(1, B, Hq, D)
    ref = oracle.decode_ref_q8(q8, qs, *hk.arrays(), lens, W)
    out = m.mqa_decode_q8(dev(q8), dev(qs), hk.to_device(), dev(lens), L, W)
    torch.cuda.synchronize()
    assert_decode_close(out, ref, 1e-4, f"q8 D={D} Hq={Hq} W={W}")


def test_query_encoding_with_kv_quantize():
    import mqa_attention_int8_amd as m
    B, Hq, D = 5, 32, 128
    qf, q8, qs = q8_case(2, B, Hq, D)
    codes = torch.zeros((B, Hq, D), dtype=torch.int8, device="cuda")
    scales = torch.zeros((B, Hq), dtype=torch.float32, device="cuda")
    m.kv_quantize_int8(dev(qf), codes, scales, torch.zeros(B, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert codes.cpu().numpy().tobytes() == q8.tobytes()
    assert scales.cpu().numpy().tobytes() == qs.tobytes()


@pytest.mark.parametrize("W", [0, 100])
def test_decode_append_q8(W):
    import mqa_attention_int8_amd as m
    from mqa_attention_int8_amd import KVView
    B, Hq, D, L = 4, 32, 128, 900
    log(f"append q8: W={W}")
    hk = HostKV.seeded(WID, 3, B, L, D)
    lens = synth.ragged_lens(synth.rng(WID, synth.T_LENS, 3), B, 1, L).astype(np.int32)
    knew = synth.normal_f32(synth.rng(WID, synth.T_KNEW, 3), (B, D))
    vnew = synth.normal_f32(synth.rng(WID, synth.T_VNEW, 3), (B, D))
    kqn, ksn = oracle.quantize_rows(knew)
    vqn, vsn = oracle.quantize_rows(vnew)
    exp = [a.copy() for a in hk.arrays()]
    for b in range(B):
        n = int(lens[b])
        exp[0][b, n - 1], exp[1][b, n - 1], exp[2][b, n - 1], exp[3][b, n - 1] = kqn[b], ksn[b], vqn[b], vsn[b]
    qf, q8, qs = q8_case(3, B, Hq, D)
    ref = oracle.decode_ref_q8(q8, qs, *exp, lens, W)
    kv_a = hk.to_device()
    kv_b = KVView(kv_a.k.clone(), kv_a.v.clone(), kv_a.k_scale.clone(), kv_a.v_scale.clone())
    q8d, qsd, seq = dev(q8), dev(qs), dev(lens)
    kn, vn = dev(knew), dev(vnew)
    out_a = m.mqa_decode_append_q8(q8d, qsd, kv_a, kn, vn, seq, L, W)
    start = dev(lens - 1)
    m.kv_quantize_int8(kn.view(B, 1, D), kv_b.k, kv_b.k_scale, start)
    m.kv_quantize_int8(vn.view(B, 1, D), kv_b.v, kv_b.v_scale, start)
    out_b = m.mqa_decode_q8(q8d, qsd, kv_b, seq, L, W)
    torch.cuda.synchronize()
    for name in ("k", "v", "k_scale", "v_scale"):
        assert torch.equal(getattr(kv_a, name), getattr(kv_b, name)), name
    assert float((out_a - out_b).abs().max()) <= 1e-6
    assert_decode_close(out_a, ref, 1e-4, f"append q8 W={W}")
