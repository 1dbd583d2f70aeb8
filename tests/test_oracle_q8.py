"""Pins for the oracle's int8-query decode (CPU only)."""
import math

import numpy as np

import oracle
import synth


def small_case(seed, B=2, L=40, Hq=3, D=16):
    qf = synth.normal_f32(synth.rng(950 + seed, 1), (B, Hq, D))
    q8, qs = oracle.quantize_rows(qf)
    kq, ks = oracle.quantize_rows(synth.normal_f32(synth.rng(950 + seed, 2), (B, L, D)))
    vq, vs = oracle.quantize_rows(synth.normal_f32(synth.rng(950 + seed, 3), (B, L, D)))
    lens = np.array([L, 17], np.int32)[:B]
    return q8, qs, kq, ks, vq, vs, lens


def test_integer_dot_products_brute_force():
    """Scalar loops over the integer form: logit = sigma * s_q * s_k * sum of
    int8 products (exact Python ints), math.exp, math.fsum."""
    q8, qs, kq, ks, vq, vs, lens = small_case(0)
    B, Hq, D = q8.shape
    sigma = float(np.float32(1.0 / math.sqrt(D)))
    for window in (0, 9):
        got = oracle.decode_ref_q8(q8, qs, kq, ks, vq, vs, lens, window)
        for b in range(B):
            n = int(lens[b])
            lo = max(0, n - window) if window > 0 else 0
            for h in range(Hq):
                z = []
                for j in range(lo, n):
                    dot = sum(int(q8[b, h, d]) * int(kq[b, j, d]) for d in range(D))
                    z.append(sigma * float(qs[b, h]) * float(ks[b, j]) * dot)
                m = max(z)
                w = [math.exp(x - m) for x in z]
                tot = math.fsum(w)
                for d in range(D):
                    ref = math.fsum(w[i] * int(vq[b, lo + i, d]) * float(vs[b, lo + i]) for i in range(len(w))) / tot
                    assert abs(got[b, h, d] - ref) <= 1e-12


def test_exactly_representable_queries_match_bf16_path():
    """Queries that are integers times 2^-7 (|integer| <= 127, one row reaching
    127) are exact in bf16 and encode with scale 2^-7 and those integers, so
    the int8-query decode equals the bf16 decode."""
    B, Hq, D, L = 2, 4, 32, 50
    ints = synth.rng(951, 1).integers(-127, 128, size=(B, Hq, D))
    ints[..., 0] = 127
    qf = (ints * 2.0 ** -7).astype(np.float32)
    q8, qs = oracle.quantize_rows(qf)
    assert np.array_equal(q8, ints) and np.all(qs == np.float32(2.0 ** -7))
    qbits = synth.f32_to_bf16_bits(qf)
    kq, ks = oracle.quantize_rows(synth.normal_f32(synth.rng(951, 2), (B, L, D)))
    vq, vs = oracle.quantize_rows(synth.normal_f32(synth.rng(951, 3), (B, L, D)))
    lens = np.array([L, 23], np.int32)
    for window in (0, 10):
        a = oracle.decode_ref_q8(q8, qs, kq, ks, vq, vs, lens, window)
        r = oracle.decode_ref(qbits, kq, ks, vq, vs, lens, window)
        assert np.max(np.abs(a - r)) <= 1e-13
