"""Pins for the oracle's int8 KV encoding (CPU only).

The encoding's reading (symmetric per-row absmax/127, fp32 scale, round half to
even) is pinned by: hand-derived rows, a pure-Python coding of the same steps
with fp32 rounding done by ``struct``, numpy's native fp32 arithmetic, and the
invariants the definition implies.
"""
import math
import struct

import numpy as np
import pytest

import oracle
import synth
from _golden import quant_rows


def f32(x):
    return struct.unpack("<f", struct.pack("<f", x))[0]


def brute_quant_row(row):
    """Same definition, scalar Python: fp32 rounding via struct, ties-to-even via round()."""
    a = max(abs(float(v)) for v in row)
    s = f32(a / 127.0)
    if s == 0.0:
        return [0] * len(row), 0.0
    q = []
    for v in row:
        r = f32(float(v) / s)
        k = int(round(r))           # Python rounds half to even
        q.append(max(-127, min(127, k)))
    return q, s


@pytest.mark.parametrize("case", quant_rows())
def test_golden_rows(case):
    x, s_exp, q_exp = case
    q, s = oracle.quantize_rows(np.array([x], dtype=np.float32))
    assert s[0] == np.float32(s_exp)
    assert q[0].tolist() == q_exp


def test_matches_scalar_python_coding():
    g = synth.rng(900, 1)
    rows = synth.normal_f32(g, (400, 64))
    rows[::7] *= np.float32(1e-3)
    rows[::11] *= np.float32(3e4)
    q, s = oracle.quantize_rows(rows)
    for i in range(rows.shape[0]):
        qb, sb = brute_quant_row(rows[i].tolist())
        assert float(s[i]) == sb
        assert q[i].tolist() == qb


def test_matches_native_fp32_arithmetic():
    """numpy float32 ops are IEEE single ops: a second coding of the fp32 steps."""
    g = synth.rng(901, 1)
    rows = synth.normal_f32(g, (16384, 128))          # 2M values
    rows[:64] *= np.float32(1e-39)                      # subnormal scales
    rows[64:128] *= np.float32(1e-30)
    a = np.max(np.abs(rows), axis=1)
    s = a / np.float32(127.0)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = rows / s[:, None]
    qn = np.where((s > 0)[:, None], np.clip(np.rint(r), -127, 127), 0).astype(np.int8)
    q, so = oracle.quantize_rows(rows)
    assert np.array_equal(so.view(np.uint32), s.astype(np.float32).view(np.uint32))
    assert np.array_equal(q, qn)


def test_ties_round_to_even_in_seeded_data():
    """Exact .5 quotients do occur in N(0,1) data; each must go to the even code."""
    g = synth.rng(902, 1)
    rows = synth.normal_f32(g, (40000, 128))
    q, s = oracle.quantize_rows(rows)
    r = (rows.astype(np.float64) / s.astype(np.float64)[:, None]).astype(np.float32)
    frac = np.abs(r - np.trunc(r))
    ties = frac == np.float32(0.5)
    assert ties.sum() > 0
    assert np.all(q[ties] % 2 == 0)


def test_invariants():
    g = synth.rng(903, 1)
    rows = synth.normal_f32(g, (5000, 128))
    q, s = oracle.quantize_rows(rows)
    assert q.dtype == np.int8 and s.dtype == np.float32
    assert q.min() >= -127 and q.max() <= 127
    am = np.argmax(np.abs(rows), axis=1)
    picked = q[np.arange(len(q)), am]
    assert np.all(np.abs(picked) == 127)
    assert np.all(np.sign(picked) == np.sign(rows[np.arange(len(q)), am]))
    err = np.abs(rows.astype(np.float64) - q.astype(np.float64) * s.astype(np.float64)[:, None])
    bound = s.astype(np.float64)[:, None] * (0.5 + 127 * 2.0 ** -24)
    assert np.all(err <= bound)


def test_zero_and_underflow_rows():
    z = np.zeros((1, 64), np.float32)
    q, s = oracle.quantize_rows(z)
    assert s[0] == 0 and not q.any()
    tiny = np.zeros((1, 64), np.float32)
    tiny[0, 3] = np.float32(np.ldexp(63.0, -149))       # a/127 rounds to zero
    q, s = oracle.quantize_rows(tiny)
    assert s[0] == 0 and not q.any()
    tiny[0, 3] = np.float32(np.ldexp(64.0, -149))       # a/127 rounds to the smallest subnormal
    q, s = oracle.quantize_rows(tiny)
    assert s[0] == np.float32(np.ldexp(1.0, -149))
    assert q[0, 3] == 64 and np.count_nonzero(q) == 1   # 64*2^-149 / 2^-149 = 64


def test_dequantize_exact():
    q = np.array([[-128, -127, 0, 1, 127]], np.int8)
    s = np.array([np.float32(0.1)], np.float32)
    xh = oracle.dequantize_rows(q, s)
    assert xh.tolist()[0] == [v * float(np.float32(0.1)) for v in (-128, -127, 0, 1, 127)]


def test_non_finite_rejected():
    with pytest.raises(ValueError):
        oracle.quantize_rows(np.array([[1.0, np.inf]], np.float32))


def test_bf16_bits_exact():
    bits = synth.f32_to_bf16_bits(np.array([1.0, -2.5, 3.140625, 1e-40], np.float32))
    vals = oracle.bf16_bits_to_f64(bits)
    assert vals[0] == 1.0 and vals[1] == -2.5 and vals[2] == 3.140625
    assert vals[3] == math.ldexp(1.0, -133)   # nearest bf16 subnormal to 1e-40
