"""kv_quantize_int8 on the GPU: bit-exact against the oracle's encoding."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import dev, log

pytestmark = pytest.mark.gpu


def run_quant(src: np.ndarray, L_cap: int, start: np.ndarray):
    from mqa_attention_int8_amd import kv_quantize_int8
    B, T, D = src.shape
    dst = torch.full((B, L_cap, D), 99, dtype=torch.int8, device="cuda")
    dsc = torch.full((B, L_cap), -7.0, dtype=torch.float32, device="cuda")
    kv_quantize_int8(dev(src), dst, dsc, dev(start.astype(np.int32)))
    torch.cuda.synchronize()
    return dst.cpu().numpy(), dsc.cpu().numpy()


def check(src, L_cap, start, what):
    log(f"quantize {what}: src {src.shape} L_cap {L_cap}")
    q, s = run_quant(src, L_cap, start)
    qr, sr = oracle.quantize_rows(src)
    B, T, D = src.shape
    for b in range(B):
        p0 = int(start[b])
        lo, hi = max(p0, 0), min(p0 + T, L_cap)
        assert np.array_equal(q[b, lo:hi], qr[b, lo - p0:hi - p0]), f"codes differ, seq {b}"
        assert np.array_equal(s[b, lo:hi].view(np.uint32), sr[b, lo - p0:hi - p0].view(np.uint32)), \
            f"scales differ, seq {b}"
        untouched = np.ones(L_cap, bool)
        untouched[lo:hi] = False
        assert np.all(q[b, untouched] == 99) and np.all(s[b, untouched] == -7.0)


@pytest.mark.parametrize("D", [64, 128])
def test_decode_write_shape(D):
    # one new token per sequence (decode step), 64 sequences
    src = synth.normal_f32(synth.rng(2, synth.T_KNEW, D), (64, 1, D))
    start = synth.ragged_lens(synth.rng(2, synth.T_LENS, 77), 64, 0, 4095)
    check(src, 4096, start, f"decode write D={D}")


def test_prefill_write_shape():
    # a 512-token chunk after an 8192-token prefix, 16 sequences
    src = synth.normal_f32(synth.rng(4, synth.T_KNEW), (16, 512, 128))
    check(src, 8704, np.full(16, 8192), "prefill chunk write")


def test_edge_rows_bit_exact():
    D = 128
    g = synth.rng(950, 1)
    rows = synth.normal_f32(g, (64, D))
    rows[0] = 0.0                                     # zero row -> scale 0
    rows[1] = 0.0
    rows[1, 5] = np.float32(np.ldexp(63.0, -149))     # absmax/127 underflows to 0
    rows[2] = 0.0
    rows[2, 9] = np.float32(np.ldexp(64.0, -149))     # smallest subnormal scale
    rows[3] *= np.float32(1e-39)                      # subnormal inputs
    rows[4] = np.float32(127.0)
    rows[4, :8] = [127, 2.5, -2.5, 3.5, 0.5, 1.5, -0.5, -127]   # ties to even with s = 1
    rows[5] *= np.float32(3e37)                       # large magnitudes
    rows[6, :] = -3.0                                 # constant negative row
    src = rows.reshape(4, 16, D)
    check(src, 40, np.array([0, 3, 24, 10]), "edge rows")


def test_seeded_ties_bit_exact():
    # many rows: exact .5 quotients occur and must round to even
    src = synth.normal_f32(synth.rng(951, 1), (8, 4096, 128))
    q, s = run_quant(src, 4096, np.zeros(8, np.int32))
    qr, sr = oracle.quantize_rows(src)
    assert np.array_equal(q, qr)
    assert np.array_equal(s.view(np.uint32), sr.view(np.uint32))


def test_out_of_range_rows_are_skipped():
    src = synth.normal_f32(synth.rng(952, 1), (3, 8, 64))
    check(src, 20, np.array([-3, 16, 20]), "clipped rows")
