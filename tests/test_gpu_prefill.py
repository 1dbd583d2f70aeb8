"""mqa_prefill_chunk on the GPU against the oracle (|gpu-ref| <= 5e-3 + 1e-2|ref|)."""
import numpy as np
import pytest
import torch

import oracle
import synth
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


def test_batch_multiple_of_eight_full():
    """B = 8: the work-group order that keeps each sequence on one XCD."""
    for window in (0, 200):
        case(85, 8, 64, 32, 128, [0, 1, 63, 64, 500, 777, 1024, 1500], window, what=f"B8 W{window}")


def test_minus_128_codes():
    """Codes the encoder never writes (-128) are still read as -128."""
    B, C, Hq, D, P = 2, 80, 32, 128, 150
    hk = HostKV.seeded(86, 0, B, P + C, D)
    hk.kq[:, ::7, ::3] = -128
    hk.vq[:, 1::5, ::2] = -128
    qb = q_bits(86, (B, C, Hq, D))
    plens = np.array([P, 40], np.int32)
    for window in (0, 90):
        log(f"prefill -128 codes W={window}")
        out = run_prefill(q_dev(qb), hk.to_device(), plens, P, window)
        ref = oracle.prefill_ref(qb, *hk.arrays(), plens, window)
        assert_prefill_close(out, ref, what=f"-128 W{window}")


# ---- extreme K/V scales -----------------------------------------------------------------------
#
# Bound per output element: |gpu - ref| <= 4e-3 * A + 1e-6 * Vmax, with A = sum_j p_j |v_j| / l
# (the oracle applied to |V|) and Vmax the largest visible |v_j|. Derivation: P = 2^(z - m) and
# V'' = v s_v 2^-E are each rounded to fp16 (2^-11 relative, so ~1e-3 of A together; the row
# sums use the same rounded P); a V'' below fp16's range flushes to at most 2^-25 * 2^E, and
# 2^E <= 2 * max s_v <= Vmax / 63.5; logits are exact products summed in fp32.

def scaled_rows(g, n, D, e_lo, e_hi):
    x = synth.normal_f32(g, (n, D))
    e = g.integers(e_lo, e_hi, size=n, endpoint=True)
    return (x * np.exp2(e)[:, None]).astype(np.float32)


def scaled_prefill(wid, k_exp, v_exp, window, what, B=2, C=96, Hq=32, D=128, plens=(300, 41)):
    plens = np.asarray(plens, np.int32)
    L = int(plens.max()) + C
    kq = np.zeros((B, L, D), np.int8); vq = np.zeros((B, L, D), np.int8)
    ks = np.zeros((B, L), np.float32); vs = np.zeros((B, L), np.float32)
    gk, gv = synth.rng(wid, synth.T_K, 9), synth.rng(wid, synth.T_V, 9)
    for b in range(B):
        kq[b], ks[b] = oracle.quantize_rows(scaled_rows(gk, L, D, *k_exp))
        vq[b], vs[b] = oracle.quantize_rows(scaled_rows(gv, L, D, *v_exp))
    hk = HostKV(kq, ks, vq, vs)
    qb = q_bits(wid, (B, C, Hq, D))
    log(f"prefill scales {what}: k 2^{k_exp} v 2^{v_exp} W={window}")
    out = run_prefill(q_dev(qb), hk.to_device(), plens, int(plens.max()), window)
    ref = oracle.prefill_ref(qb, kq, ks, vq, vs, plens, window)
    ref_abs = oracle.prefill_ref(qb, kq, ks, np.abs(vq), vs, plens, window)
    vmax = np.zeros((B, C))
    for b in range(B):
        for i in range(C):
            lo, hi = oracle.prefill_visible(int(plens[b]) + i, window)
            vmax[b, i] = float(np.max(np.abs(vq[b, lo:hi].astype(np.float64)) * vs[b, lo:hi, None]))
    g = out.detach().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    bound = 4e-3 * ref_abs + 1e-6 * vmax[:, :, None, None]
    excess = np.abs(g - ref) - bound
    rel = float(np.max(np.abs(g - ref) / np.maximum(ref_abs, 1e-300)))
    log(f"  {what}: worst |err| / A = {rel:.3e}, elements over the bound: {int((excess > 0).sum())}")
    assert np.all(excess <= 0), f"{what}: {int((excess > 0).sum())} elements outside the bound"


@pytest.mark.parametrize("v_exp", [(-40, 40), (90, 100), (-110, -100)])
@pytest.mark.parametrize("window", [0, 70])
def test_prefill_value_scales(v_exp, window):
    scaled_prefill(87, (0, 0), v_exp, window, what=f"v 2^{v_exp}")


def test_prefill_key_scales_spread():
    scaled_prefill(88, (-2, 2), (-3, 3), 0, what="k spread")


def test_window_ignores_large_value_before_its_start():
    """A key no query of the chunk sees (just before the first query's window
    start) with a V scale 2^12 times the others must not reach the output."""
    B, C, Hq, D, P, W = 1, 16, 32, 128, 100, 64
    hk = HostKV.seeded(89, 0, B, P + C, D)
    first = P - W + 1                          # first key the first query sees
    hk.vs[0, first - 1] *= np.float32(4096.0)  # exact: a power-of-two rescale of the row's scale
    qb = q_bits(89, (B, C, Hq, D))
    out = run_prefill(q_dev(qb), hk.to_device(), [P], P, W)
    ref = oracle.prefill_ref(qb, *hk.arrays(), np.array([P], np.int32), W)
    assert_prefill_close(out, ref, what="large V before the window")
