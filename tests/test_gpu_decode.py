"""mqa_decode on the GPU against the oracle (max abs error <= 1e-4)."""
import numpy as np
import pytest
import torch

import mqa_attention_int8_amd as m
import oracle
import synth
from gpu_util import HostKV, assert_decode_close, log, q_bits, q_dev, dev

pytestmark = pytest.mark.gpu

TOL = 1e-4


def run_decode(q, kv, lens, max_len, window, scale=None, out=None):
    from mqa_attention_int8_amd import mqa_decode
    o = mqa_decode(q, kv, dev(np.asarray(lens, np.int32)), max_len, window, scale, out=out)
    torch.cuda.synchronize()
    return o


def case(wid, B, L, Hq, D, lens, window, max_len=None, scale=None, what=""):
    log(f"decode {what}: B={B} L={L} Hq={Hq} D={D} W={window}")
    hk = HostKV.seeded(wid, 0, B, L, D)
    qb = q_bits(wid, (B, Hq, D))
    kv = hk.to_device()
    lens = np.asarray(lens, np.int32)
    out = run_decode(q_dev(qb), kv, lens, int(lens.max()) if max_len is None else max_len, window,
                     scale)
    ref = oracle.decode_ref(qb, *hk.arrays(), lens, window,
                            None if scale is None else np.float32(scale))
    return assert_decode_close(out, ref, TOL, what)


def test_tiny_config():
    # 1 sequence, 8 query heads, D = 64, 256 keys, global
    case(1, 1, 256, 8, 64, [256], 0, what="tiny")


@pytest.mark.parametrize("window", [0, 1024])
def test_decode_config_full(window):
    # 64 sequences x 4096 keys, 32 heads, D = 128: global and window layers on one buffer
    case(2, 64, 4096, 32, 128, [4096] * 64, window, what=f"B64 L4096 W{window}")


@pytest.mark.parametrize("Hq,D", [(1, 64), (8, 128), (16, 64), (20, 128), (32, 64), (48, 128), (64, 128)])
def test_head_counts(Hq, D):
    lens = [1, 31, 32, 33, 100, 257, 700, 1000]
    case(60 + Hq, 8, 1000, Hq, D, lens, 0, what=f"Hq{Hq} D{D}")


@pytest.mark.parametrize("window", [1, 2, 31, 32, 33, 100, 999, 1000, 5000])
def test_windows_ragged(window):
    lens = [1, 2, 33, 64, 65, 511, 1000, 1777, 2048, 2049]
    case(70, len(lens), 2100, 32, 128, lens, window, what=f"ragged W{window}")


@pytest.mark.parametrize("window", [32, 64, 1024, 2048])
def test_full_windows_tiled_from_their_first_key(window):
    """A window of a multiple of 32 keys over a sequence at least that long is
    tiled from its first key (no partly visible tiles); shorter sequences
    keep 32-row-aligned tiles. Lengths on both sides of the switch."""
    W = window
    lens = [W - 1, W, W + 1, W + 17, W + 31, W + 32, W + 33, 3 * W + 5]
    case(79, len(lens), 3 * W + 64, 32, 128, lens, W, what=f"full window W{W}")


def test_empty_and_single():
    lens = [0, 1, 0, 2]
    case(71, 4, 64, 32, 128, lens, 0, max_len=64, what="empty/single")


def test_single_partition_and_many_partitions():
    # max_seq_len hints change the partition plan; the answer must not change
    lens = [300, 1200, 2500, 4000]
    for max_len in (4000, 4096, 9000):
        case(72, 4, 9000, 32, 128, lens, 0, max_len=max_len, what=f"hint {max_len}")
    case(72, 1, 9000, 32, 128, [64], 0, max_len=64, what="one partition")


def test_explicit_scale():
    case(73, 3, 600, 32, 128, [600, 17, 333], 0, scale=0.05, what="scale 0.05")


def test_minus_128_codes():
    B, L, Hq, D = 2, 300, 32, 128
    hk = HostKV.seeded(74, 0, B, L, D)
    hk.kq[:, ::7, ::3] = -128
    hk.vq[:, ::5, ::2] = -128
    qb = q_bits(74, (B, Hq, D))
    lens = np.array([300, 123], np.int32)
    out = run_decode(q_dev(qb), hk.to_device(), lens, 300, 0)
    ref = oracle.decode_ref(qb, *hk.arrays(), lens, 0)
    assert_decode_close(out, ref, TOL, "-128 codes")


def test_garbage_beyond_length_is_ignored():
    # rows past seq_len hold NaN scales and random codes; they must not leak in
    B, L, Hq, D = 3, 512, 32, 128
    hk = HostKV.seeded(75, 0, B, L, D)
    lens = np.array([100, 257, 511], np.int32)
    for b in range(B):
        hk.ks[b, lens[b]:] = np.nan
        hk.vs[b, lens[b]:] = np.nan
    qb = q_bits(75, (B, Hq, D))
    out = run_decode(q_dev(qb), hk.to_device(), lens, 512, 0)
    for b in range(B):
        hk.ks[b, lens[b]:] = 0
        hk.vs[b, lens[b]:] = 0
    ref = oracle.decode_ref(qb, *hk.arrays(), lens, 0)
    assert_decode_close(out, ref, TOL, "NaN beyond length")
    out_w = run_decode(q_dev(qb), hk.to_device(), lens, 512, 64)
    ref_w = oracle.decode_ref(qb, *hk.arrays(), lens, 64)
    assert_decode_close(out_w, ref_w, TOL, "window, zero-scale rows before window")


@pytest.fixture
def deterministic():
    """Fixed tile-to-wave assignment for the test, restored afterwards."""
    prev = m.mqa_set_deterministic(True)
    yield
    m.mqa_set_deterministic(prev)


def test_shared_buffer_equals_copied_buffer(deterministic):
    """Layers reading one shared buffer get exactly what they would from
    private copies (deterministic mode: bitwise)."""
    B, L, Hq, D = 8, 2048, 32, 128
    hk = HostKV.seeded(76, 0, B, L, D)
    kv = hk.to_device()
    from mqa_attention_int8_amd import KVView
    kv2 = KVView(kv.k.clone(), kv.v.clone(), kv.k_scale.clone(), kv.v_scale.clone())
    lens = synth.ragged_lens(synth.rng(76, synth.T_LENS), B, 1, L)
    for li, W in enumerate((0, 1024, 1024)):
        q = q_dev(q_bits(76, (B, Hq, D), li))
        a = run_decode(q, kv, lens, L, W)
        b = run_decode(q, kv2, lens, L, W)
        assert torch.equal(a, b)
        assert_decode_close(a, oracle.decode_ref(q_bits(76, (B, Hq, D), li), *hk.arrays(), np.asarray(lens, np.int32),
                                                 W), TOL, f"W={W}")


def test_repeatable_and_output_fully_written(deterministic):
    B, L, Hq, D = 16, 3000, 32, 128
    hk = HostKV.seeded(77, 0, B, L, D)
    kv = hk.to_device()
    lens = synth.ragged_lens(synth.rng(77, synth.T_LENS), B, 0, L)
    q = q_dev(q_bits(77, (B, Hq, D)))
    out = torch.full((B, Hq, D), float("nan"), device="cuda")
    a = run_decode(q, kv, lens, L, 0, out=out).clone()
    assert torch.isfinite(a).all()
    for _ in range(3):
        assert torch.equal(run_decode(q, kv, lens, L, 0), a)   # bitwise, run after run


def test_repeatable_across_entry_points(deterministic):
    """Deterministic mode covers the ragged, fused-append and allocation-free
    entry points too: each is bitwise repeatable, and all agree with the oracle."""
    B, L, Hq, D = 12, 4096, 32, 128
    hk = HostKV.seeded(78, 0, B, L, D)
    lens = np.asarray(synth.ragged_lens(synth.rng(78, synth.T_LENS), B, 1, L), np.int32)
    qb = q_bits(78, (B, Hq, D))
    q = q_dev(qb)
    kv = hk.to_device()
    seq = dev(lens)
    ref = oracle.decode_ref(qb, *hk.arrays(), lens, 0)
    for name, fn in (("ragged", lambda: m.mqa_decode_ragged(q, kv, seq, L, 0)),
                     ("noalloc", lambda: m.mqa_decode_noalloc(q, kv, seq, L, 0)),
                     ("window", lambda: m.mqa_decode(q, kv, seq, L, 1000))):
        a = fn().clone()
        b = fn()
        assert torch.equal(a, b), name
        if name != "window":
            assert_decode_close(a, ref, TOL, name)


def test_errors_are_reported():
    from mqa_attention_int8_amd import MQAError, KVView
    kv = KVView.empty(2, 64, 96)
    q = torch.zeros((2, 8, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(MQAError) as e:
        run_decode(q, kv, [4, 4], 64, 0)
    assert e.value.code == 3   # unsupported head_dim
    kv = KVView.empty(2, 64, 128)
    q = torch.zeros((2, 8, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(MQAError) as e:
        run_decode(q, kv, [4, 4], 65, 0)
    assert e.value.code == 2   # max_seq_len beyond the cache


def test_workspace_reused_across_calls_and_shapes():
    """One workspace serves many later calls of different shapes."""
    from mqa_attention_int8_amd import decode_workspace, mqa_decode
    B, L, Hq, D = 16, 8192, 32, 128
    hk = HostKV.seeded(78, 0, B, L, D)
    kv = hk.to_device()
    ws = decode_workspace(B, Hq, D, L, 0)
    assert ws is not None
    for it, (lens_hi, W) in enumerate(((L, 0), (5000, 0), (L, 1024), (3000, 77), (L, 0))):
        lens = synth.ragged_lens(synth.rng(78, synth.T_LENS, it), B, 1, lens_hi)
        qb = q_bits(78, (B, Hq, D), it)
        out = mqa_decode(q_dev(qb), kv, dev(lens), lens_hi, W, workspace=ws)
        torch.cuda.synchronize()
        ref = oracle.decode_ref(qb, *hk.arrays(), lens, W)
        assert_decode_close(out, ref, TOL, f"reuse call {it}")


# ---- extreme scales (the fp16 P'' = 2^(z - m) s_v path and its range guard) ----------------
#
# Bound used below, per output element: |gpu - ref| <= 1e-5 * A + 1e-6 * Vmax, where
# A = sum_j p_j |v_j| / l (the oracle applied to |V|) and Vmax = max visible |v_j|.
# Each weighted term carries the fp16 hi + lo split's 2^-22 relative error (or, below 2^-3 of
# the fp16 scale, an absolute 2^-25 against a largest P'' of at least 2^7) and fp32 sums;
# logits stay moderate in these cases, so their fp32 rounding adds ~1e-7 relative.

def scaled_rows(g, n, D, e_lo, e_hi):
    """n rows of N(0,1) fp32 values, row r multiplied by 2^e_r with e_r uniform in [e_lo, e_hi]."""
    x = synth.normal_f32(g, (n, D))
    e = g.integers(e_lo, e_hi, size=n, endpoint=True)
    return (x * np.exp2(e)[:, None]).astype(np.float32)


def scaled_case(wid, k_exp, v_exp, q_exp=None, what="", B=4, L=1500, Hq=32, D=128, window=0):
    lens = np.asarray([L, L - 1, 777, 33][:B], np.int32)
    kq = np.zeros((B, L, D), np.int8); vq = np.zeros((B, L, D), np.int8)
    ks = np.zeros((B, L), np.float32); vs = np.zeros((B, L), np.float32)
    gk, gv = synth.rng(wid, synth.T_K, 7), synth.rng(wid, synth.T_V, 7)
    for b in range(B):
        kq[b], ks[b] = oracle.quantize_rows(scaled_rows(gk, L, D, *k_exp))
        vq[b], vs[b] = oracle.quantize_rows(scaled_rows(gv, L, D, *v_exp))
    if q_exp is None:
        qb = q_bits(wid, (B, Hq, D))
    else:
        gq = synth.rng(wid, synth.T_Q, 7)
        qf = synth.normal_f32(gq, (B, Hq, D)) * np.exp2(gq.integers(q_exp[0], q_exp[1], size=(B, Hq, D), endpoint=True))
        qb = synth.f32_to_bf16_bits(qf.astype(np.float32))
    hk = HostKV(kq, ks, vq, vs)
    log(f"decode scales {what}: k 2^{k_exp} v 2^{v_exp} q {q_exp}")
    out = run_decode(q_dev(qb), hk.to_device(), lens, int(lens.max()), window)
    ref = oracle.decode_ref(qb, kq, ks, vq, vs, lens, window)
    ref_abs = oracle.decode_ref(qb, kq, ks, np.abs(vq), vs, lens, window)
    vmax = np.zeros(B)
    for b in range(B):
        j0 = max(0, int(lens[b]) - window) if window > 0 else 0
        if lens[b] > j0:
            vmax[b] = float(np.max(np.abs(vq[b, j0:lens[b]].astype(np.float64)) * vs[b, j0:lens[b], None]))
    g = out.detach().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    bound = 1e-5 * ref_abs + 1e-6 * vmax[:, None, None]
    excess = np.abs(g - ref) - bound
    rel = float(np.max(np.abs(g - ref) / np.maximum(ref_abs, 1e-300)))
    log(f"  {what}: worst |err| / A = {rel:.3e}, elements over the bound: {int((excess > 0).sum())}")
    assert np.all(excess <= 0), f"{what}: {int((excess > 0).sum())} elements outside the bound"


@pytest.mark.parametrize("v_exp", [(-40, 40), (90, 100), (-110, -100)])
def test_value_scales(v_exp):
    """Row scales of V spread over 2^80, or uniformly huge / tiny: the P'' range guard re-bases."""
    scaled_case(80, (0, 0), v_exp, what=f"v 2^{v_exp}")


def test_key_scales_spread():
    """Row scales of K spread by 2^4: logits differ strongly between keys."""
    scaled_case(81, (-2, 2), (-3, 3), what="k spread")


def test_query_dynamic_range():
    """q elements spread over 2^-30 .. 2^0 (the per-wave power-of-two q scaling)."""
    scaled_case(82, (0, 0), (0, 0), q_exp=(-30, 0), what="q spread")


def test_value_scales_window():
    scaled_case(83, (0, 0), (-40, 40), what="v spread, window 300", window=300)
