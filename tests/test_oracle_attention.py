"""Pins for the oracle's attention (CPU only).

Each pin checks the oracle against something other than itself: scalar
brute force, a library attention routine, closed forms and invariants that
the definition implies, and values the pages print.
"""
import math
import struct

import numpy as np
import pytest
import torch

import oracle
import synth
from _golden import kv_bytes


def bf16_to_float(bits):
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def make_case(seed, B, L, Hq, D, lens=None):
    g = synth.rng(700 + seed, 1)
    q = synth.q_bf16(g, (B, Hq, D))
    k = synth.normal_f32(synth.rng(700 + seed, 2), (B, L, D))
    v = synth.normal_f32(synth.rng(700 + seed, 3), (B, L, D))
    kq, ks = oracle.quantize_rows(k)
    vq, vs = oracle.quantize_rows(v)
    if lens is None:
        lens = synth.ragged_lens(synth.rng(700 + seed, 4), B, 1, L)
    return q, kq, ks, vq, vs, np.asarray(lens, np.int32)


# ---------------------------------------------------------------------------
# brute force: scalar Python loops, math.fsum / math.exp
# ---------------------------------------------------------------------------

def brute_decode(q, kq, ks, vq, vs, lens, window, sigma):
    B, Hq, D = q.shape
    out = np.zeros((B, Hq, D))
    for b in range(B):
        n = int(lens[b])
        lo = 0 if window <= 0 else max(0, n - window)
        keys = list(range(lo, n))
        for h in range(Hq):
            qv = [bf16_to_float(q[b, h, d]) for d in range(D)]
            z = []
            for j in keys:
                kk = [float(kq[b, j, d]) * float(ks[b, j]) for d in range(D)]
                z.append(sigma * math.fsum(qv[d] * kk[d] for d in range(D)))
            if not z:
                continue
            m = max(z)
            p = [math.exp(t - m) for t in z]
            l = math.fsum(p)
            for d in range(D):
                out[b, h, d] = math.fsum(p[t] * float(vq[b, j, d]) * float(vs[b, j])
                                         for t, j in enumerate(keys)) / l
    return out


def brute_prefill(q, kq, ks, vq, vs, plens, window, sigma):
    B, C, Hq, D = q.shape
    out = np.zeros((B, C, Hq, D))
    for b in range(B):
        for i in range(C):
            pos = int(plens[b]) + i
            lo = 0 if window <= 0 else max(0, pos - window + 1)
            keys = list(range(lo, pos + 1))
            for h in range(Hq):
                qv = [bf16_to_float(q[b, i, h, d]) for d in range(D)]
                z = [sigma * math.fsum(qv[d] * float(kq[b, j, d]) * float(ks[b, j])
                                       for d in range(D)) for j in keys]
                m = max(z)
                p = [math.exp(t - m) for t in z]
                l = math.fsum(p)
                for d in range(D):
                    out[b, i, h, d] = math.fsum(p[t] * float(vq[b, j, d]) * float(vs[b, j])
                                                for t, j in enumerate(keys)) / l
    return out


@pytest.mark.parametrize("window", [0, 1, 5, 17, 100])
def test_decode_brute_force(window):
    q, kq, ks, vq, vs, lens = make_case(1, B=2, L=40, Hq=4, D=16)
    sigma = float(np.float32(0.3))
    ref = oracle.decode_ref(q, kq, ks, vq, vs, lens, window, np.float32(0.3))
    bf = brute_decode(q, kq, ks, vq, vs, lens, window, sigma)
    assert np.max(np.abs(ref - bf)) <= 1e-12


@pytest.mark.parametrize("window", [0, 3, 9])
def test_prefill_brute_force(window):
    B, C, Hq, D, L = 2, 5, 3, 8, 24
    g = synth.rng(710, 1)
    q = synth.q_bf16(g, (B, C, Hq, D))
    kq, ks = oracle.quantize_rows(synth.normal_f32(synth.rng(710, 2), (B, L, D)))
    vq, vs = oracle.quantize_rows(synth.normal_f32(synth.rng(710, 3), (B, L, D)))
    plens = np.array([7, 19], np.int32)
    sigma = oracle.default_softmax_scale(D)
    ref = oracle.prefill_ref(q, kq, ks, vq, vs, plens, window)
    bf = brute_prefill(q, kq, ks, vq, vs, plens, window, float(sigma))
    assert np.max(np.abs(ref - bf)) <= 1e-12


# ---------------------------------------------------------------------------
# library routine: scaled_dot_product_attention with the KV head replicated
# (multi-head attention whose heads all equal the single shared head)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("window", [0, 64, 200])
def test_decode_matches_sdpa_mha_replicated(window):
    B, L, Hq, D = 3, 300, 8, 64
    q, kq, ks, vq, vs, lens = make_case(2, B, L, Hq, D, lens=[300, 129, 1])
    ref = oracle.decode_ref(q, kq, ks, vq, vs, lens, window)
    sigma = float(oracle.default_softmax_scale(D))
    qf = torch.from_numpy(oracle.bf16_bits_to_f64(q))
    for b in range(B):
        n = int(lens[b])
        kh = torch.from_numpy(kq[b, :n].astype(np.float64) * ks[b, :n, None].astype(np.float64))
        vh = torch.from_numpy(vq[b, :n].astype(np.float64) * vs[b, :n, None].astype(np.float64))
        K = kh[None, None].expand(1, Hq, n, D).contiguous()
        V = vh[None, None].expand(1, Hq, n, D).contiguous()
        mask = torch.zeros(1, 1, 1, n, dtype=torch.bool)
        lo = 0 if window <= 0 else max(0, n - window)
        mask[..., lo:n] = True
        o = torch.nn.functional.scaled_dot_product_attention(
            qf[b][None, :, None, :], K, V, attn_mask=mask, scale=sigma)
        assert torch.max(torch.abs(o[0, :, 0, :] - torch.from_numpy(ref[b]))) <= 1e-12


def test_prefill_matches_sdpa():
    B, C, Hq, D, L = 2, 33, 4, 32, 120
    q = synth.q_bf16(synth.rng(720, 1), (B, C, Hq, D))
    kq, ks = oracle.quantize_rows(synth.normal_f32(synth.rng(720, 2), (B, L, D)))
    vq, vs = oracle.quantize_rows(synth.normal_f32(synth.rng(720, 3), (B, L, D)))
    plens = np.array([50, 87], np.int32)
    for window in (0, 16):
        ref = oracle.prefill_ref(q, kq, ks, vq, vs, plens, window)
        sigma = float(oracle.default_softmax_scale(D))
        for b in range(B):
            n = int(plens[b]) + C
            kh = torch.from_numpy(kq[b, :n].astype(np.float64) * ks[b, :n, None])
            vh = torch.from_numpy(vq[b, :n].astype(np.float64) * vs[b, :n, None])
            qf = torch.from_numpy(oracle.bf16_bits_to_f64(q[b])).permute(1, 0, 2)  # [Hq, C, D]
            pos = torch.arange(C)[:, None] + int(plens[b])
            j = torch.arange(n)[None, :]
            mask = j <= pos
            if window > 0:
                mask &= j > pos - window
            o = torch.nn.functional.scaled_dot_product_attention(
                qf[None], kh[None, None].expand(1, Hq, n, D), vh[None, None].expand(1, Hq, n, D),
                attn_mask=mask[None, None], scale=sigma)
            assert torch.max(torch.abs(o[0].permute(1, 0, 2) - torch.from_numpy(ref[b]))) <= 1e-12


# ---------------------------------------------------------------------------
# invariants and closed forms
# ---------------------------------------------------------------------------

def test_softmax_rows_sum_to_one():
    q, kq, ks, vq, vs, lens = make_case(3, 1, 4096, 32, 128, lens=[4096])
    khat = oracle.dequantize_rows(kq[0], ks[0])
    w = oracle.attention_weights(oracle.bf16_bits_to_f64(q[0]), khat,
                                 np.ones((32, 4096), bool), 0.0883883)
    assert np.max(np.abs(w.sum(axis=1) - 1.0)) <= 1e-12
    assert np.all(w >= 0)


def test_constant_values_give_that_constant():
    q, kq, ks, vq, vs, lens = make_case(4, 2, 64, 8, 32, lens=[64, 10])
    vq[:] = 127
    vs[:] = np.float32(0.75 / 127)
    out = oracle.decode_ref(q, kq, ks, vq, vs, lens, 0)
    c = 127 * float(np.float32(0.75 / 127))
    assert np.max(np.abs(out - c)) <= 1e-15 * 64


@pytest.mark.parametrize("n", [1, 7, 50])
def test_window_at_least_n_is_global(n):
    q, kq, ks, vq, vs, _ = make_case(5, 1, 64, 4, 16, lens=[n])
    lens = np.array([n], np.int32)
    g = oracle.decode_ref(q, kq, ks, vq, vs, lens, 0)
    for W in (n, n + 1, 1000):
        w = oracle.decode_ref(q, kq, ks, vq, vs, lens, W)
        assert np.array_equal(g, w)


def test_window_one_and_single_key_return_the_value_row():
    q, kq, ks, vq, vs, _ = make_case(6, 1, 64, 4, 16, lens=[1])
    for n, W in ((30, 1), (1, 0), (1, 1024)):
        lens = np.array([n], np.int32)
        out = oracle.decode_ref(q, kq, ks, vq, vs, lens, W)
        vlast = vq[0, n - 1].astype(np.float64) * float(vs[0, n - 1])
        assert np.array_equal(out[0], np.broadcast_to(vlast, out[0].shape))


@pytest.mark.parametrize("n,W", [(100, 10), (100, 99), (100, 1), (9, 0), (1024, 1024), (2000, 1024)])
def test_zero_query_averages_exactly_the_visible_window(n, W):
    """q = 0 makes every visible logit equal: the output is the mean of the visible
    values, so an off-by-one at either window end changes the answer."""
    L, D = max(n, 8), 16
    _, kq, ks, vq, vs, _ = make_case(7, 1, L, 2, D, lens=[n])
    q = np.zeros((1, 2, D), np.uint16)
    out = oracle.decode_ref(q, kq, ks, vq, vs, np.array([n], np.int32), W)
    lo = 0 if W <= 0 else n - min(W, n)
    vh = vq[0, lo:n].astype(np.float64) * vs[0, lo:n, None].astype(np.float64)
    mean = np.array([math.fsum(vh[:, d]) / (n - lo) for d in range(D)])
    assert np.max(np.abs(out[0, 0] - mean)) <= 1e-13
    # and differs from the mean over one key more or one key less
    if lo > 0:
        vh2 = vq[0, lo - 1:n].astype(np.float64) * vs[0, lo - 1:n, None]
        assert np.max(np.abs(out[0, 0] - vh2.mean(axis=0))) > 1e-6


def test_empty_sequence_outputs_zero():
    q, kq, ks, vq, vs, _ = make_case(8, 2, 16, 2, 8, lens=[1, 1])
    out = oracle.decode_ref(q, kq, ks, vq, vs, np.array([0, 5], np.int32), 0)
    assert not out[0].any() and out[1].any()


def test_shared_buffer_equals_copied_buffer():
    q, kq, ks, vq, vs, lens = make_case(9, 3, 80, 8, 32)
    qs = [synth.q_bf16(synth.rng(730, 1, li), q.shape) for li in range(3)]
    shared = {"A": (kq, ks, vq, vs)}
    copied = {"A": (kq, ks, vq, vs), "A2": (kq.copy(), ks.copy(), vq.copy(), vs.copy()),
              "A3": (kq.copy(), ks.copy(), vq.copy(), vs.copy())}
    o1 = oracle.hybrid_block_ref(qs, [("A", 0), ("A", 16), ("A", 16)], shared, lens)
    o2 = oracle.hybrid_block_ref(qs, [("A", 0), ("A2", 16), ("A3", 16)], copied, lens)
    for a, b in zip(o1, o2):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_partition_merge_reproduces_softmax(seed):
    q, kq, ks, vq, vs, _ = make_case(10 + seed, 1, 700, 8, 32, lens=[700])
    qr = oracle.bf16_bits_to_f64(q[0])
    kh = oracle.dequantize_rows(kq[0], ks[0])
    vh = oracle.dequantize_rows(vq[0], vs[0])
    sigma = 0.17
    full = oracle.attend(qr, kh, vh, np.ones((8, 700), bool), sigma)
    g = np.random.default_rng(seed)
    cuts = np.sort(g.choice(np.arange(0, 701), size=6, replace=True))
    bounds = [0, *cuts.tolist(), 700]
    parts = [oracle.lse_partial(qr, kh[a:b], vh[a:b], sigma) for a, b in zip(bounds[:-1], bounds[1:])]
    parts.append(oracle.lse_partial(qr, kh[:0], vh[:0], sigma))   # an empty partition
    assert np.max(np.abs(oracle.lse_merge(parts) - full)) <= 1e-12


def test_prefill_single_token_equals_decode():
    q, kq, ks, vq, vs, _ = make_case(11, 2, 300, 8, 64, lens=[1, 1])
    lens = np.array([300, 77], np.int32)
    for W in (0, 33):
        dec = oracle.decode_ref(q, kq, ks, vq, vs, lens, W)
        pre = oracle.prefill_ref(q[:, None], kq, ks, vq, vs, lens - 1, W)
        assert np.max(np.abs(pre[:, 0] - dec)) <= 1e-13


def test_prefill_is_causal():
    B, C, Hq, D, L = 1, 12, 2, 16, 40
    q = synth.q_bf16(synth.rng(740, 1), (B, C, Hq, D))
    kq, ks = oracle.quantize_rows(synth.normal_f32(synth.rng(740, 2), (B, L, D)))
    vq, vs = oracle.quantize_rows(synth.normal_f32(synth.rng(740, 3), (B, L, D)))
    plens = np.array([20], np.int32)
    base = oracle.prefill_ref(q, kq, ks, vq, vs, plens, 0)
    i = 5                                   # query at absolute position 25
    kq2, vq2 = kq.copy(), vq.copy()
    kq2[0, 26:] = -kq2[0, 26:]
    vq2[0, 26:] = 127
    pert = oracle.prefill_ref(q, kq2, ks, vq2, vs, plens, 0)
    assert np.array_equal(base[0, :i + 1], pert[0, :i + 1])
    assert not np.array_equal(base[0, i + 1:], pert[0, i + 1:])


def test_kv_bytes_printed_in_workshop():
    per_token, totals = kv_bytes()
    for D, layers, heads, nbytes, expect in per_token:
        assert oracle.kv_bytes_per_token(D, layers, heads, nbytes) == expect
    for D, layers, heads, nbytes, tokens, users, printed, digits in totals:
        gb = oracle.kv_bytes_per_token(D, layers, heads, nbytes) * tokens * users / 1e9
        # the transcript truncates its decimal-GB figures
        assert printed <= gb < printed + 10.0 ** (-digits)


def test_int8_mqa_accounting():
    # one shared head, int8 K and V plus an fp32 scale each
    assert oracle.int8_kv_bytes_per_key(128) == 264
    assert oracle.int8_kv_bytes_per_key(64) == 136
    assert oracle.decode_visible_keys([4096] * 64, 0) * 264 == 69_206_016
    assert oracle.decode_visible_keys([4096] * 64, 1024) * 264 == 17_301_504
    assert oracle.prefill_visible_pairs([8192] * 16, 512, 1024) == 16 * 512 * 1024


@pytest.mark.parametrize("window", [0, 1, 3, 7, 64, 1000])
def test_visible_counts_brute_force(window):
    """Key/query pair counts behind the bandwidth and flop figures, against a
    direct count of the mask predicate (key j visible to the query at
    absolute position p iff j <= p and, with a window W > 0, j > p - W), and
    the closed forms: global C P + C (C + 1) / 2 per sequence; C W once the
    prefix holds at least W keys."""
    prefixes, C = [0, 1, 5, 9, 70], 11
    want = 0
    for P in prefixes:
        for i in range(C):
            p = P + i
            want += sum(1 for j in range(P + C) if j <= p and (window <= 0 or j > p - window))
    assert oracle.prefill_visible_pairs(prefixes, C, window) == want
    if window <= 0:
        assert want == sum(C * P + C * (C + 1) // 2 for P in prefixes)
    for P in (window, window + 3) if window > 0 else ():
        assert oracle.prefill_visible_pairs([P], C, window) == C * window
    lens = [0, 1, 2, 6, 7, 8, 63, 64, 65, 999, 1000, 1001]
    want_d = sum(sum(1 for j in range(n) if window <= 0 or j >= n - window) for n in lens)
    assert oracle.decode_visible_keys(lens, window) == want_d


# ---------------------------------------------------------------------------
# default softmax scale: 1/sqrt(head_dim), not the model width
# [explinks.com page, 代码块描述: the snippet divides by the square root of
# the embedding size, which for its multi-head code is the whole model
# width; the reading is the head dimension of the one shared head]
# ---------------------------------------------------------------------------

def test_default_softmax_scale_values():
    assert oracle.default_softmax_scale(64) == np.float32(0.125)
    assert oracle.default_softmax_scale(16) == np.float32(0.25)
    # fl32(1/sqrt(128)): the fp32 nearest to 0.08838834764..., bit pattern 0x3DB504F3
    s128 = oracle.default_softmax_scale(128)
    assert s128.dtype == np.float32
    assert struct.pack("<f", s128) == struct.pack("<I", 0x3DB504F3)


@pytest.mark.parametrize("D,qlead", [(4, 2.0), (64, 8.0), (16, 4.0)])
def test_default_scale_inside_attention_closed_form(D, qlead):
    """Two keys: k_0 = 0, k_1 = e_0 (code 1, scale 1); values v_0 = 0, v_1 =
    all ones. With q = qlead * e_0 and qlead = sqrt(D), the logits are 0 and
    qlead / sqrt(D) = 1, so every output column is e / (1 + e). A scale of
    1/D, or 1/sqrt(Hq * D), or none at all gives another value."""
    Hq = 3
    q = np.zeros((1, Hq, D), np.uint16)
    q[0, :, 0] = synth.f32_to_bf16_bits(np.float32(qlead))
    kq = np.zeros((1, 2, D), np.int8)
    kq[0, 1, 0] = 1
    ks = np.array([[0.0, 1.0]], np.float32)
    vq = np.zeros((1, 2, D), np.int8)
    vq[0, 1, :] = 1
    vs = np.array([[0.0, 1.0]], np.float32)
    out = oracle.decode_ref(q, kq, ks, vq, vs, np.array([2], np.int32), 0)
    want = math.e / (1.0 + math.e)
    # sigma = fl32(1/sqrt(D)) is exact for these D
    assert np.max(np.abs(out - want)) <= 1e-15
    rows = oracle.decode_ref_rows(q, kq, ks, vq, vs, np.array([2], np.int32), 0, [(0, 1)])
    assert np.max(np.abs(rows - want)) <= 1e-15


# ---------------------------------------------------------------------------
# decode_ref_rows (the sampled-row checker) against scalar brute force
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("window", [0, 1, 5])
def test_decode_rows_brute_force(window):
    B, L, Hq, D = 5, 30, 3, 8
    q, kq, ks, vq, vs, lens = make_case(21, B, L, Hq, D, lens=[0, 1, 4, 17, 30])
    sigma = float(oracle.default_softmax_scale(D))
    bf = brute_decode(q, kq, ks, vq, vs, lens, window, sigma)
    picks = [(b, h) for b in range(B) for h in range(Hq)][::-1] + [(3, 1), (0, 0)]
    got = oracle.decode_ref_rows(q, kq, ks, vq, vs, lens, window, picks)
    assert got.shape == (len(picks), D)
    for i, (b, h) in enumerate(picks):
        assert np.max(np.abs(got[i] - bf[b, h])) <= 1e-12, (b, h)
    # the empty sequence (n = 0) gives a zero row
    assert not got[picks.index((0, 0))].any()
    assert oracle.decode_ref_rows(q, kq, ks, vq, vs, lens, window, []).shape == (0, D)
