"""mqa_decode_ragged / mqa_decode_append_ragged (a planning kernel cuts the
list of all sequences' visible tiles into ranges of equal cost, a tile
costing one unit and a sequence start a fixed number, one per work-group,
which walks the sequence segments inside its range) against the oracle, and
against mqa_decode on the same inputs (the same arithmetic summed in another
order); the plan itself against a host model of its documented layout."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import HostKV, assert_decode_close, dev, log, q_bits, q_dev

pytestmark = pytest.mark.gpu

T_KNEW, T_VNEW = synth.T_KNEW, synth.T_VNEW


def ragged_case(wid, B, L, Hq, D, lens, window, what, max_len=None, fill=None):
    import mqa_attention_int8_amd as m
    lens = np.asarray(lens, np.int32)
    max_len = int(lens.max()) if max_len is None else max_len
    log(f"ragged {what}: B={B} L={L} Hq={Hq} D={D} W={window} lens {int(lens.min())}..{int(lens.max())} "
        f"workspace {m.mqa_decode_ragged_workspace_bytes(B, Hq, D, max_len, window)} B")
    rows = fill if fill is not None else [(b, 0, int(min(n, L))) for b, n in enumerate(lens)]
    hk = HostKV.seeded(wid, 0, B, L, D, rows=rows)
    kv = hk.to_device()
    qb = q_bits(wid, (B, Hq, D))
    q, seq = q_dev(qb), dev(lens)
    out = m.mqa_decode_ragged(q, kv, seq, max_len, window)
    torch.cuda.synchronize()
    ref = oracle.decode_ref(qb, *hk.arrays(), np.minimum(lens, max_len), window)
    assert_decode_close(out, ref, 1e-4, f"{what}: ragged vs oracle")
    uni = m.mqa_decode(q, kv, seq, max_len, window)
    torch.cuda.synchronize()
    assert_decode_close(out, uni.cpu().numpy().astype(np.float64), 2e-5, f"{what}: ragged vs mqa_decode")


def test_hybrid_global_layer_full():
    """The hybrid block's global layer: 128 sequences of 1024..32768 keys."""
    w = synth.HYBRID
    lens = w.lens()
    L = (int(lens.max()) + 31) // 32 * 32
    ragged_case(w.wid, w.B, L, w.Hq, w.D, lens, 0, "hybrid global layer")


@pytest.mark.parametrize("window", [0, 100, 5000, 4096])
def test_mixed_lengths(window):
    lens = [0, 1, 31, 32, 33, 64, 1000, 4096, 20000, 7, 12345, 0, 3, 9000, 15000, 2]
    ragged_case(97, len(lens), 20000, 32, 128, lens, window, f"mixed W{window}")


def test_many_short_sequences():
    """1000 sequences of 0..300 keys: most are a single piece written directly."""
    lens = synth.ragged_lens(synth.rng(98, synth.T_LENS), 1000, 0, 300)
    ragged_case(98, 1000, 320, 8, 64, lens, 0, "1000 short")


def test_planner_carries_over_several_passes():
    """2500 sequences: the one-work-group planner walks the batch in three
    passes of 1024 (prefix sums carried across passes), and every
    work-group's range holds a dozen or more sequence segments."""
    lens = synth.ragged_lens(synth.rng(103, synth.T_LENS), 2500, 0, 700)
    ragged_case(103, 2500, 704, 8, 64, lens, 0, "2500 sequences")


@pytest.mark.parametrize("Hq,D", [(64, 128), (8, 64), (20, 128)])
def test_head_counts(Hq, D):
    lens = synth.ragged_lens(synth.rng(99, synth.T_LENS, Hq), 12, 1, 9000)
    ragged_case(99, 12, 9024, Hq, D, lens, 0, f"Hq{Hq} D{D}")


def test_uniform_lengths_and_one_sequence():
    ragged_case(100, 64, 4096, 32, 128, [4096] * 64, 0, "uniform B64 L4096")
    ragged_case(101, 1, 40000, 32, 128, [40000], 0, "one sequence of 40000")


def test_lengths_beyond_max_seq_len_are_clamped():
    """A seq_lens entry above max_seq_len is read as max_seq_len (the planner
    and the attention kernel clamp alike)."""
    ragged_case(102, 4, 2048, 32, 128, [3000, 100, 2000, 5000], 0, "clamped", max_len=1500)


def test_append_ragged_hybrid_global():
    """The owner layer of the global buffer: the new token's K and V are
    encoded into row n - 1 (bit-exact) and attended to in the same call."""
    import mqa_attention_int8_amd as m
    w = synth.HYBRID
    B, Hq, D = w.B, w.Hq, w.D
    lens = w.lens()
    L = (int(lens.max()) + 31) // 32 * 32
    log(f"append ragged hybrid global: B={B}")
    hk = HostKV.seeded(w.wid, 3, B, L, D, rows=[(b, 0, int(n) - 1) for b, n in enumerate(lens)])
    knew = synth.normal_f32(synth.rng(w.wid, T_KNEW, 3), (B, D))
    vnew = synth.normal_f32(synth.rng(w.wid, T_VNEW, 3), (B, D))
    kq_new, ks_new = oracle.quantize_rows(knew)
    vq_new, vs_new = oracle.quantize_rows(vnew)
    exp = [a.copy() for a in hk.arrays()]
    for b in range(B):
        n = int(lens[b])
        exp[0][b, n - 1], exp[1][b, n - 1] = kq_new[b], ks_new[b]
        exp[2][b, n - 1], exp[3][b, n - 1] = vq_new[b], vs_new[b]
    qb = q_bits(w.wid, (B, Hq, D), 3)
    kv = hk.to_device()
    out = m.mqa_decode_append_ragged(q_dev(qb), kv, dev(knew), dev(vnew), dev(lens), int(lens.max()), 0)
    torch.cuda.synchronize()
    for name, got, want in (("k", kv.k, exp[0]), ("k_scale", kv.k_scale, exp[1]), ("v", kv.v, exp[2]),
                            ("v_scale", kv.v_scale, exp[3])):
        g = got.cpu().numpy()
        assert g.view(np.uint8).tobytes() == np.ascontiguousarray(want).view(np.uint8).tobytes(), \
            f"cache {name} differs from the oracle encoding"
    ref = oracle.decode_ref(qb, *exp, lens, 0)
    assert_decode_close(out, ref, 1e-4, "append ragged vs oracle")


@pytest.mark.parametrize("case", ["hybrid", "mixed_w4096", "2500", "sparse"])
def test_plan_words_match_the_model(case):
    """The plan words (start of the workspace, which is filled with 0xff
    first) against the host model of the documented layout. Batches of more
    than 512 sequences are planned by the planning kernel, which writes every
    word (the segment slots past the last used one are not compared);
    smaller ones inside the attention kernel, which writes only the
    per-sequence words the merge kernel reads."""
    import mqa_attention_int8_amd as m
    from plan_model import n_words, plan_words, unpack
    window, Hq, D = 0, 32, 128
    if case == "hybrid":
        lens = synth.HYBRID.lens()
    elif case == "mixed_w4096":
        lens, window = np.array([0, 1, 31, 32, 33, 64, 1000, 4096, 20000, 7, 12345, 0, 3, 9000, 15000, 2]), 4096
    elif case == "2500":
        lens, Hq, D = synth.ragged_lens(synth.rng(103, synth.T_LENS), 2500, 0, 700), 8, 64
    else:   # few tiles: most work-groups' ranges hold only sequence-start cost
        lens = np.array([40, 3000, 0, 5, 0, 0, 700])
    lens = np.asarray(lens, np.int32)
    B, L = len(lens), int(lens.max())
    Lc = (L + 31) // 32 * 32
    G = torch.cuda.get_device_properties(0).multi_processor_count // ((Hq + 31) // 32)
    log(f"plan words {case}: B={B} G={G} W={window}")
    kv = m.KVView.empty(B, Lc, D)
    for t in (kv.k, kv.v):
        t.zero_()
    kv.k_scale.fill_(1.0)
    kv.v_scale.fill_(1.0)
    ws = m.ragged_workspace(B, Hq, D, L, window)
    ws.fill_(255)
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    m.mqa_decode_ragged(q, kv, dev(lens), L, window, workspace=ws)
    torch.cuda.synchronize()
    got = ws[:4 * n_words(G, B)].view(torch.int32).cpu().numpy()
    want, S = plan_words(lens, window, L, G)
    gh, gw, gs, gq = unpack(got, G, B)
    wh, ww, ws_, wq = unpack(want, G, B)
    assert np.array_equal(gq, wq)
    if B > 512:
        assert np.array_equal(gh, wh), (gh, wh)
        assert np.array_equal(gw, ww)
        assert np.array_equal(gs[:S], ws_[:S])
    else:
        assert np.all(gh == -1) and np.all(gw == -1)   # the planning kernel did not run


@pytest.mark.parametrize("B", [512, 513])
def test_plan_inside_and_outside_the_kernel(B):
    """512 sequences are planned inside the attention kernel, 513 by the
    planning kernel: both against the oracle, lengths 0..2000 keys."""
    lens = synth.ragged_lens(synth.rng(104, synth.T_LENS, B), B, 0, 2000)
    ragged_case(104, B, 2016, 8, 64, lens, 0, f"B{B} plan switch")
