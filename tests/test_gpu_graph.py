"""The library's calls captured in a HIP graph and replayed.

The benchmark times graph replays, and callers may capture a decode step.
Each case runs the calls eagerly, captures the same calls (explicit output
and workspace buffers, nothing allocated in the capture) and replays the
graph several times with other eager work and synchronisations in between;
every replay must give the eager result (up to the last bits that the
decode's dynamic tile order may change) and stay within the oracle's bar.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import HostKV, assert_decode_close, assert_prefill_close, dev, log, q_bits, q_dev

pytestmark = pytest.mark.gpu

REPLAYS = 4


def replay_and_check(calls, outs, refs, check, eager_tol):
    """calls(): issue the captured work; outs: its output tensors; refs: oracle arrays."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    for o, r, i in zip(eager, refs, range(len(outs))):
        check(o, r, f"eager output {i}")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        calls()
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        for o in outs:
            o.fill_(float("nan"))                    # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e, r) in enumerate(zip(outs, eager, refs)):
            d = float((o - e).abs().max())
            assert d <= eager_tol, f"replay {rep} output {i}: differs from eager by {d}"
            check(o, r, f"replay {rep} output {i}")
    del g


def test_decode_step_in_a_graph():
    import mqa_attention_int8_amd as m
    B, Hq, D, L = 16, 32, 128, 4096
    lens = synth.ragged_lens(synth.rng(41, synth.T_LENS), B, 1500, L)
    lens[0], lens[1] = L, 1
    log(f"graph decode: B={B} Hq={Hq} D={D} lens {lens.min()}..{lens.max()}")
    hk = HostKV.seeded(41, 0, B, L, D)
    knew = synth.normal_f32(synth.rng(41, synth.T_KNEW), (B, D))
    vnew = synth.normal_f32(synth.rng(41, synth.T_VNEW), (B, D))
    qg, qw = q_bits(41, (B, Hq, D), 0), q_bits(41, (B, Hq, D), 1)
    # host cache after the fused append: row n - 1 holds the oracle's encoding of the new rows
    kq, ks = oracle.quantize_rows(knew)
    vq, vs = oracle.quantize_rows(vnew)
    exp = [a.copy() for a in hk.arrays()]
    for b in range(B):
        r = int(lens[b]) - 1
        exp[0][b, r], exp[1][b, r], exp[2][b, r], exp[3][b, r] = kq[b], ks[b], vq[b], vs[b]
    refs = [oracle.decode_ref(qg, *exp, lens, 0), oracle.decode_ref(qw, *exp, lens, 1024)]

    kv = hk.to_device()
    seq, kn, vn = dev(lens), dev(knew), dev(vnew)
    q0, q1 = q_dev(qg), q_dev(qw)
    outs = [torch.empty((B, Hq, D), device="cuda") for _ in range(2)]
    wsg = m.decode_workspace(B, Hq, D, L, 0)
    wsw = m.decode_workspace(B, Hq, D, L, 1024)
    assert wsg is not None  # the global layer runs as partitions plus the merge kernel here

    def calls():
        # the append is idempotent (same row, same values), so every replay sees the same cache
        m.mqa_decode_append(q0, kv, kn, vn, seq, L, 0, out=outs[0], workspace=wsg)
        m.mqa_decode(q1, kv, seq, L, 1024, out=outs[1], workspace=wsw)

    replay_and_check(calls, outs, refs, lambda o, r, w: assert_decode_close(o, r, 1e-4, w), 1e-6)
    got = [x.cpu().numpy() for x in (kv.k, kv.k_scale, kv.v, kv.v_scale)]
    for g_, e in zip(got, exp):
        assert np.array_equal(g_, e)


@pytest.mark.parametrize("window", [0, 64])
def test_prefill_chunk_in_a_graph(window):
    import mqa_attention_int8_amd as m
    B, C, Hq, D = 3, 96, 32, 128
    plens = np.array([0, 130, 700], np.int32)
    L = int(plens.max()) + C
    log(f"graph prefill: B={B} C={C} Hq={Hq} D={D} prefix={plens.tolist()} W={window}")
    hk = HostKV.seeded(42, 0, B, L, D)
    qb = q_bits(42, (B, C, Hq, D))
    ref = oracle.prefill_ref(qb, *hk.arrays(), plens, window)
    kv, q, pl = hk.to_device(), q_dev(qb), dev(plens)
    out = torch.empty((B, C, Hq, D), device="cuda")
    ws = m.prefill_workspace(B, C, D, int(plens.max()))

    def calls():
        m.mqa_prefill_chunk(q, kv, pl, int(plens.max()), window, out=out, workspace=ws)

    replay_and_check(calls, [out], [ref], lambda o, r, w: assert_prefill_close(o, r, what=w), 0.0)


def test_ragged_decode_in_a_graph():
    """The balanced plan in a graph: the planner kernel rewrites the plan in
    the workspace on every replay (here after the workspace was overwritten
    with garbage between replays), then the partitions and the merge read it.
    Also the allocation-free call, whose states live in the library's
    static array."""
    import mqa_attention_int8_amd as m
    B, Hq, D, L = 40, 32, 128, 6144
    lens = synth.ragged_lens(synth.rng(43, synth.T_LENS), B, 0, L)
    lens[0], lens[1] = L, 0
    log(f"graph ragged decode: B={B} lens {lens.min()}..{lens.max()}")
    hk = HostKV.seeded(43, 0, B, L, D)
    knew = synth.normal_f32(synth.rng(43, synth.T_KNEW), (B, D))
    vnew = synth.normal_f32(synth.rng(43, synth.T_VNEW), (B, D))
    qg, qn = q_bits(43, (B, Hq, D), 0), q_bits(43, (B, Hq, D), 1)
    kq, ks = oracle.quantize_rows(knew)
    vq, vs = oracle.quantize_rows(vnew)
    exp = [a.copy() for a in hk.arrays()]
    for b in range(B):
        r = int(lens[b]) - 1
        if r >= 0:
            exp[0][b, r], exp[1][b, r], exp[2][b, r], exp[3][b, r] = kq[b], ks[b], vq[b], vs[b]
    refs = [oracle.decode_ref(qg, *exp, lens, 0), oracle.decode_ref(qn, *exp, lens, 0)]
    kv = hk.to_device()
    seq, kn, vn = dev(lens), dev(knew), dev(vnew)
    q0, q1 = q_dev(qg), q_dev(qn)
    outs = [torch.empty((B, Hq, D), device="cuda") for _ in range(2)]
    ws = m.ragged_workspace(B, Hq, D, L, 0)

    def calls():
        m.mqa_decode_append_ragged(q0, kv, kn, vn, seq, L, 0, out=outs[0], workspace=ws)
        m.mqa_decode_noalloc(q1, kv, seq, L, 0, out=outs[1])

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    for o, r in zip(eager, refs):
        assert_decode_close(o, r, 1e-4, "eager")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        calls()
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        ws.fill_(255)                                # the plan must be rebuilt by the replay
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e, r) in enumerate(zip(outs, eager, refs)):
            assert float((o - e).abs().max()) <= 1e-6, f"replay {rep} output {i}"
            assert_decode_close(o, r, 1e-4, f"replay {rep} output {i}")
    del g
    got = [x.cpu().numpy() for x in (kv.k, kv.k_scale, kv.v, kv.v_scale)]
    for g_, e in zip(got, exp):
        assert np.array_equal(g_, e)
