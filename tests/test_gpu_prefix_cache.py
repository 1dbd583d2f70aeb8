"""Host prefix cache on the GPU: KV blocks go to a pinned host pool and back
bit for bit, for several shared buffers at once, and attention over a prefix
restored from the pool equals the oracle's over the original sequence."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import HostKV, assert_prefill_close, dev, log, q_bits

pytestmark = pytest.mark.gpu

WID = 62


@pytest.mark.parametrize("D,bs", [(128, 32), (64, 16)])
def test_round_trip_three_buffers(D, bs):
    import mqa_attention_int8_amd as m
    B, L = 3, 512
    log(f"prefix cache round trip: D={D} bs={bs}")
    hosts = [HostKV.seeded(WID, i, B, L, D) for i in range(3)]
    bufs = [h.to_device() for h in hosts]
    cache = m.PrefixCache(bs, 64)
    pool = m.host_pool(64, 3, bs, D)
    tokens = synth.rng(WID, 9).integers(0, 1000, size=300).tolist()   # 300 tokens: 300 // bs full blocks
    b = 1
    slots, first, n = cache.insert(tokens)
    assert first == 0 and n == 300 // bs
    m.mqa_kv_blocks_to_host(bufs, b, 0, slots, bs, pool)
    torch.cuda.synchronize()
    fresh = [m.KVView.empty(B, L, D) for _ in range(3)]
    for f in fresh:
        f.k.zero_(); f.v.zero_(); f.k_scale.zero_(); f.v_scale.zero_()
    got, mslots = cache.match(tokens + [1, 2, 3])
    assert got == n * bs
    m.mqa_kv_blocks_to_device(fresh, b, 0, mslots, bs, pool)
    torch.cuda.synchronize()
    for h, f in zip(hosts, fresh):
        for name, want in zip(("k", "k_scale", "v", "v_scale"), h.arrays()):
            g = getattr(f, name).cpu().numpy()
            assert g[b, :got].tobytes() == want[b, :got].tobytes(), name
            assert not g[b, got:].any() and not g[:b].any() and not g[b + 1:].any(), name
    cache.close()


def test_prefill_over_restored_prefix():
    """Turn 1 writes a conversation's KV and caches it; the device buffer is
    dropped; turn 2 restores the cached prefix, writes the rest of its prompt
    (the partial last block plus the new message) and runs the chunk's
    attention. The oracle sees the whole sequence as if it had never left
    the device."""
    import mqa_attention_int8_amd as m
    B, Hq, D, bs = 2, 32, 128, 32
    hist_len = [700, 333]
    C = 64
    L = 1024
    log("prefill over a restored prefix")
    k = synth.normal_f32(synth.rng(WID, synth.T_K, 5), (B, L, D))
    v = synth.normal_f32(synth.rng(WID, synth.T_V, 5), (B, L, D))
    kq, ks = oracle.quantize_rows(k)
    vq, vs = oracle.quantize_rows(v)
    toks = [synth.rng(WID, 10, b).integers(0, 5000, size=L).tolist() for b in range(B)]
    cache = m.PrefixCache(bs, 128)
    pool = m.host_pool(128, 1, bs, D)
    # turn 1: the history is on the device, then cached
    kv1 = HostKV(kq.copy(), ks.copy(), vq.copy(), vs.copy()).to_device()
    for b in range(B):
        slots, first, n = cache.insert(toks[b][: hist_len[b]])
        m.mqa_kv_blocks_to_host([kv1], b, first, slots[first:n], bs, pool)
    torch.cuda.synchronize()
    del kv1
    # turn 2: restore what is cached, write the rest of the prompt, prefill the chunk
    kv2 = m.KVView.empty(B, L, D)
    kv2.k.zero_(); kv2.v.zero_()
    prefix = []
    for b in range(B):
        got, slots = cache.match(toks[b][: hist_len[b] + C])
        assert got == (hist_len[b] // bs) * bs
        m.mqa_kv_blocks_to_device([kv2], b, 0, slots, bs, pool)
        prefix.append(got)
    P = np.array([hist_len[b] + 0 for b in range(B)], np.int32)   # the chunk starts after the history
    # rows [got, P + C) come from the model's projections: written with kv_quantize_int8
    for b in range(B):
        lo, hi = prefix[b], int(P[b]) + C
        start = torch.tensor([lo], dtype=torch.int32, device="cuda")
        m.kv_quantize_int8(dev(k[b:b + 1, lo:hi]), kv2.k[b:b + 1], kv2.k_scale[b:b + 1], start)
        m.kv_quantize_int8(dev(v[b:b + 1, lo:hi]), kv2.v[b:b + 1], kv2.v_scale[b:b + 1], start)
    qb = q_bits(WID, (B, C, Hq, D), 5)
    out = m.mqa_prefill_chunk(dev(qb.view(np.int16), torch.bfloat16), kv2, dev(P), int(P.max()), 0)
    torch.cuda.synchronize()
    ref = oracle.prefill_ref(qb, kq, ks, vq, vs, P, 0)
    assert_prefill_close(out, ref, what="prefill over restored prefix")
    cache.close()
