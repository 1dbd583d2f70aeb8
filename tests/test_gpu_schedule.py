"""Several decode steps of two hybrid 6-layer blocks whose global layers share
one KV buffer across the blocks. [9c1h.cn news page on Character.AI's
inference tricks, section "秘訣1", item "跨層KV共享": adjacent layers are tied
to one KV cache, and the global layers' caches are tied across blocks, since
they dominate the cache at long context; explinks.com page "Character.AI 的最佳
实践", section "跨层 KV 共享".]

Per block: layer 0 is global over buffer G (shared by both blocks), layers
1-3 use a 1024-key window over the block's buffer A, layers 4-5 over its
buffer B. In every step only the first layer that uses a buffer writes the
new token's K/V (fused append); the layers after it read the row it wrote.
Each layer's output is checked against the oracle (decode on host caches
updated with the oracle's encoding of the same new rows), and after the last
step every device cache equals its host copy bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import HostKV, assert_decode_close, dev, log, q_bits, q_dev

pytestmark = pytest.mark.gpu

WID = 31
W = 1024
# (buffer name of block k, window, writes the new row)
BLOCK = [("G", 0, True), ("A", W, True), ("A", W, False), ("A", W, False), ("B", W, True), ("B", W, False)]


def test_two_blocks_shared_global_buffer_several_steps():
    import mqa_attention_int8_amd as m
    B, Hq, D, steps = 8, 32, 128, 3
    n0 = np.array([1, 33, 1000, 1023, 1024, 1025, 1600, 2100], np.int32)
    L_cap = (int(n0.max()) + steps + 31) // 32 * 32  # decode takes whole 32-row tiles: a multiple of 32 rows
    log(f"schedule: 2 blocks x 6 layers, B={B} Hq={Hq} D={D} lens {n0.tolist()} + {steps} steps, L_cap={L_cap}")

    # the cache before step 0 holds rows [0, n0 - 1); window buffers only their visible part
    def rows(window):
        return [(b, max(0, int(n) - 1 - window) if window else 0, int(n) - 1) for b, n in enumerate(n0)]

    names = ["G", "A0", "B0", "A1", "B1"]
    host = {nm: HostKV.seeded(WID, i, B, L_cap, D, rows=rows(0 if nm == "G" else W)) for i, nm in enumerate(names)}
    hk = {nm: [a.copy() for a in h.arrays()] for nm, h in host.items()}  # kq, ks, vq, vs
    dv = {nm: h.to_device() for nm, h in host.items()}

    layer = 0
    for t in range(steps):
        lens = (n0 + t).astype(np.int32)
        seq = dev(lens)
        max_len = int(lens.max())
        outs = []
        for blk in range(2):
            for li, (base, window, writes) in enumerate(BLOCK):
                nm = "G" if base == "G" else f"{base}{blk}"
                writes = writes and (nm != "G" or blk == 0)  # block 1's global layer reads what block 0 wrote
                qb = q_bits(WID, (B, Hq, D), 1000 * t + 10 * blk + li)
                if writes:
                    knew = synth.normal_f32(synth.rng(WID, synth.T_KNEW, 1000 * t + 10 * blk + li), (B, D))
                    vnew = synth.normal_f32(synth.rng(WID, synth.T_VNEW, 1000 * t + 10 * blk + li), (B, D))
                    kq, ks = oracle.quantize_rows(knew)
                    vq, vs = oracle.quantize_rows(vnew)
                    a = hk[nm]
                    for b in range(B):
                        r = int(lens[b]) - 1
                        a[0][b, r], a[1][b, r], a[2][b, r], a[3][b, r] = kq[b], ks[b], vq[b], vs[b]
                    out = m.mqa_decode_append(q_dev(qb), dv[nm], dev(knew), dev(vnew), seq, max_len, window)
                else:
                    out = m.mqa_decode(q_dev(qb), dv[nm], seq, max_len, window)
                ref = oracle.decode_ref(qb, *hk[nm], lens, window)
                outs.append((out, ref, f"step {t} block {blk} layer {li} ({nm}, W={window}, "
                                       f"{'append' if writes else 'read'})"))
                layer += 1
        torch.cuda.synchronize()
        for out, ref, what in outs:
            assert_decode_close(out, ref, 1e-4, what)

    for nm in names:
        got = [x.cpu().numpy() for x in (dv[nm].k, dv[nm].k_scale, dv[nm].v, dv[nm].v_scale)]
        for g, e, part in zip(got, hk[nm], ("k", "k_scale", "v", "v_scale")):
            assert np.array_equal(g.view(np.uint8) if g.dtype == np.int8 else g.view(np.uint32),
                                  e.view(np.uint8) if e.dtype == np.int8 else e.view(np.uint32)), f"{nm}.{part}"
    log(f"  caches bit-identical after {steps} steps ({layer} layer calls)")
