#!/usr/bin/env python3
"""Benchmark of MQA int8-KV decode on one MI355X.

One step = one decode step of two attention layers that share ONE int8 KV
buffer (cross-layer KV sharing): the global layer owns the buffer and runs
mqa_decode_append (the new token's K and V rows are encoded into it in the
same launch), then the sliding-window (1024) layer runs mqa_decode over it.
Shapes: B = 64 sequences of 4096 keys, 32 query heads, one KV head,
head_dim 128.

Inputs are synthetic (seeded N(0,1) on the device, K/V encoded with the
library's own quantizer) and resident in HBM before timing. The step is
rotated over enough buffer copies (>= 1 GB) that the 256 MB Infinity Cache
cannot serve the KV reads. Steps are captured in a HIP graph so the timing is
the GPU's, not Python's.

Prints ONE JSON line. ``value`` = decode tokens/s of the step (B tokens per
step, attention only). ``roofline`` describes the global-layer call
(partition kernel with the fused append + merge kernel). ``cpu_baseline`` times the CPU oracle
on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, datasheet
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, datasheet
METRIC = "MQA int8-KV decode: KV-read HBM GB/s (% of peak) and decode tokens/s"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of graph replay")
    ap.add_argument("--no-extra", action="store_true", help="skip the hybrid/long/prefill lines")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU-baseline time budget")
    ap.add_argument("--only", choices=["decode", "hybrid", "long", "prefill", "paged", "q8", "prefix_cache",
                                       "ceilings"],
                    default=None,
                    help="time a single workload (for profiling runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    return ap.parse_args()


class Timer:
    """HIP events on the stream the kernels run on."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def start(self):
        self.a.record(self.stream)

    def stop_ms(self):
        self.b.record(self.stream)
        self.b.synchronize()
        return self.a.elapsed_time(self.b)


def make_decode_buffers(torch, m, B, L, D, copies, gen):
    """`copies` KV buffers filled with N(0,1) rows encoded by kv_quantize_int8."""
    bufs = []
    start = torch.zeros(B, dtype=torch.int32, device="cuda")
    chunk = max(1, (1 << 28) // (L * D * 4))          # <= 256 MiB of fp32 at a time
    for _ in range(copies):
        kv = m.KVView.empty(B, L, D)
        for b0 in range(0, B, chunk):
            b1 = min(B, b0 + chunk)
            for dst, dsc in ((kv.k, kv.k_scale), (kv.v, kv.v_scale)):
                x = torch.randn((b1 - b0, L, D), generator=gen, device="cuda", dtype=torch.float32)
                m.kv_quantize_int8(x, dst[b0:b1], dsc[b0:b1], start[b0:b1])
        bufs.append(kv)
    torch.cuda.synchronize()
    return bufs


def run_steps(torch, fn, steps, use_graph, stream, warm=1):
    """Replay `fn` (which runs `period` steps) steps/period times after `warm`
    untimed replays; returns ms."""
    timer = Timer(torch, stream)
    if use_graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            fn()
        torch.cuda.synchronize()
        reps = steps
        for _ in range(max(1, warm)):
            g.replay()
        torch.cuda.synchronize()
        timer.start()
        for _ in range(reps):
            g.replay()
        ms = timer.stop_ms()
        return ms, g
    timer.start()
    for _ in range(steps):
        fn()
    return timer.stop_ms(), None


def bench_decode(torch, m, acct, args, stream):
    B, Hq, D, L = 64, 32, 128, 4096
    windows = (0, 1024)
    bytes_per_copy = B * L * (2 * D + 8)
    R = max(2, math.ceil((1 << 30) / bytes_per_copy))              # >= 1 GiB of KV
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2)
    bufs = make_decode_buffers(torch, m, B, L, D, R, gen)
    seq_lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    q = [[torch.randn((B, Hq, D), generator=gen, device="cuda").to(torch.bfloat16) for _ in windows]
         for _ in range(R)]
    knew = [torch.randn((B, 1, D), generator=gen, device="cuda") for _ in range(R)]
    vnew = [torch.randn((B, 1, D), generator=gen, device="cuda") for _ in range(R)]
    outs = [torch.empty((B, Hq, D), device="cuda") for _ in windows]
    ws = [m.decode_workspace(B, Hq, D, L, w) for w in windows]

    def one_step(r):
        # the global layer owns the buffer: it appends the new token (fused), the window layer reads it
        kv = bufs[r]
        m.mqa_decode_append(q[r][0], kv, knew[r].view(B, D), vnew[r].view(B, D), seq_lens, L, windows[0],
                            out=outs[0], workspace=ws[0])
        m.mqa_decode(q[r][1], kv, seq_lens, L, windows[1], out=outs[1], workspace=ws[1])

    def period():
        for r in range(R):
            one_step(r)

    def global_only():
        for r in range(R):
            m.mqa_decode_append(q[r][0], bufs[r], knew[r].view(B, D), vnew[r].view(B, D), seq_lens, L, 0,
                                out=outs[0], workspace=ws[0])

    with torch.cuda.stream(stream):
        for _ in range(max(1, args.warmup // R)):
            period()
        torch.cuda.synchronize()
        use_graph = not args.no_graph
        reps = max(1, args.steps // R)
        ms, _ = run_steps(torch, period, reps, use_graph, stream)
        steps_done = reps * R
        ms_step = ms / steps_done
        # dominant kernel: the global layer's call (fused append + partitions, then the merge)
        ms_g, _ = run_steps(torch, global_only, reps, use_graph, stream)
        ms_call = ms_g / (reps * R)
    kv_step = sum(acct.decode_kv_bytes([L] * B, w, D) for w in windows)
    kv_global = acct.decode_kv_bytes([L] * B, 0, D)
    res = {
        "steps_done": steps_done, "ms_per_step": ms_step, "tokens_per_s": B / (ms_step * 1e-3),
        "kv_bytes_per_step": kv_step, "step_kv_GBps": kv_step / (ms_step * 1e-3) / 1e9,
        "global_call_us": ms_call * 1e3, "global_kv_bytes": kv_global,
        "global_GBps": kv_global / (ms_call * 1e-3) / 1e9, "rotation_copies": R,
        "graph": use_graph,
    }
    return res


def load_ceilings():
    """libmqa_ceilings.so (measurement kernels); raises if it is not built."""
    import ctypes
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "mqa_attention_int8_amd", "libmqa_ceilings.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    lib.mqa_ceiling_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p,
                                            ctypes.c_void_p]
    lib.mqa_ceiling_mfma_bf16.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    lib.mqa_ceiling_mfma_bf16_flops.argtypes = [ctypes.c_int32, ctypes.c_int32]
    lib.mqa_ceiling_mfma_bf16_flops.restype = ctypes.c_double
    return lib


def bench_ceilings(torch, stream):
    """Achievable ceilings on this GPU: one-pass HBM streaming (the global
    decode call's 69.2 MB and 1 GiB, each over >= 1 GiB of rotated copies so
    no cache holds them) and dense bf16 MFMA throughput."""
    lib = load_ceilings()
    sp = stream.cuda_stream
    res = {}
    blocks = 4096                     # 16 KB chunks per work-group; the fastest of 2048-16384 on 69 MB
    partial = torch.empty(blocks, dtype=torch.int32, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    for name, nbytes in (("stream_read_69MB", 69_206_016), ("stream_read_1GiB", 1 << 30)):
        R = max(2, math.ceil((1 << 30) / nbytes))
        bufs = [torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda", generator=gen)
                for _ in range(R)]
        torch.cuda.synchronize()          # the fills ran on the default stream
        with torch.cuda.stream(stream):
            # every word read exactly once: the partial sums add up to the buffer's sum mod 2^32
            rc = lib.mqa_ceiling_stream_read(bufs[0].data_ptr(), nbytes, blocks, partial.data_ptr(), sp)
            if rc != 0:
                raise RuntimeError(f"mqa_ceiling_stream_read: status {rc}")
            torch.cuda.synchronize()
            got = int(partial.to(torch.int64).sum().item()) & 0xFFFFFFFF
            want = int(bufs[0].to(torch.int64).sum().item()) & 0xFFFFFFFF
            if got != want:
                raise RuntimeError(f"streaming checksum {got:#x} != {want:#x}")

            def period():
                for r in range(R):
                    lib.mqa_ceiling_stream_read(bufs[r].data_ptr(), nbytes, blocks, partial.data_ptr(),
                                                torch.cuda.current_stream().cuda_stream)
            reps = max(2, 64 // R)
            ms, _ = run_steps(torch, period, reps, True, stream, warm=3)
        us = ms / (reps * R) * 1e3
        res[name] = {"bytes": nbytes, "us": us, "GBps": nbytes / (us * 1e-6) / 1e9,
                     "frac_hbm_peak": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, "rotation_copies": R,
                     "blocks": blocks}
        del bufs
    mb, iters = 1024, 2048
    sink = torch.empty(mb * 512, dtype=torch.float32, device="cuda")
    with torch.cuda.stream(stream):
        def mm():
            rc = lib.mqa_ceiling_mfma_bf16(mb, iters, sink.data_ptr(), torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise RuntimeError(f"mqa_ceiling_mfma_bf16: status {rc}")
        mm()
        torch.cuda.synchronize()
        if not bool(torch.isfinite(sink).all()):
            raise RuntimeError("MFMA loop produced non-finite sums")
        ms, _ = run_steps(torch, mm, 10, True, stream, warm=20)
    fl = lib.mqa_ceiling_mfma_bf16_flops(mb, iters)
    tf = fl / (ms / 10 * 1e-3) / 1e12
    res["mfma_bf16"] = {"flops_per_launch": fl, "us": ms / 10 * 1e3, "TFLOPs": tf, "frac_bf16_peak": tf / BF16_PEAK_TFLOPS,
                        "kernel": "v_mfma_f32_16x16x32_bf16, 8 independent chains per wave, 8 waves per work-group, "
                                  f"{mb} work-groups"}
    return res


def bench_hybrid(torch, m, acct, stream):
    """6-layer block: 1 global + 5 window-1024 layers, buffers G (l0), A (l1-3), B (l4-5)."""
    import numpy as np
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import synth
    w = synth.HYBRID
    B, Hq, D = w.B, w.Hq, w.D
    lens = w.lens()
    L = int(lens.max())
    L_cap = (L + 15) // 16 * 16
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3)
    bufs = {name: make_decode_buffers(torch, m, B, L_cap, D, 1, gen)[0] for name in ("G", "A", "Bf")}
    seq_lens = torch.from_numpy(lens).cuda()
    q = [torch.randn((B, Hq, D), generator=gen, device="cuda").to(torch.bfloat16) for _ in w.layers]
    knew = torch.randn((B, D), generator=gen, device="cuda")
    vnew = torch.randn((B, D), generator=gen, device="cuda")
    out = torch.empty((B, Hq, D), device="cuda")
    ws = torch.zeros(max(m.mqa_decode_workspace_bytes(B, Hq, D, L, win) for _, win in w.layers) + 16,
                     dtype=torch.uint8, device="cuda")
    owners = {}
    for li, (name, _) in enumerate(w.layers):
        owners.setdefault(name, li)

    def block():
        for li, (name, win) in enumerate(w.layers):
            kv = bufs[name]
            if owners[name] == li:             # first layer of a sharing group writes the token (fused)
                m.mqa_decode_append(q[li], kv, knew, vnew, seq_lens, L, win, out=out, workspace=ws)
            else:
                m.mqa_decode(q[li], kv, seq_lens, L, win, out=out, workspace=ws)

    with torch.cuda.stream(stream):
        for _ in range(3):
            block()
        torch.cuda.synchronize()
        reps = 30
        ms, _ = run_steps(torch, block, reps, True, stream)
    ms_block = ms / reps
    kv = sum(acct.decode_kv_bytes(lens, win, D) for _, win in w.layers)
    return {"workload": w.name, "ms_per_block_step": ms_block, "tokens_per_s": B / (ms_block * 1e-3),
            "kv_bytes": kv, "kv_GBps": kv / (ms_block * 1e-3) / 1e9,
            "note": "layers 2,3,5 re-read a buffer the previous layer just read (Infinity Cache may serve them)"}


def bench_long(torch, m, acct, stream):
    B, Hq, D, L = 8, 32, 128, 131072
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    bufs = make_decode_buffers(torch, m, B, L, D, 4, gen)
    seq_lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    q = torch.randn((B, Hq, D), generator=gen, device="cuda").to(torch.bfloat16)
    out = torch.empty((B, Hq, D), device="cuda")
    ws = m.decode_workspace(B, Hq, D, L, 0)

    def calls():
        for kv in bufs:
            m.mqa_decode(q, kv, seq_lens, L, 0, out=out, workspace=ws)

    with torch.cuda.stream(stream):
        calls()
        torch.cuda.synchronize()
        reps = 25
        ms, _ = run_steps(torch, calls, reps, True, stream)
    ms_call = ms / (reps * len(bufs))
    kv = acct.decode_kv_bytes([L] * B, 0, D)
    return {"workload": "long_decode_B8_Hq32_D128_L131072", "us_per_call": ms_call * 1e3,
            "tokens_per_s": B / (ms_call * 1e-3), "kv_GBps": kv / (ms_call * 1e-3) / 1e9,
            "frac_hbm_peak": kv / (ms_call * 1e-3) / 1e9 / HBM_PEAK_GBPS}


def bench_paged(torch, m, acct, stream):
    """Paged layouts on the decode workload's shape: the global layer (fused
    append) over a pool of 32-token blocks in shuffled order, and a window-1024
    layer over a ring of 1024 slots per sequence; each against the same call on
    contiguous buffers, timed in this run."""
    B, Hq, D, L, bs, W = 64, 32, 128, 4096, 32, 1024
    TL = L // bs
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    per = B * L * (2 * D + 8)
    R = max(2, math.ceil((1 << 30) / per))
    cont = make_decode_buffers(torch, m, B, L, D, R, gen)
    pools = []
    for kv in cont:
        perm = torch.randperm(B * TL, generator=gen, device="cuda")
        table = perm.view(B, TL).to(torch.int32).contiguous()
        pk = torch.empty((B * TL, bs, D), dtype=torch.int8, device="cuda")
        pv = torch.empty_like(pk)
        pks = torch.empty((B * TL, bs), dtype=torch.float32, device="cuda")
        pvs = torch.empty_like(pks)
        pk[perm] = kv.k.view(B * TL, bs, D)
        pv[perm] = kv.v.view(B * TL, bs, D)
        pks[perm] = kv.k_scale.view(B * TL, bs)
        pvs[perm] = kv.v_scale.view(B * TL, bs)
        pools.append(m.PagedKV(pk, pv, pks, pvs, table))
    # window-only ring buffers: 1024 slots per sequence, positions 0..L-1 appended in order
    TLr = W // bs
    ring_per = B * W * (2 * D + 8)
    Rr = max(2, math.ceil((1 << 30) / ring_per))
    rings = []
    for _ in range(Rr):
        table = torch.randperm(B * TLr, generator=gen, device="cuda").view(B, TLr).to(torch.int32).contiguous()
        kvr = m.PagedKV.empty(B * TLr, bs, D, table)
        kvr.k.copy_(torch.randint(-127, 128, kvr.k.shape, generator=gen, device="cuda", dtype=torch.int8))
        kvr.v.copy_(torch.randint(-127, 128, kvr.v.shape, generator=gen, device="cuda", dtype=torch.int8))
        kvr.k_scale.copy_(torch.rand(kvr.k_scale.shape, generator=gen, device="cuda") * 0.03)
        kvr.v_scale.copy_(torch.rand(kvr.v_scale.shape, generator=gen, device="cuda") * 0.03)
        rings.append(kvr)
    seq_lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    q = torch.randn((B, Hq, D), generator=gen, device="cuda").to(torch.bfloat16)
    knew = torch.randn((B, D), generator=gen, device="cuda")
    vnew = torch.randn((B, D), generator=gen, device="cuda")
    out = torch.empty((B, Hq, D), device="cuda")
    ws_c = [m.decode_workspace(B, Hq, D, L, w) for w in (0, W)]
    nws = max(m.mqa_decode_paged_workspace_bytes(B, Hq, D, L, w, bs) for w in (0, W))
    ws_p = torch.empty(max(nws, 16), dtype=torch.uint8, device="cuda")

    def g_cont():
        for kv in cont:
            m.mqa_decode_append(q, kv, knew, vnew, seq_lens, L, 0, out=out, workspace=ws_c[0])

    def g_paged():
        for kv in pools:
            m.mqa_decode_append_paged(q, kv, knew, vnew, seq_lens, L, 0, out=out, workspace=ws_p)

    def w_cont():
        for kv in cont:
            m.mqa_decode(q, kv, seq_lens, L, W, out=out, workspace=ws_c[1])

    def w_ring():
        for kv in rings:
            m.mqa_decode_paged(q, kv, seq_lens, L, W, out=out, workspace=ws_p)

    res = {"workload": "decode_B64_Hq32_D128_L4096", "block_size": bs, "ring_slots": W}
    with torch.cuda.stream(stream):
        for name, fn, n in (("global_contiguous_us", g_cont, R), ("global_paged_us", g_paged, R),
                            ("window_contiguous_us", w_cont, R), ("window_ring_us", w_ring, Rr)):
            fn()
            torch.cuda.synchronize()
            reps = 20
            ms, _ = run_steps(torch, fn, reps, True, stream)
            res[name] = ms * 1e3 / (reps * n)
    kv_g = acct.decode_kv_bytes([L] * B, 0, D)
    kv_w = acct.decode_kv_bytes([L] * B, W, D)
    res["global_paged_GBps"] = kv_g / (res["global_paged_us"] * 1e-6) / 1e9
    res["window_ring_GBps"] = kv_w / (res["window_ring_us"] * 1e-6) / 1e9
    res["window_buffer_bytes_per_seq"] = {"ring": W * (2 * D + 8), "contiguous": L * (2 * D + 8)}
    return res


def bench_q8(torch, m, acct, stream):
    """The decode step of the main workload with int8 queries (int8 MFMA for
    Q K^T; the query rows encoded by kv_quantize_int8 outside the timed
    region, as a projection with int8 outputs would deliver them), against the
    bf16-query step in the same run."""
    B, Hq, D, L = 64, 32, 128, 4096
    windows = (0, 1024)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(8)
    R = max(2, math.ceil((1 << 30) / (B * L * (2 * D + 8))))
    bufs = make_decode_buffers(torch, m, B, L, D, R, gen)
    seq_lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    zero = torch.zeros(B, dtype=torch.int32, device="cuda")
    qf = [torch.randn((B, Hq, D), generator=gen, device="cuda").to(torch.bfloat16) for _ in windows]
    q8 = [torch.empty((B, Hq, D), dtype=torch.int8, device="cuda") for _ in windows]
    qs = [torch.empty((B, Hq), dtype=torch.float32, device="cuda") for _ in windows]
    for i in range(len(windows)):
        m.kv_quantize_int8(qf[i].float().contiguous(), q8[i], qs[i], zero)
    knew = torch.randn((B, D), generator=gen, device="cuda")
    vnew = torch.randn((B, D), generator=gen, device="cuda")
    out = torch.empty((B, Hq, D), device="cuda")
    ws = [m.decode_workspace(B, Hq, D, L, w) for w in windows]

    def step_bf16():
        for kv in bufs:
            m.mqa_decode_append(qf[0], kv, knew, vnew, seq_lens, L, 0, out=out, workspace=ws[0])
            m.mqa_decode(qf[1], kv, seq_lens, L, windows[1], out=out, workspace=ws[1])

    def step_q8():
        for kv in bufs:
            m.mqa_decode_append_q8(q8[0], qs[0], kv, knew, vnew, seq_lens, L, 0, out=out, workspace=ws[0])
            m.mqa_decode_q8(q8[1], qs[1], kv, seq_lens, L, windows[1], out=out, workspace=ws[1])

    def global_q8():
        for kv in bufs:
            m.mqa_decode_append_q8(q8[0], qs[0], kv, knew, vnew, seq_lens, L, 0, out=out, workspace=ws[0])

    res = {"workload": "decode_B64_Hq32_D128_L4096 (global + window-1024 layer), int8 queries"}
    with torch.cuda.stream(stream):
        for name, fn in (("step_bf16_us", step_bf16), ("step_q8_us", step_q8), ("global_q8_us", global_q8)):
            fn()
            torch.cuda.synchronize()
            reps = 20
            ms, _ = run_steps(torch, fn, reps, True, stream)
            res[name] = ms * 1e3 / (reps * R)
    res["tokens_per_s_q8"] = B / (res["step_q8_us"] * 1e-6)
    kv_g = acct.decode_kv_bytes([L] * B, 0, D)
    res["global_q8_GBps"] = kv_g / (res["global_q8_us"] * 1e-6) / 1e9
    return res


def bench_prefix_cache(torch, m, stream):
    """Host-memory prefix cache: restore (host pool -> device) and store
    bandwidth of an 8192-token prefix over three shared KV buffers, and the
    control plane on a synthetic multi-turn stream (conversations of ~180
    messages, the pages' average; the hit rate is a property of this stream,
    not a claim about real traffic)."""
    import time
    import numpy as np
    B, D, bs, L, nb = 4, 128, 32, 8192, 3
    bufs = [m.KVView.empty(B, L, D) for _ in range(nb)]
    for kv in bufs:
        kv.k.random_(-127, 128)
        kv.v.random_(-127, 128)
        kv.k_scale.uniform_(0, 0.03)
        kv.v_scale.uniform_(0, 0.03)
    n_blocks = L // bs
    pool = m.host_pool(n_blocks, nb, bs, D)
    slots = np.arange(n_blocks, dtype=np.int64)
    nbytes = n_blocks * m.kv_block_bytes(nb, bs, D)
    res = {"prefix_tokens": L, "buffers": nb, "block_size": bs, "bytes": nbytes}
    timer = Timer(torch, stream)
    with torch.cuda.stream(stream):
        for name, fn in (("store", m.mqa_kv_blocks_to_host), ("restore", m.mqa_kv_blocks_to_device)):
            for _ in range(3):
                fn(bufs, 1, 0, slots, bs, pool, stream=stream)
            torch.cuda.synchronize()
            reps = 20
            timer.start()
            for _ in range(reps):
                fn(bufs, 1, 0, slots, bs, pool, stream=stream)
            ms = timer.stop_ms() / reps
            res[name + "_us"] = ms * 1e3
            res[name + "_GBps"] = nbytes / (ms * 1e-3) / 1e9
    # control plane on a synthetic stream
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import synth
    g = synth.rng(990, 1)
    n_conv, turns = 64, 90                      # 2 messages per turn: ~180 messages per conversation
    cache = m.PrefixCache(16, 1 << 18)
    hist = [[] for _ in range(n_conv)]
    order = [c for _ in range(turns) for c in g.permutation(n_conv)]
    t0 = time.perf_counter()
    for c in order:
        req = hist[c] + g.integers(0, 32000, size=int(g.integers(8, 64))).tolist()
        cache.match(req)
        hist[c] = req + g.integers(0, 32000, size=int(g.integers(8, 64))).tolist()
        cache.insert(hist[c])
    dt = time.perf_counter() - t0
    st = cache.stats()
    cache.close()
    res["control_plane_us_per_turn"] = dt / len(order) * 1e6
    res["synthetic_stream_token_hit_rate"] = st["matched_tokens"] / max(1, st["lookup_tokens"])
    res["synthetic_stream"] = f"{n_conv} conversations x {turns} turns, messages 8-63 tokens, block 16"
    return res


def bench_prefill(torch, m, acct, stream):
    B, C, P, Hq, D = 16, 512, 8192, 32, 128
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4)
    kv = make_decode_buffers(torch, m, B, P + C, D, 1, gen)[0]
    q = torch.randn((B, C, Hq, D), generator=gen, device="cuda").to(torch.bfloat16)
    plens = torch.full((B,), P, dtype=torch.int32, device="cuda")
    out = torch.empty((B, C, Hq, D), device="cuda")
    ws = m.prefill_workspace(B, C, D, P)
    res = {"workload": "prefill_B16_C512_P8192_Hq32_D128"}
    with torch.cuda.stream(stream):
        for win in (0, 1024):
            def call():
                m.mqa_prefill_chunk(q, kv, plens, P, win, out=out, workspace=ws)
            call()
            torch.cuda.synchronize()
            # untimed replays first (~0.1 s): the first ~50 ms of back-to-back
            # calls of this MFMA-bound kernel run up to ~15% slower than the
            # settled rate
            reps = 10
            ms, _ = run_steps(torch, call, reps, True, stream, warm=80 if win == 0 else 200)
            ms_call = ms / reps
            fl = acct.prefill_flops([P] * B, C, win, Hq, D)
            tf = fl / (ms_call * 1e-3) / 1e12
            res[f"W{win}"] = {"ms": ms_call, "flops": fl, "TFLOPs": tf, "frac_bf16_peak": tf / BF16_PEAK_TFLOPS}
    return res


def counted_traffic():
    """HBM bytes per global-layer decode call from the committed rocprofv3
    counter summary, or None when the decode kernel source has changed since
    the counters were taken."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", "decode_global_traffic.json")
    try:
        rec = json.load(open(path))
        h = hashlib.sha256()
        for f in rec["source_files"]:
            h.update(open(os.path.join(root, f), "rb").read())
        if h.hexdigest() != rec["source_sha256"]:
            return None
        return rec["traffic_bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(budget_s: float):
    """The oracle (numpy, float64) on a bounded sample of the decode workload.

    Per sequence, the timed work is what one step does: encode the new token's
    K and V rows, then the global and the window-1024 layer. The 64
    sequences' caches are encoded once, outside the timed region; steps over
    them are repeated until about ``budget_s`` seconds of timed work."""
    import numpy as np
    from threadpoolctl import threadpool_info
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import oracle
    import synth
    B, Hq, D, L, n = 64, 32, 128, 4096, 4
    t_all = time.perf_counter()
    chunks = []
    for c0 in range(0, B, n):
        k = synth.normal_f32(synth.rng(2, synth.T_K, 1000 + c0), (n, L, D))
        v = synth.normal_f32(synth.rng(2, synth.T_V, 1000 + c0), (n, L, D))
        q = synth.q_bf16(synth.rng(2, synth.T_Q, 1000 + c0), (n, Hq, D))
        kq, ks = oracle.quantize_rows(k[:, :-1])
        vq, vs = oracle.quantize_rows(v[:, :-1])
        kq = np.concatenate([kq, np.zeros((n, 1, D), np.int8)], axis=1)
        vq = np.concatenate([vq, np.zeros((n, 1, D), np.int8)], axis=1)
        ks = np.concatenate([ks, np.zeros((n, 1), np.float32)], axis=1)
        vs = np.concatenate([vs, np.zeros((n, 1), np.float32)], axis=1)
        chunks.append((k[:, -1].copy(), v[:, -1].copy(), q, kq, ks, vq, vs))
    lens = np.full(n, L, np.int32)
    done, t_work, steps = 0, 0.0, 0
    while t_work < budget_s:
        for knew, vnew, q, kq, ks, vq, vs in chunks:
            t0 = time.perf_counter()
            kq[:, -1], ks[:, -1] = oracle.quantize_rows(knew)
            vq[:, -1], vs[:, -1] = oracle.quantize_rows(vnew)
            for w in (0, 1024):
                oracle.decode_ref(q, kq, ks, vq, vs, lens, w)
            t_work += time.perf_counter() - t0
            done += n
        steps += 1
    info = threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    return {"value": done / t_work, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{steps} decode steps of all 64 sequences (append + global layer + window-1024 layer, "
                      f"4096 keys, 32 heads, D=128); numpy float64 oracle, {t_work:.1f} s of timed work",
            "host_cpus": len(os.sched_getaffinity(0)), "wall_s": time.perf_counter() - t_all}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (--gpus {args.gpus} requested); "
              "the decode path shards by sequence with no exchange, see the design notes.", file=sys.stderr)
        sys.exit(2)
    import torch
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import mqa_attention_int8_amd as m
    from mqa_attention_int8_amd import accounting as acct
    m.load_library()
    torch.cuda.init()
    stream = torch.cuda.Stream()
    if args.copy_calibration:
        x = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each_way": x.numel() * 4, "copies": 3}), file=sys.stderr)
    extra = {}
    if args.only in (None, "decode"):
        dec = bench_decode(torch, m, acct, args, stream)
    else:
        dec = None
    if not args.no_extra:
        if args.only in (None, "hybrid"):
            extra["hybrid_block"] = bench_hybrid(torch, m, acct, stream)
        if args.only in (None, "long"):
            extra["long_context"] = bench_long(torch, m, acct, stream)
        if args.only in (None, "prefill"):
            extra["prefill"] = bench_prefill(torch, m, acct, stream)
        if args.only in (None, "paged"):
            extra["paged"] = bench_paged(torch, m, acct, stream)
        if args.only in (None, "q8"):
            extra["q8"] = bench_q8(torch, m, acct, stream)
        if args.only in (None, "prefix_cache"):
            extra["prefix_cache"] = bench_prefix_cache(torch, m, stream)
        if args.only in (None, "ceilings"):
            extra["ceilings"] = bench_ceilings(torch, stream)
    if dec is None:
        print(json.dumps({"extra": extra}))
        return
    cpu = None if args.no_cpu else cpu_baseline(args.cpu_seconds)
    achieved = dec["global_GBps"]
    line = {
        "metric": METRIC, "value": dec["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": dec["steps_done"], "warmup": args.warmup, "ms_per_step": dec["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": "decode_B64_Hq32_D128_L4096: append + global layer + window-1024 layer "
                               "sharing one int8 KV buffer",
                   "B": 64, "Hq": 32, "D": 128, "seq_len": 4096, "windows": [0, 1024],
                   "kv_rotation_copies": dec["rotation_copies"], "graph_replay": dec["graph"]},
        "kv_read_GBps": dec["step_kv_GBps"], "kv_read_frac_hbm_peak": dec["step_kv_GBps"] / HBM_PEAK_GBPS,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": counted_traffic(),
                     "kernel": "global layer: mqa_decode_append (decode_partition_kernel + decode_merge_kernel)",
                     "algorithmic_bytes_per_launch": dec["global_kv_bytes"],
                     "avg_launch_us": dec["global_call_us"]},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
