#!/usr/bin/env python3
"""Benchmark of MQA int8-KV decode on one MI355X.

One step = one decode step of the hybrid 6-layer block: layer 0 is global
over buffer G, layers 1-3 use a 1024-key sliding window over buffer A,
layers 4-5 over buffer B (cross-layer KV sharing: the first layer of each
group appends the new token's K and V to its buffer in the same launch,
mqa_decode_append; the others read it, mqa_decode). B = 128 sequences with
ragged lengths uniform on [1024, 32768] (seeded), 32 query heads, one KV
head, head_dim 128.

Inputs are synthetic (seeded N(0,1) on the device, K/V encoded with the
library's own quantizer) and resident in HBM before timing. The three
buffers hold 3.2 GB, and one block step reads 744 MB of them, well beyond the
256 MB Infinity Cache; layers 2, 3 and 5 re-read the window a previous layer
of the step just read, which the cache may serve (the real schedule). Steps
are captured in a HIP graph so the timing is the GPU's, not Python's.

Prints ONE JSON line. ``value`` = decode tokens/s of the block step (B tokens
per step, attention only: no projections or MLP). ``roofline`` describes the
block's dominant call, the global layer (decode partition kernel with the
fused append + merge kernel). ``cpu_baseline`` times the CPU oracle on a
bounded sample of the same workload. ``extra`` holds the per-layer times
(flushed and in the block's order), the two-layer decode step (64 x 4096
keys), the long context (8 x 131072 keys), prefill, paged and int8-query
variants, the host prefix cache and the measured ceilings.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import statistics
import sys
import time

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, datasheet
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, datasheet
METRIC = "MQA int8-KV decode: KV-read HBM GB/s (% of peak) and decode tokens/s"
MIN_REPLAYS = 20                # individually timed replays behind every median
DTYPE = ("int8 KV with fp32 per-token scales; bf16 q; exact int8 operands on fp16 MFMA, "
         "P'' as fp16 hi+lo; fp32 softmax and accumulation; fp32 out")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50, help="block steps timed for the headline value")
    ap.add_argument("--warmup", type=int, default=10, help="untimed block steps before timing")
    ap.add_argument("--no-extra", action="store_true", help="only the headline workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU-baseline time budget")
    ap.add_argument("--only", choices=["hybrid", "hybrid_global", "decode", "long", "prefill", "paged", "q8",
                                       "prefix_cache", "ceilings"],
                    default=None, help="time a single workload (for profiling runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# timing
# ---------------------------------------------------------------------------

def capture(torch, fn, stream):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn()
    torch.cuda.synchronize()
    return g


def replay_times(torch, g, stream, reps, warm):
    """`warm` untimed replays, then `reps` replays each bracketed by its own
    HIP event pair on `stream` (the stream the graph's kernels run on).
    Returns the list of milliseconds per replay."""
    for _ in range(warm):
        g.replay()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(stream)
        g.replay()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def summary(ms_list, per=1):
    """Median, mean, min and max of per-replay times, divided by `per` calls per replay, in us."""
    us = sorted(m * 1e3 / per for m in ms_list)
    return {"median_us": statistics.median(us), "mean_us": statistics.fmean(us), "min_us": us[0],
            "max_us": us[-1], "replays": len(us)}


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


def rotation(bytes_per_copy):
    """Copies of a call's inputs that add up to >= 1 GiB (beyond the Infinity Cache)."""
    return max(2, math.ceil((1 << 30) / bytes_per_copy))


# ---------------------------------------------------------------------------
# headline: the hybrid 6-layer block (ragged 1024..32768 keys, 3 shared buffers)
# ---------------------------------------------------------------------------

def bench_hybrid(torch, m, acct, args, stream):
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import synth
    w = synth.HYBRID
    B, Hq, D = w.B, w.Hq, w.D
    lens = w.lens()
    L = int(lens.max())
    L_cap = (L + 31) // 32 * 32
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3)
    bufs = {name: make_decode_buffers(torch, m, B, L_cap, D, 1, gen)[0] for name in ("G", "A", "Bf")}
    seq_lens = torch.from_numpy(lens).cuda()
    q = [torch.randn((B, Hq, D), generator=gen, device="cuda").to(torch.bfloat16) for _ in w.layers]
    knew = torch.randn((B, D), generator=gen, device="cuda")
    vnew = torch.randn((B, D), generator=gen, device="cuda")
    out = torch.empty((B, Hq, D), device="cuda")
    ws = torch.zeros(max(max(m.mqa_decode_workspace_bytes(B, Hq, D, L, win),
                             m.mqa_decode_ragged_workspace_bytes(B, Hq, D, L, win)) for _, win in w.layers) + 16,
                     dtype=torch.uint8, device="cuda")
    owners = {}
    for li, (name, _) in enumerate(w.layers):
        owners.setdefault(name, li)

    def layer(li):
        # the global layer's lengths differ widely: it runs the balanced (ragged) plan; the window
        # layers see at most 1024 keys per sequence and keep the whole-window plan
        name, win = w.layers[li]
        kv = bufs[name]
        if win <= 0:
            if owners[name] == li:             # first layer of a sharing group writes the token (fused)
                m.mqa_decode_append_ragged(q[li], kv, knew, vnew, seq_lens, L, win, out=out, workspace=ws)
            else:
                m.mqa_decode_ragged(q[li], kv, seq_lens, L, win, out=out, workspace=ws)
        elif owners[name] == li:
            m.mqa_decode_append(q[li], kv, knew, vnew, seq_lens, L, win, out=out, workspace=ws)
        else:
            m.mqa_decode(q[li], kv, seq_lens, L, win, out=out, workspace=ws)

    def block():
        for li in range(len(w.layers)):
            layer(li)

    kv_layers = [acct.decode_kv_bytes(lens, win, D) for _, win in w.layers]
    kv_block = sum(kv_layers)
    res = {"workload": w.name, "B": B, "Hq": Hq, "D": D, "seq_len_range": [int(lens.min()), int(lens.max())],
           "layers": [{"buffer": n, "window": win} for n, win in w.layers], "kv_bytes_per_step": kv_block}
    with torch.cuda.stream(stream):
        for _ in range(2):
            block()
        torch.cuda.synchronize()
        g = capture(torch, block, stream)
        for _ in range(max(1, args.warmup)):
            g.replay()
        # headline: exactly `steps` block steps between two events, synchronised on both sides
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(args.steps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        ms_total = a.elapsed_time(b)
        res["steps_timed"] = args.steps
        res["ms_per_step"] = ms_total / args.steps
        res["block_step"] = summary(replay_times(torch, g, stream, max(MIN_REPLAYS, 20), 2))
        del g
        # the global layer's call alone (the dominant call): replays of one call
        gg = capture(torch, lambda: layer(0), stream)
        res["global_call"] = summary(replay_times(torch, gg, stream, max(MIN_REPLAYS, 30), 3))
        del gg
        # per layer: after a 1 GiB write (HBM figure) and right after the previous
        # layer of the block (the real schedule; layers 2, 3, 5 re-read a window)
        flush_buf = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        per_layer = []
        for li in range(len(w.layers)):
            fl, un = [], []
            for r in range(MIN_REPLAYS):
                for kind in ("flushed", "after_previous_layer"):
                    flush_buf.fill_(float(r))
                    if kind == "after_previous_layer":
                        layer((li - 1) % len(w.layers))
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    layer(li)
                    e1.record(stream)
                    (fl if kind == "flushed" else un).append((e0, e1))
            torch.cuda.synchronize()
            f = summary([x.elapsed_time(y) for x, y in fl])
            u = summary([x.elapsed_time(y) for x, y in un])
            name, win = w.layers[li]
            per_layer.append({"layer": li, "buffer": name, "window": win, "kv_bytes": kv_layers[li],
                              "flushed_us": f["median_us"], "after_previous_layer_us": u["median_us"],
                              "flushed_GBps": kv_layers[li] / (f["median_us"] * 1e-6) / 1e9,
                              "after_previous_layer_GBps": kv_layers[li] / (u["median_us"] * 1e-6) / 1e9})
        del flush_buf
    res["per_layer"] = per_layer
    res["tokens_per_s"] = B / (res["ms_per_step"] * 1e-3)
    res["kv_GBps"] = kv_block / (res["ms_per_step"] * 1e-3) / 1e9
    res["global_kv_bytes"] = kv_layers[0]
    res["global_GBps"] = kv_layers[0] / (res["global_call"]["mean_us"] * 1e-6) / 1e9
    res["note"] = ("per-layer times are eager calls bracketed by events, each after a 1 GiB write (flushed) "
                   "or after the block's previous layer, so they include launch gaps the graph-replayed block "
                   "step does not have; the block step is one graph replay")
    return res


def bench_hybrid_global_only(torch, m, stream, calls=8):
    """The hybrid block's global-layer call alone, a few times (for counter runs)."""
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import synth
    w = synth.HYBRID
    B, Hq, D = w.B, w.Hq, w.D
    lens = w.lens()
    L = int(lens.max())
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3)
    kv = make_decode_buffers(torch, m, B, (L + 31) // 32 * 32, D, 1, gen)[0]
    seq_lens = torch.from_numpy(lens).cuda()
    q = torch.randn((B, Hq, D), generator=gen, device="cuda").to(torch.bfloat16)
    knew = torch.randn((B, D), generator=gen, device="cuda")
    vnew = torch.randn((B, D), generator=gen, device="cuda")
    out = torch.empty((B, Hq, D), device="cuda")
    ws = m.ragged_workspace(B, Hq, D, L, 0)
    with torch.cuda.stream(stream):
        for _ in range(calls):
            m.mqa_decode_append_ragged(q, kv, knew, vnew, seq_lens, L, 0, out=out, workspace=ws)
        torch.cuda.synchronize()
    return {"workload": w.name + " global layer", "calls": calls}


# ---------------------------------------------------------------------------
# the two-layer decode step: 64 sequences x 4096 keys, global + window 1024
# ---------------------------------------------------------------------------

def bench_decode(torch, m, acct, stream):
    B, Hq, D, L = 64, 32, 128, 4096
    windows = (0, 1024)
    R = rotation(B * L * (2 * D + 8))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2)
    bufs = make_decode_buffers(torch, m, B, L, D, R, gen)
    seq_lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    q = [[torch.randn((B, Hq, D), generator=gen, device="cuda").to(torch.bfloat16) for _ in windows]
         for _ in range(R)]
    knew = [torch.randn((B, D), generator=gen, device="cuda") for _ in range(R)]
    vnew = [torch.randn((B, D), generator=gen, device="cuda") for _ in range(R)]
    outs = [torch.empty((B, Hq, D), device="cuda") for _ in windows]
    ws = [m.decode_workspace(B, Hq, D, L, w) for w in windows]

    def step(r):
        # the global layer owns the buffer: it appends the new token (fused), the window layer reads it
        m.mqa_decode_append(q[r][0], bufs[r], knew[r], vnew[r], seq_lens, L, windows[0], out=outs[0],
                            workspace=ws[0])
        m.mqa_decode(q[r][1], bufs[r], seq_lens, L, windows[1], out=outs[1], workspace=ws[1])

    def period():
        for r in range(R):
            step(r)

    def global_only():
        for r in range(R):
            m.mqa_decode_append(q[r][0], bufs[r], knew[r], vnew[r], seq_lens, L, 0, out=outs[0], workspace=ws[0])

    def window_only():
        for r in range(R):
            m.mqa_decode(q[r][1], bufs[r], seq_lens, L, windows[1], out=outs[1], workspace=ws[1])

    res = {"workload": "decode_B64_Hq32_D128_L4096: append + global layer + window-1024 layer sharing one "
                       "int8 KV buffer", "rotation_copies": R}
    with torch.cuda.stream(stream):
        period()
        torch.cuda.synchronize()
        for name, fn in (("step", period), ("global_call", global_only), ("window_call", window_only)):
            g = capture(torch, fn, stream)
            res[name] = summary(replay_times(torch, g, stream, MIN_REPLAYS, 3), per=R)
            del g
    kv_g = acct.decode_kv_bytes([L] * B, 0, D)
    kv_w = acct.decode_kv_bytes([L] * B, 1024, D)
    res["tokens_per_s"] = B / (res["step"]["median_us"] * 1e-6)
    res["global_kv_bytes"], res["window_kv_bytes"] = kv_g, kv_w
    res["global_GBps"] = kv_g / (res["global_call"]["median_us"] * 1e-6) / 1e9
    res["window_GBps"] = kv_w / (res["window_call"]["median_us"] * 1e-6) / 1e9
    res["global_frac_hbm_peak"] = res["global_GBps"] / HBM_PEAK_GBPS
    res["window_frac_hbm_peak"] = res["window_GBps"] / HBM_PEAK_GBPS
    res["global_traffic_bytes"] = counted_traffic("decode_global_traffic.json")
    return res


def bench_long(torch, m, acct, stream):
    B, Hq, D, L = 8, 32, 128, 131072
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    R = rotation(B * L * (2 * D + 8))
    bufs = make_decode_buffers(torch, m, B, L, D, R, gen)
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
        g = capture(torch, calls, stream)
        s = summary(replay_times(torch, g, stream, MIN_REPLAYS, 2), per=len(bufs))
        del g
    kv = acct.decode_kv_bytes([L] * B, 0, D)
    return {"workload": "long_decode_B8_Hq32_D128_L131072", "call": s, "rotation_copies": R,
            "tokens_per_s": B / (s["median_us"] * 1e-6), "kv_GBps": kv / (s["median_us"] * 1e-6) / 1e9,
            "frac_hbm_peak": kv / (s["median_us"] * 1e-6) / 1e9 / HBM_PEAK_GBPS}


# ---------------------------------------------------------------------------
# ceilings: one-pass streaming and dense MFMA on this GPU
# ---------------------------------------------------------------------------

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
    """Achievable ceilings on this GPU: one-pass HBM streaming of the decode
    calls' byte counts (window layer 17.3 MB, hybrid window layer 34.6 MB,
    global layer 69.2 MB) and of 1 GiB, each over >= 1 GiB of rotated copies
    so no cache holds them, and dense bf16 MFMA throughput."""
    lib = load_ceilings()
    res = {}
    blocks = 4096                     # 16 KB chunks per work-group; the fastest of 2048-16384 on 69 MB
    partial = torch.empty(blocks, dtype=torch.int32, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    for name, nbytes in (("stream_read_17MB", 17_301_504), ("stream_read_35MB", 34_603_008),
                         ("stream_read_69MB", 69_206_016), ("stream_read_1GiB", 1 << 30)):
        R = rotation(nbytes)
        bufs = [torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda", generator=gen)
                for _ in range(R)]
        torch.cuda.synchronize()          # the fills ran on the default stream
        with torch.cuda.stream(stream):
            # every word read exactly once: the partial sums add up to the buffer's sum mod 2^32
            rc = lib.mqa_ceiling_stream_read(bufs[0].data_ptr(), nbytes, blocks, partial.data_ptr(),
                                             stream.cuda_stream)
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
            g = capture(torch, period, stream)
            s = summary(replay_times(torch, g, stream, MIN_REPLAYS, 3), per=R)
            del g
        res[name] = {"bytes": nbytes, "us": s["median_us"], "GBps": nbytes / (s["median_us"] * 1e-6) / 1e9,
                     "frac_hbm_peak": nbytes / (s["median_us"] * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                     "rotation_copies": R, "blocks": blocks}
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
        g = capture(torch, mm, stream)
        s = summary(replay_times(torch, g, stream, MIN_REPLAYS, 20))
        del g
    fl = lib.mqa_ceiling_mfma_bf16_flops(mb, iters)
    tf = fl / (s["median_us"] * 1e-6) / 1e12
    res["mfma_bf16"] = {"flops_per_launch": fl, "us": s["median_us"], "TFLOPs": tf,
                        "frac_bf16_peak": tf / BF16_PEAK_TFLOPS,
                        "kernel": "v_mfma_f32_16x16x32_bf16, 8 independent chains per wave, 8 waves per "
                                  f"work-group, {mb} work-groups"}
    return res


# ---------------------------------------------------------------------------
# other paths of the library
# ---------------------------------------------------------------------------

def bench_paged(torch, m, acct, stream):
    """Paged layouts on the decode step's shape: the global layer (fused
    append) over a pool of 32-token blocks in shuffled order, and a window-1024
    layer over a ring of 1024 slots per sequence; each against the same call on
    contiguous buffers, timed in this run."""
    B, Hq, D, L, bs, W = 64, 32, 128, 4096, 32, 1024
    TL = L // bs
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    R = rotation(B * L * (2 * D + 8))
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
    Rr = rotation(B * W * (2 * D + 8))
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
            g = capture(torch, fn, stream)
            res[name] = summary(replay_times(torch, g, stream, MIN_REPLAYS, 2), per=n)["median_us"]
            del g
    kv_g = acct.decode_kv_bytes([L] * B, 0, D)
    kv_w = acct.decode_kv_bytes([L] * B, W, D)
    res["global_paged_GBps"] = kv_g / (res["global_paged_us"] * 1e-6) / 1e9
    res["window_ring_GBps"] = kv_w / (res["window_ring_us"] * 1e-6) / 1e9
    res["window_buffer_bytes_per_seq"] = {"ring": W * (2 * D + 8), "contiguous": L * (2 * D + 8)}
    return res


def bench_q8(torch, m, acct, stream):
    """The two-layer decode step with int8 queries (int8 MFMA for Q K^T; the
    query rows encoded by kv_quantize_int8 outside the timed region, as a
    projection with int8 outputs would deliver them), against the bf16-query
    step in the same run."""
    B, Hq, D, L = 64, 32, 128, 4096
    windows = (0, 1024)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(8)
    R = rotation(B * L * (2 * D + 8))
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
            g = capture(torch, fn, stream)
            res[name] = summary(replay_times(torch, g, stream, MIN_REPLAYS, 2), per=R)["median_us"]
            del g
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
    with torch.cuda.stream(stream):
        for name, fn in (("store", m.mqa_kv_blocks_to_host), ("restore", m.mqa_kv_blocks_to_device)):
            for _ in range(3):
                fn(bufs, 1, 0, slots, bs, pool, stream=stream)
            torch.cuda.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(MIN_REPLAYS)]
            for a, b in ev:
                a.record(stream)
                fn(bufs, 1, 0, slots, bs, pool, stream=stream)
                b.record(stream)
            torch.cuda.synchronize()
            us = statistics.median(a.elapsed_time(b) for a, b in ev) * 1e3
            res[name + "_us"] = us
            res[name + "_GBps"] = nbytes / (us * 1e-6) / 1e9
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
            g = capture(torch, call, stream)
            # the first untimed replay is timed too (cold: right after an idle GPU)
            cold = replay_times(torch, g, stream, 1, 0)[0]
            # then ~0.1 s of untimed replays: the first ~50 ms of back-to-back calls
            # of this MFMA-bound kernel run up to ~15% slower than the settled rate
            s = summary(replay_times(torch, g, stream, MIN_REPLAYS, 80 if win == 0 else 200))
            del g
            fl = acct.prefill_flops([P] * B, C, win, Hq, D)
            tf = fl / (s["median_us"] * 1e-6) / 1e12
            res[f"W{win}"] = {"ms": s["median_us"] * 1e-3, "min_ms": s["min_us"] * 1e-3,
                              "max_ms": s["max_us"] * 1e-3, "cold_first_call_ms": cold, "flops": fl,
                              "TFLOPs": tf, "frac_bf16_peak": tf / BF16_PEAK_TFLOPS,
                              "cold_frac_bf16_peak": fl / (cold * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}
    return res


def counted_traffic(record="hybrid_global_traffic.json"):
    """HBM bytes per launch of a call from a committed rocprofv3 counter
    summary, or None when the sources it names have changed since the
    counters were taken."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", record)
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


def host_description():
    model = None
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return model or platform.processor() or "unknown"


def cpu_baseline(budget_s: float):
    """The oracle (numpy, float64) on a bounded sample of the hybrid block.

    Per sequence, the timed work is what one block step does: encode the new
    token's K and V rows into the three buffers' owners, then the six layers
    (the global one over the sequence's whole context, the five window layers
    over its last 1024 keys). Every sequence's cache is generated and encoded
    once, outside the timed region; then passes over the batch are timed,
    sequence by sequence, until about ``budget_s`` seconds of timed work."""
    import numpy as np
    from threadpoolctl import threadpool_info
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import oracle
    import synth
    w = synth.HYBRID
    Hq, D = w.Hq, w.D
    lens = w.lens()
    t_all = time.perf_counter()
    cases = []
    for b in range(w.B):
        n = int(lens[b])
        g = synth.rng(3, synth.T_K, 5000 + b)
        bufs = {}
        for name in ("G", "A", "Bf"):
            rows = n if name == "G" else min(n, 1024)
            k = synth.normal_f32(g, (1, rows, D))
            v = synth.normal_f32(g, (1, rows, D))
            kq, ks = oracle.quantize_rows(k)
            vq, vs = oracle.quantize_rows(v)
            bufs[name] = (kq, ks, vq, vs)
        qs = [synth.q_bf16(g, (1, Hq, D)) for _ in w.layers]
        knew, vnew = synth.normal_f32(g, (1, D)), synth.normal_f32(g, (1, D))
        cases.append((n, bufs, qs, knew, vnew))
    done, t_work, keys = 0, 0.0, 0
    while t_work < budget_s:
        for n, bufs, qs, knew, vnew in cases:
            t0 = time.perf_counter()
            for name in ("G", "A", "Bf"):             # the owners' fused append: the new token is the last row
                kq, ks, vq, vs = bufs[name]
                kq[0, -1], ks[0, -1] = oracle.quantize_rows(knew[0])
                vq[0, -1], vs[0, -1] = oracle.quantize_rows(vnew[0])
            for li, (name, win) in enumerate(w.layers):
                kq, ks, vq, vs = bufs[name]
                rows = kq.shape[1]
                oracle.decode_ref(qs[li], kq, ks, vq, vs, np.array([rows], np.int32), win)
            t_work += time.perf_counter() - t0
            done += 1
            keys += n + 5 * min(n, 1024)
            if t_work >= budget_s:
                break
    info = threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    blas = [{"api": i.get("internal_api"), "version": i.get("version"), "threads": i.get("num_threads")}
            for i in info]
    return {"value": done / t_work, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} sequence-steps over the {w.B} sequences of the hybrid block (each: append + 1 "
                      f"global layer over the whole context + 5 window-1024 layers; {keys} visible keys in all), "
                      f"numpy float64 oracle, {t_work:.1f} s of timed work",
            "cpu_model": host_description(), "host_cpus": len(os.sched_getaffinity(0)),
            "numpy": np.__version__, "blas": blas, "wall_s": time.perf_counter() - t_all}


# `--only` value of each entry of `extra` whose key differs from its name
ONLY_KEY = {"decode_step_B64_L4096": "decode", "long_context": "long"}
EXTRA_NAMES = ("decode_step_B64_L4096", "long_context", "prefill", "paged", "q8", "prefix_cache", "ceilings")


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
        del x, y
    if args.only == "hybrid_global":
        print(json.dumps({"extra": {"hybrid_global": bench_hybrid_global_only(torch, m, stream)}}))
        return
    hyb = bench_hybrid(torch, m, acct, args, stream) if args.only in (None, "hybrid") else None
    extra = {}
    if not args.no_extra:
        fns = {"decode_step_B64_L4096": lambda: bench_decode(torch, m, acct, stream),
               "long_context": lambda: bench_long(torch, m, acct, stream),
               "prefill": lambda: bench_prefill(torch, m, acct, stream),
               "paged": lambda: bench_paged(torch, m, acct, stream),
               "q8": lambda: bench_q8(torch, m, acct, stream),
               "prefix_cache": lambda: bench_prefix_cache(torch, m, stream),
               "ceilings": lambda: bench_ceilings(torch, stream)}
        for name in EXTRA_NAMES:
            fn = fns[name]
            if args.only in (None, ONLY_KEY.get(name, name)):
                extra[name] = fn()
                print(f"bench: {name} done", file=sys.stderr, flush=True)
    if hyb is None:
        print(json.dumps({"extra": extra}))
        return
    cpu = None if args.no_cpu else cpu_baseline(args.cpu_seconds)
    g = hyb["global_call"]
    line = {
        "metric": METRIC, "value": hyb["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": hyb["steps_timed"], "warmup": args.warmup, "ms_per_step": hyb["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": DTYPE,
        "data": "synthetic",
        "config": {"workload": "hybrid 6-layer block decode step: 1 global + 5 window-1024 layers over 3 shared "
                               "int8 KV buffers (G: layer 0; A: layers 1-3; B: layers 4-5), B=128 ragged "
                               "1024..32768 keys, Hq=32, 1 KV head, D=128",
                   "B": hyb["B"], "Hq": hyb["Hq"], "D": hyb["D"], "seq_len_range": hyb["seq_len_range"],
                   "layers": hyb["layers"], "graph_replay": True},
        "kv_read_GBps": hyb["kv_GBps"], "kv_read_frac_hbm_peak": hyb["kv_GBps"] / HBM_PEAK_GBPS,
        "block_step_median_us": hyb["block_step"]["median_us"],
        "roofline": {"bound": "hbm", "achieved": hyb["global_GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": hyb["global_GBps"] / HBM_PEAK_GBPS, "traffic": counted_traffic(),
                     "kernel": "global layer of the block: mqa_decode_append_ragged (decode_partition_kernel, "
                               "which plans its own range, + decode_merge_kernel)",
                     "algorithmic_bytes_per_launch": hyb["global_kv_bytes"],
                     "avg_launch_us": g["mean_us"], "median_launch_us": g["median_us"],
                     "launch_us_min_max": [g["min_us"], g["max_us"]], "replays": g["replays"]},
        "cpu_baseline": cpu,
        "per_layer": hyb["per_layer"],
        "extra": extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
