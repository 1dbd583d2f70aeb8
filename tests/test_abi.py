"""The C-ABI library on the host (no GPU needed): exports, status strings,
argument validation and workspace sizing. Only invalid-argument paths are
called, which return before any HIP call; no kernel is launched."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mqa_int8.h")


@pytest.fixture(scope="module")
def lib():
    import mqa_attention_int8_amd as m
    return m.load_library()


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_every_declared_function_is_exported(lib):
    names = declared_functions()
    assert {"kv_quantize_int8", "mqa_decode", "mqa_decode_append", "mqa_prefill_chunk",
            "mqa_decode_workspace_bytes", "mqa_status_string", "kv_quantize_int8_paged", "mqa_decode_paged",
            "mqa_decode_append_paged", "mqa_prefill_chunk_paged", "mqa_decode_paged_workspace_bytes",
            "mqa_decode_q8", "mqa_decode_append_q8"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in mqa_int8.h but not exported"


def test_ceilings_library_exports_its_header():
    """libmqa_ceilings.so (the benchmark's measurement kernels) loads and
    exports what csrc/mqa_ceilings.h declares; only invalid arguments are
    passed, which return before any launch."""
    path = os.path.join(ROOT, "mqa_attention_int8_amd", "libmqa_ceilings.so")
    assert os.path.exists(path), "build first"
    cl = ctypes.CDLL(path)
    names = declared_functions(os.path.join(ROOT, "mqa_attention_int8_amd", "csrc", "mqa_ceilings.h"))
    assert set(names) == {"mqa_ceiling_stream_read", "mqa_ceiling_mfma_bf16", "mqa_ceiling_mfma_bf16_flops"}
    for n in names:
        assert hasattr(cl, n), f"{n} declared in mqa_ceilings.h but not exported"
    cl.mqa_ceiling_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p,
                                           ctypes.c_void_p]
    cl.mqa_ceiling_mfma_bf16.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    cl.mqa_ceiling_mfma_bf16_flops.argtypes = [ctypes.c_int32, ctypes.c_int32]
    cl.mqa_ceiling_mfma_bf16_flops.restype = ctypes.c_double
    fake = 1 << 20
    assert cl.mqa_ceiling_stream_read(None, 64, 4, fake, None) == 1
    assert cl.mqa_ceiling_stream_read(fake, 60, 4, fake, None) == 2        # not a multiple of 16
    assert cl.mqa_ceiling_stream_read(fake + 8, 64, 4, fake, None) == 2    # misaligned
    assert cl.mqa_ceiling_mfma_bf16(0, 4, fake, None) == 2
    assert cl.mqa_ceiling_mfma_bf16(4, 4, None, None) == 1
    # 8 waves x iters x 8 MFMAs of 16 x 16 x 32 multiply-adds per work-group
    assert cl.mqa_ceiling_mfma_bf16_flops(3, 5) == 3 * 8 * 5 * 8 * 16 * 16 * 32 * 2


def test_one_hip_runtime(lib):
    import mqa_attention_int8_amd as m
    assert len(m.binding.hip_runtimes_mapped()) == 1


def test_status_strings(lib):
    import mqa_attention_int8_amd as m
    for code in range(7):
        assert m.mqa_status_string(code)
    assert m.mqa_status_string(99) == "unknown status"


FAKE = 0x10000  # a 16-byte aligned address that is never dereferenced


def kv(L_cap=64, k=FAKE, ks=FAKE):
    from mqa_attention_int8_amd.binding import mqa_kv_view
    return mqa_kv_view(k, FAKE, ks, FAKE, L_cap)


def decode(lib, **kw):
    a = dict(q=FAKE, kv=kv(), seq=FAKE, max_len=64, B=2, Hq=8, D=128, W=0, scale=0.1, out=FAKE,
             ws=None, ws_bytes=0)
    a.update(kw)
    v = a["kv"]
    return lib.mqa_decode(a["q"], ctypes.byref(v) if v is not None else None, a["seq"], a["max_len"], a["B"],
                          a["Hq"], a["D"], a["W"], a["scale"], a["out"], a["ws"], a["ws_bytes"], None)


def test_decode_validation(lib):
    assert decode(lib, q=None) == 1
    assert decode(lib, kv=None) == 1
    assert decode(lib, kv=kv(k=None)) == 1
    assert decode(lib, B=0) == 2
    assert decode(lib, max_len=-1) == 2
    assert decode(lib, max_len=65) == 2                      # beyond L_cap
    assert decode(lib, D=96) == 3
    assert decode(lib, Hq=65) == 3
    assert decode(lib, q=FAKE + 8) == 4
    assert decode(lib, kv=kv(L_cap=62), max_len=60) == 4     # scales read 4 keys at a time
    assert decode(lib, kv=kv(L_cap=80), max_len=60) == 4     # whole 32-row tiles: L_cap a multiple of 32
    assert decode(lib, kv=kv(ks=FAKE + 4)) == 4
    # needs a workspace (many partitions) but none given
    assert decode(lib, kv=kv(L_cap=1 << 16), max_len=1 << 16, B=64) == 5
    # one sequence's K rows must stay below 4 GiB (32-bit offsets)
    assert decode(lib, kv=kv(L_cap=1 << 25), max_len=64, D=128) == 2
    assert decode(lib, kv=kv(L_cap=1 << 26), max_len=64, D=64) == 2


def test_noalloc_decode_rejects_before_any_launch(lib):
    """The allocation-free decode validates like mqa_decode and rejects calls
    whose partition states would not fit in its static 8 MiB array; every
    case returns before any HIP call."""
    def call(**kw):
        a = dict(q=FAKE, kv=kv(), seq=FAKE, max_len=64, B=2, Hq=8, D=128, W=0, scale=0.1, out=FAKE)
        a.update(kw)
        v = a["kv"]
        return lib.mqa_decode_noalloc(a["q"], ctypes.byref(v) if v is not None else None, a["seq"], a["max_len"],
                                      a["B"], a["Hq"], a["D"], a["W"], a["scale"], a["out"], None)
    assert call(q=None) == 1
    assert call(kv=None) == 1
    assert call(B=0) == 2
    assert call(max_len=65) == 2
    assert call(D=96) == 3
    assert call(kv=kv(L_cap=80), max_len=60) == 4
    import mqa_attention_int8_amd as m
    # 127 sequences x 64 heads x 65536 keys: two partitions per sequence, 8,453,120 bytes of states
    need = m.mqa_decode_workspace_bytes(127, 64, 128, 65536, 0)
    assert need > (8 << 20)
    assert call(kv=kv(L_cap=65536), max_len=65536, B=127, Hq=64) == 5


def test_quantize_validation(lib):
    assert lib.kv_quantize_int8(None, FAKE, FAKE, FAKE, 1, 1, 128, 8, None) == 1
    assert lib.kv_quantize_int8(FAKE, FAKE, FAKE, FAKE, 1, 9, 128, 8, None) == 2
    assert lib.kv_quantize_int8(FAKE, FAKE, FAKE, FAKE, 1, 1, 32, 8, None) == 3
    assert lib.kv_quantize_int8(FAKE + 4, FAKE, FAKE, FAKE, 1, 1, 128, 8, None) == 4


def test_prefill_validation(lib):
    v = kv(L_cap=100)
    big = 1 << 30
    f = lambda **k: lib.mqa_prefill_chunk(k.get("q", FAKE), ctypes.byref(v), FAKE, k.get("P", 10), 2,
                                          k.get("C", 20), k.get("Hq", 8), k.get("D", 128), 0, 0.1,
                                          k.get("out", FAKE), k.get("ws", FAKE), k.get("wsb", big), None)
    assert f(q=None) == 1
    assert f(C=0) == 2
    assert f(P=81) == 2          # P + C > L_cap
    assert f(D=80) == 3
    assert f(out=FAKE + 2) == 4
    assert f(ws=None) == 5
    assert f(wsb=16) == 5
    # a sequence's staged tiles must stay below 2^31 bytes: 63550 tiles of
    # 33792 bytes at D = 128 is the last size that fits
    v = kv(L_cap=1 << 24)
    assert f(P=63551 * 64 - 20, wsb=1 << 62) == 2
    assert f(P=123362 * 64 - 20, D=64, wsb=1 << 62) == 2   # 17408-byte tiles at D = 64
    assert f(ws=FAKE + 8) == 4
    need = lib.mqa_prefill_workspace_bytes(2, 20, 128, 10)
    assert need >= 2 * 64 * 128 * 2 * 2      # at least one converted K and V tile per sequence
    assert lib.mqa_prefill_workspace_bytes(2, 0, 128, 10) == 0


def test_workspace_sizes(lib):
    import mqa_attention_int8_amd as m
    # a single partition needs no workspace
    assert m.mqa_decode_workspace_bytes(1, 8, 64, 128, 0) == 0
    # many partitions: at least one fp32 accumulator + (m, l) per partition and head
    for B, Hq, D, L, W in ((64, 32, 128, 4096, 0), (8, 32, 128, 131072, 0), (128, 32, 128, 32768, 1024)):
        n = m.mqa_decode_workspace_bytes(B, Hq, D, L, W)
        assert n == 0 or n >= 2 * B * Hq * (D + 2) * 4
    assert m.mqa_decode_workspace_bytes(8, 32, 128, 131072, 0) > 0
    assert m.mqa_decode_workspace_bytes(0, 32, 128, 4096, 0) == 0      # invalid -> 0
    # the balanced plan counts tiles plus 40 per sequence start in 32-bit
    # integers: B * (ceil(L / 32) + 1 + 40) must stay below 2^31
    assert m.mqa_decode_ragged_workspace_bytes(65535, 8, 64, 32727 * 32, 0) > 0
    assert m.mqa_decode_ragged_workspace_bytes(65535, 8, 64, 32727 * 32 + 1, 0) == 0


def test_accounting_matches_oracle():
    import numpy as np
    import oracle
    from mqa_attention_int8_amd import accounting as acct
    import synth
    lens = synth.HYBRID.lens()
    for W in (0, 1024, 1):
        assert acct.decode_kv_bytes(lens, W, 128) == oracle.decode_visible_keys(lens, W) * oracle.int8_kv_bytes_per_key(128)
    for W in (0, 1024, 7):
        assert acct.prefill_pairs([8192] * 3 + [5], 512, W) == oracle.prefill_visible_pairs([8192] * 3 + [5], 512, W)
    assert acct.decode_kv_bytes(np.full(64, 4096), 0, 128) == 69_206_016


def append(lib, **kw):
    from mqa_attention_int8_amd.binding import mqa_kv_cache
    a = dict(q=FAKE, kv=mqa_kv_cache(FAKE, FAKE, FAKE, FAKE, 64), kn=FAKE, vn=FAKE, seq=FAKE, max_len=64, B=2,
             Hq=8, D=128, W=0, scale=0.1, out=FAKE, ws=None, ws_bytes=0)
    a.update(kw)
    v = a["kv"]
    return lib.mqa_decode_append(a["q"], ctypes.byref(v) if v is not None else None, a["kn"], a["vn"], a["seq"],
                                 a["max_len"], a["B"], a["Hq"], a["D"], a["W"], a["scale"], a["out"], a["ws"],
                                 a["ws_bytes"], None)


def test_decode_append_validation(lib):
    """mqa_decode_append rejects bad arguments on the host, before any launch."""
    assert append(lib, kn=None) == 1                 # MQA_ERR_NULL
    assert append(lib, vn=None) == 1
    assert append(lib, kv=None) == 1
    assert append(lib, kn=FAKE + 2) == 4             # MQA_ERR_ALIGN (rows are fp32)
    assert append(lib, D=96) == 3                    # MQA_ERR_UNSUPPORTED
    assert append(lib, max_len=65) == 2              # MQA_ERR_SHAPE (beyond L_cap)
    assert append(lib, B=0) == 2
    from mqa_attention_int8_amd.binding import mqa_kv_cache
    assert append(lib, kv=mqa_kv_cache(FAKE, FAKE, FAKE, FAKE, 62), max_len=60) == 4   # scales 4 at a time
    # many partitions need a workspace
    assert append(lib, B=8, max_len=60000, kv=mqa_kv_cache(FAKE, FAKE, FAKE, FAKE, 65536)) == 5


def paged(bs=32, TL=8, nb=64, table=FAKE, k=FAKE, ks=FAKE):
    from mqa_attention_int8_amd.binding import mqa_kv_paged
    return mqa_kv_paged(k, FAKE, ks, FAKE, table, bs, TL, nb)


def decode_paged(lib, **kw):
    a = dict(q=FAKE, kv=paged(), seq=FAKE, max_len=64, B=2, Hq=8, D=128, W=0, scale=0.1, out=FAKE,
             ws=None, ws_bytes=0)
    a.update(kw)
    v = a["kv"]
    return lib.mqa_decode_paged(a["q"], ctypes.byref(v) if v is not None else None, a["seq"], a["max_len"],
                                a["B"], a["Hq"], a["D"], a["W"], a["scale"], a["out"], a["ws"], a["ws_bytes"], None)


def test_decode_paged_validation(lib):
    NULL, SHAPE, UNSUP, ALIGN = 1, 2, 3, 4
    assert decode_paged(lib, kv=None) == NULL
    assert decode_paged(lib, kv=paged(table=None)) == NULL
    for bs in (16, 48, 8192, 0):
        assert decode_paged(lib, kv=paged(bs=bs)) == SHAPE, bs
    assert decode_paged(lib, kv=paged(TL=0)) == SHAPE
    assert decode_paged(lib, kv=paged(nb=0)) == SHAPE
    assert decode_paged(lib, kv=paged(k=FAKE + 8)) == ALIGN
    assert decode_paged(lib, kv=paged(ks=FAKE + 4)) == ALIGN
    assert decode_paged(lib, kv=paged(table=FAKE + 2)) == ALIGN
    assert decode_paged(lib, D=96) == UNSUP
    # the table (8 blocks of 32 = 256 positions) wraps for longer sequences:
    # only a windowed layer whose window fits in those 256 positions may read it
    assert decode_paged(lib, max_len=257, W=0) == SHAPE
    assert decode_paged(lib, max_len=4096, W=257) == SHAPE
    # a window that fits passes validation and then needs its workspace
    assert lib.mqa_decode_paged_workspace_bytes(2, 8, 128, 4096, 256, 32) > 0
    assert decode_paged(lib, max_len=4096, W=256, ws=None, ws_bytes=0) == 5
    assert lib.mqa_decode_paged_workspace_bytes(2, 8, 128, 4096, 0, 48) == 0


def test_decode_append_paged_validation(lib):
    kvp = paged()
    r = lib.mqa_decode_append_paged(FAKE, ctypes.byref(kvp), None, FAKE, FAKE, 64, 2, 8, 128, 0, 0.1, FAKE, None,
                                    0, None)
    assert r == 1
    r = lib.mqa_decode_append_paged(FAKE, ctypes.byref(kvp), FAKE + 2, FAKE, FAKE, 64, 2, 8, 128, 0, 0.1, FAKE,
                                    None, 0, None)
    assert r == 4


def test_quantize_paged_validation(lib):
    kvp = paged()
    q = lambda **kw: lib.kv_quantize_int8_paged(kw.get("k", FAKE), FAKE, ctypes.byref(kw.get("kv", kvp)), FAKE,
                                                kw.get("B", 2), kw.get("T", 4), kw.get("D", 128), None)
    assert q(k=None) == 1
    assert q(T=0) == 2
    assert q(T=257) == 2      # one call would write a pool row twice
    assert q(D=32) == 3
    assert q(k=FAKE + 4) == 4
    assert q(kv=paged(bs=100)) == 2


def test_prefill_paged_validation(lib):
    def pf(kvp, max_prefix=64, C=16, W=0, ws=FAKE, ws_bytes=1 << 40):
        return lib.mqa_prefill_chunk_paged(FAKE, ctypes.byref(kvp), FAKE, max_prefix, 2, C, 8, 128, W, 0.1, FAKE,
                                           ws, ws_bytes, None)
    assert pf(paged(table=None)) == 1
    assert pf(paged(), max_prefix=250, C=16, W=0) == 2          # global layer past the table
    assert pf(paged(), max_prefix=1000, C=16, W=242) == 2       # W + C - 1 = 257 > 256
    assert pf(paged(), max_prefix=64, C=16, ws=None, ws_bytes=0) == 5


def test_decode_q8_validation(lib):
    v = kv()
    d = lambda **kw: lib.mqa_decode_q8(kw.get("q8", FAKE), kw.get("qs", FAKE), ctypes.byref(v), FAKE,
                                       kw.get("max_len", 64), 2, kw.get("Hq", 8), kw.get("D", 128), 0, 0.1, FAKE,
                                       None, 0, None)
    assert d(q8=None) == 1
    assert d(qs=None) == 1
    assert d(q8=FAKE + 8) == 4
    assert d(qs=FAKE + 2) == 4
    assert d(D=96) == 3
    assert d(Hq=65) == 3
    assert d(max_len=65) == 2
    c = __import__("mqa_attention_int8_amd").binding.mqa_kv_cache(FAKE, FAKE, FAKE, FAKE, 64)
    assert lib.mqa_decode_append_q8(FAKE, FAKE, ctypes.byref(c), None, FAKE, FAKE, 64, 2, 8, 128, 0, 0.1, FAKE,
                                    None, 0, None) == 1


def test_kv_transfer_validation(lib):
    from mqa_attention_int8_amd.binding import mqa_kv_view, mqa_kv_cache
    views = (mqa_kv_view * 2)(kv(L_cap=256), kv(L_cap=256))
    slots = (ctypes.c_int64 * 4)(0, 1, 2, 3)
    t = lambda **kw: lib.mqa_kv_blocks_to_host(kw.get("views", views), kw.get("n_bufs", 2), kw.get("B", 2),
                                               kw.get("b", 0), kw.get("first", 0),
                                               kw.get("n", 4), kw.get("bs", 32), kw.get("D", 128),
                                               kw.get("slots", slots), kw.get("pool", FAKE), kw.get("pool_slots", 8),
                                               None)
    assert t(pool=None) == 1
    assert t(slots=None) == 1
    assert t(n_bufs=0) == 2 and t(n_bufs=9) == 2
    assert t(bs=24) == 2
    assert t(first=5) == 2                  # (5 + 4) * 32 > L_cap
    assert t(pool_slots=3) == 2             # slot 3 outside the pool
    assert t(D=96) == 3
    assert t(pool=FAKE + 8) == 4
    assert t(b=2) == 2 and t(b=-1) == 2 and t(B=0) == 2
    assert t(n=0) == 0                      # nothing to copy: no launch
    caches = (mqa_kv_cache * 1)(mqa_kv_cache(FAKE, FAKE, FAKE, FAKE, 64))
    assert lib.mqa_kv_blocks_to_device(caches, 1, 1, 0, 0, 4, 32, 128, slots, FAKE, 8, None) == 2  # 4 blocks > 64 rows


def test_prefix_cache_create_validation(lib):
    h = ctypes.c_void_p()
    assert lib.mqa_prefix_cache_create(0, 10, ctypes.byref(h)) == 2
    assert lib.mqa_prefix_cache_create(16, 0, ctypes.byref(h)) == 2
    assert lib.mqa_prefix_cache_create(16, 10, None) == 1



def test_decode_plan_short_ranges(lib):
    """The decode planner (seen through the workspace it asks for): a
    1024-key window over 64 sequences of 32 heads runs as whole-window
    16-head work-groups with no partition states; the same sequences' global
    layer is split into partitions that need them; a window too wide for the
    short-range plan, or more 16-head groups than compute units, falls back
    to partitions. (Without a GPU the planner assumes 256 compute units.)"""
    import mqa_attention_int8_amd as m
    assert m.mqa_decode_workspace_bytes(64, 32, 128, 4096, 1024) == 0
    assert m.mqa_decode_workspace_bytes(64, 32, 128, 4096, 0) > 0
    assert m.mqa_decode_workspace_bytes(64, 32, 128, 4096, 2048) > 0      # 65 tiles: partitions
    assert m.mqa_decode_workspace_bytes(8, 32, 128, 1000, 0) == 0         # 32 tiles, 16 groups
    assert m.mqa_decode_workspace_bytes(200, 32, 128, 32768, 1024) > 0    # 400 groups > 256 units


def test_deterministic_switch_returns_previous_setting(lib):
    """mqa_set_deterministic is host-only: no device needed."""
    lib.mqa_set_deterministic.argtypes = [ctypes.c_int]
    lib.mqa_set_deterministic.restype = ctypes.c_int
    first = lib.mqa_set_deterministic(1)
    try:
        assert first in (0, 1)
        assert lib.mqa_set_deterministic(7) == 1      # any non-zero value turns it on
        assert lib.mqa_set_deterministic(0) == 1
        assert lib.mqa_set_deterministic(0) == 0
    finally:
        lib.mqa_set_deterministic(first)
