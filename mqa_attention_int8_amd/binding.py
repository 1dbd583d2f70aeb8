"""Thin Python binding of libmqa_int8.so (argument marshalling only).

Every function here has the name of the C entry point it calls and does no
arithmetic of its own: shapes and dtypes are checked, raw device pointers and
torch's current HIP stream are handed to the library, and a non-zero status
raises ``MQAError``. PyTorch is used for device memory and streams only.

The library must be built (``python -m mqa_attention_int8_amd.build``); a
missing library raises at first use - there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmqa_int8.so")
_lock = threading.Lock()
_lib = None

MQA_OK = 0


class MQAError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = int(code)
        super().__init__(f"{where}: status {code}: {mqa_status_string(code)}")


class mqa_kv_view(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p), ("L_cap", ctypes.c_int32)]


class mqa_kv_cache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p), ("L_cap", ctypes.c_int32)]


class mqa_kv_paged(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p), ("block_table", ctypes.c_void_p), ("block_size", ctypes.c_int32),
                ("table_len", ctypes.c_int32), ("num_blocks", ctypes.c_int32)]


class mqa_prefix_cache_stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("capacity_blocks", "used_blocks", "lookups", "lookup_tokens",
                                              "matched_tokens", "inserted_blocks", "evicted_blocks")]


def library_path() -> str:
    return _LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load libmqa_int8.so once (after torch, so both share one HIP runtime)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is not built; run python -m mqa_attention_int8_amd.build")
        lib = ctypes.CDLL(_LIB_PATH)
        i32, vp, f32 = ctypes.c_int32, ctypes.c_void_p, ctypes.c_float
        lib.mqa_status_string.argtypes = [ctypes.c_int]
        lib.mqa_status_string.restype = ctypes.c_char_p
        lib.kv_quantize_int8.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, vp]
        lib.kv_quantize_int8.restype = ctypes.c_int
        lib.mqa_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
        lib.mqa_decode_workspace_bytes.restype = ctypes.c_size_t
        lib.mqa_decode.argtypes = [vp, ctypes.POINTER(mqa_kv_view), vp, i32, i32, i32, i32, i32, f32,
                                   vp, vp, ctypes.c_size_t, vp]
        lib.mqa_decode.restype = ctypes.c_int
        lib.mqa_decode_noalloc.argtypes = [vp, ctypes.POINTER(mqa_kv_view), vp, i32, i32, i32, i32, i32, f32,
                                           vp, vp]
        lib.mqa_decode_noalloc.restype = ctypes.c_int
        lib.mqa_decode_append.argtypes = [vp, ctypes.POINTER(mqa_kv_cache), vp, vp, vp, i32, i32, i32, i32, i32,
                                          f32, vp, vp, ctypes.c_size_t, vp]
        lib.mqa_decode_append.restype = ctypes.c_int
        lib.mqa_decode_ragged_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
        lib.mqa_decode_ragged_workspace_bytes.restype = ctypes.c_size_t
        lib.mqa_decode_ragged.argtypes = [vp, ctypes.POINTER(mqa_kv_view), vp, i32, i32, i32, i32, i32, f32,
                                          vp, vp, ctypes.c_size_t, vp]
        lib.mqa_decode_ragged.restype = ctypes.c_int
        lib.mqa_decode_append_ragged.argtypes = [vp, ctypes.POINTER(mqa_kv_cache), vp, vp, vp, i32, i32, i32, i32,
                                                 i32, f32, vp, vp, ctypes.c_size_t, vp]
        lib.mqa_decode_append_ragged.restype = ctypes.c_int
        lib.mqa_prefill_workspace_bytes.argtypes = [i32, i32, i32, i32]
        lib.mqa_prefill_workspace_bytes.restype = ctypes.c_size_t
        lib.mqa_prefill_chunk.argtypes = [vp, ctypes.POINTER(mqa_kv_view), vp, i32, i32, i32, i32, i32,
                                          i32, f32, vp, vp, ctypes.c_size_t, vp]
        lib.mqa_prefill_chunk.restype = ctypes.c_int
        pg = ctypes.POINTER(mqa_kv_paged)
        lib.kv_quantize_int8_paged.argtypes = [vp, vp, pg, vp, i32, i32, i32, vp]
        lib.kv_quantize_int8_paged.restype = ctypes.c_int
        lib.mqa_decode_paged_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
        lib.mqa_decode_paged_workspace_bytes.restype = ctypes.c_size_t
        lib.mqa_decode_paged.argtypes = [vp, pg, vp, i32, i32, i32, i32, i32, f32, vp, vp, ctypes.c_size_t, vp]
        lib.mqa_decode_paged.restype = ctypes.c_int
        lib.mqa_decode_append_paged.argtypes = [vp, pg, vp, vp, vp, i32, i32, i32, i32, i32, f32, vp, vp,
                                                ctypes.c_size_t, vp]
        lib.mqa_decode_append_paged.restype = ctypes.c_int
        lib.mqa_prefill_chunk_paged.argtypes = [vp, pg, vp, i32, i32, i32, i32, i32, i32, f32, vp, vp,
                                                ctypes.c_size_t, vp]
        lib.mqa_prefill_chunk_paged.restype = ctypes.c_int
        lib.mqa_decode_q8.argtypes = [vp, vp, ctypes.POINTER(mqa_kv_view), vp, i32, i32, i32, i32, i32, f32, vp,
                                      vp, ctypes.c_size_t, vp]
        lib.mqa_decode_q8.restype = ctypes.c_int
        lib.mqa_decode_append_q8.argtypes = [vp, vp, ctypes.POINTER(mqa_kv_cache), vp, vp, vp, i32, i32, i32, i32,
                                             i32, f32, vp, vp, ctypes.c_size_t, vp]
        lib.mqa_decode_append_q8.restype = ctypes.c_int
        i64, p64 = ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)
        lib.mqa_prefix_cache_create.argtypes = [i32, i64, ctypes.POINTER(vp)]
        lib.mqa_prefix_cache_create.restype = ctypes.c_int
        lib.mqa_prefix_cache_destroy.argtypes = [vp]
        lib.mqa_prefix_cache_destroy.restype = None
        lib.mqa_prefix_cache_match.argtypes = [vp, vp, i64, p64, vp]
        lib.mqa_prefix_cache_match.restype = ctypes.c_int
        lib.mqa_prefix_cache_insert.argtypes = [vp, vp, i64, vp, p64, p64]
        lib.mqa_prefix_cache_insert.restype = ctypes.c_int
        lib.mqa_prefix_cache_get_stats.argtypes = [vp, ctypes.POINTER(mqa_prefix_cache_stats)]
        lib.mqa_prefix_cache_get_stats.restype = ctypes.c_int
        lib.mqa_kv_blocks_to_host.argtypes = [ctypes.POINTER(mqa_kv_view), i32, i32, i32, i64, i64, i32, i32, vp,
                                              vp, i64, vp]
        lib.mqa_kv_blocks_to_host.restype = ctypes.c_int
        lib.mqa_kv_blocks_to_device.argtypes = [ctypes.POINTER(mqa_kv_cache), i32, i32, i32, i64, i64, i32, i32, vp,
                                                vp, i64, vp]
        lib.mqa_kv_blocks_to_device.restype = ctypes.c_int
        lib.mqa_set_deterministic.argtypes = [ctypes.c_int]
        lib.mqa_set_deterministic.restype = ctypes.c_int
        _lib = lib
        return lib


def mqa_status_string(code: int) -> str:
    return load_library().mqa_status_string(int(code)).decode()


def mqa_set_deterministic(enable: bool) -> bool:
    """Fixed tile-to-wave assignment in decode calls launched from now on
    (bitwise repeatable results); returns the previous setting."""
    return bool(load_library().mqa_set_deterministic(1 if enable else 0))


def _check(code: int, where: str):
    if code != MQA_OK:
        raise MQAError(code, where)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t: torch.Tensor, dtype, name: str, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class KVView:
    """One KV buffer: int8 K/V [B, L_cap, D] and fp32 scales [B, L_cap].

    Several layers may hold the same KVView (cross-layer KV sharing)."""

    def __init__(self, k: torch.Tensor, v: torch.Tensor, k_scale: torch.Tensor, v_scale: torch.Tensor):
        for t, n in ((k, "k"), (v, "v")):
            _need(t, torch.int8, n, 3)
        for t, n in ((k_scale, "k_scale"), (v_scale, "v_scale")):
            _need(t, torch.float32, n, 2)
        if k.shape != v.shape or k_scale.shape != v_scale.shape or tuple(k.shape[:2]) != tuple(k_scale.shape):
            raise ValueError("inconsistent KV buffer shapes")
        self.k, self.v, self.k_scale, self.v_scale = k, v, k_scale, v_scale
        self.B, self.L_cap, self.D = (int(x) for x in k.shape)

    @classmethod
    def empty(cls, B: int, L_cap: int, D: int, device="cuda"):
        return cls(torch.empty((B, L_cap, D), dtype=torch.int8, device=device),
                   torch.empty((B, L_cap, D), dtype=torch.int8, device=device),
                   torch.zeros((B, L_cap), dtype=torch.float32, device=device),
                   torch.zeros((B, L_cap), dtype=torch.float32, device=device))

    def c_view(self) -> mqa_kv_view:
        return mqa_kv_view(self.k.data_ptr(), self.v.data_ptr(), self.k_scale.data_ptr(),
                           self.v_scale.data_ptr(), self.L_cap)

    def c_cache(self) -> mqa_kv_cache:
        return mqa_kv_cache(self.k.data_ptr(), self.v.data_ptr(), self.k_scale.data_ptr(),
                            self.v_scale.data_ptr(), self.L_cap)


def kv_quantize_int8(src: torch.Tensor, dst: torch.Tensor, dst_scale: torch.Tensor,
                     start_pos: torch.Tensor, stream=None) -> None:
    """Quantize src fp32 [B, T, D] into rows start_pos[b].. of dst / dst_scale."""
    lib = load_library()
    _need(src, torch.float32, "src", 3)
    _need(dst, torch.int8, "dst", 3)
    _need(dst_scale, torch.float32, "dst_scale", 2)
    _need(start_pos, torch.int32, "start_pos", 1)
    B, T, D = (int(x) for x in src.shape)
    if dst.shape[0] != B or dst.shape[2] != D or tuple(dst_scale.shape) != tuple(dst.shape[:2]) \
            or start_pos.shape[0] != B:
        raise ValueError("kv_quantize_int8: shape mismatch")
    _check(lib.kv_quantize_int8(_ptr(src), _ptr(dst), _ptr(dst_scale), _ptr(start_pos), B, T, D,
                                int(dst.shape[1]), _stream(stream)), "kv_quantize_int8")


def append_kv(kv: KVView, k_new: torch.Tensor, v_new: torch.Tensor, start_pos: torch.Tensor,
              stream=None) -> None:
    """Write new K and V rows (fp32 [B, T, D]) into a KV buffer: two kv_quantize_int8 calls."""
    kv_quantize_int8(k_new, kv.k, kv.k_scale, start_pos, stream)
    kv_quantize_int8(v_new, kv.v, kv.v_scale, start_pos, stream)


def mqa_decode_workspace_bytes(B: int, Hq: int, D: int, max_seq_len: int, window: int) -> int:
    return int(load_library().mqa_decode_workspace_bytes(B, Hq, D, max_seq_len, window))


def decode_workspace(B: int, Hq: int, D: int, max_seq_len: int, window: int, device="cuda"):
    """A workspace for mqa_decode (None when none is needed); reusable by any
    later call on the same stream that it is large enough for."""
    need = mqa_decode_workspace_bytes(B, Hq, D, max_seq_len, window)
    if need == 0:
        return None
    return torch.empty(need, dtype=torch.uint8, device=device)


def default_softmax_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)


def mqa_decode(q: torch.Tensor, kv: KVView, seq_lens: torch.Tensor, max_seq_len: int, window: int,
               softmax_scale: float | None = None, out: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """One decode step: q bf16 [B, Hq, D] -> out fp32 [B, Hq, D]."""
    lib = load_library()
    _need(q, torch.bfloat16, "q", 3)
    _need(seq_lens, torch.int32, "seq_lens", 1)
    B, Hq, D = (int(x) for x in q.shape)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    _need(out, torch.float32, "out", 3)
    need = mqa_decode_workspace_bytes(B, Hq, D, max_seq_len, window)
    if workspace is None and need > 0:
        workspace = decode_workspace(B, Hq, D, max_seq_len, window, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    scale = default_softmax_scale(D) if softmax_scale is None else float(softmax_scale)
    view = kv.c_view()
    _check(lib.mqa_decode(_ptr(q), ctypes.byref(view), _ptr(seq_lens), int(max_seq_len), B, Hq, D,
                          int(window), scale, _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)),
           "mqa_decode")
    return out


def mqa_decode_noalloc(q: torch.Tensor, kv: KVView, seq_lens: torch.Tensor, max_seq_len: int, window: int,
                       softmax_scale: float | None = None, out: torch.Tensor | None = None,
                       stream=None) -> torch.Tensor:
    """mqa_decode with the partition states in the library's static device
    array (no workspace; the C call allocates nothing). Pass `out` to keep
    the binding itself from allocating the output."""
    lib = load_library()
    _need(q, torch.bfloat16, "q", 3)
    _need(seq_lens, torch.int32, "seq_lens", 1)
    B, Hq, D = (int(x) for x in q.shape)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    _need(out, torch.float32, "out", 3)
    scale = default_softmax_scale(D) if softmax_scale is None else float(softmax_scale)
    view = kv.c_view()
    _check(lib.mqa_decode_noalloc(_ptr(q), ctypes.byref(view), _ptr(seq_lens), int(max_seq_len), B, Hq, D,
                                  int(window), scale, _ptr(out), _stream(stream)),
           "mqa_decode_noalloc")
    return out


def mqa_decode_append(q: torch.Tensor, kv: KVView, k_new: torch.Tensor, v_new: torch.Tensor,
                      seq_lens: torch.Tensor, max_seq_len: int, window: int,
                      softmax_scale: float | None = None, out: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Append the new token's K/V rows (fp32 [B, D]) at row seq_lens[b] - 1 of
    ``kv`` and run one decode step on it, in one launch."""
    lib = load_library()
    _need(q, torch.bfloat16, "q", 3)
    _need(seq_lens, torch.int32, "seq_lens", 1)
    B, Hq, D = (int(x) for x in q.shape)
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, torch.float32, n, 2)
        if tuple(t.shape) != (B, D):
            raise ValueError(f"{n} must have shape {(B, D)}")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    _need(out, torch.float32, "out", 3)
    need = mqa_decode_workspace_bytes(B, Hq, D, max_seq_len, window)
    if workspace is None and need > 0:
        workspace = decode_workspace(B, Hq, D, max_seq_len, window, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    scale = default_softmax_scale(D) if softmax_scale is None else float(softmax_scale)
    cache = kv.c_cache()
    _check(lib.mqa_decode_append(_ptr(q), ctypes.byref(cache), _ptr(k_new), _ptr(v_new), _ptr(seq_lens),
                                 int(max_seq_len), B, Hq, D, int(window), scale, _ptr(out), _ptr(workspace),
                                 ws_bytes, _stream(stream)),
           "mqa_decode_append")
    return out


def mqa_decode_ragged_workspace_bytes(B: int, Hq: int, D: int, max_seq_len: int, window: int) -> int:
    return int(load_library().mqa_decode_ragged_workspace_bytes(B, Hq, D, max_seq_len, window))


def ragged_workspace(B: int, Hq: int, D: int, max_seq_len: int, window: int, device="cuda"):
    """A workspace for mqa_decode_ragged / mqa_decode_append_ragged (None when none is needed)."""
    need = mqa_decode_ragged_workspace_bytes(B, Hq, D, max_seq_len, window)
    if need == 0:
        return None
    return torch.empty(need, dtype=torch.uint8, device=device)


def _ragged_ws(B, Hq, D, max_seq_len, window, workspace, device):
    need = mqa_decode_ragged_workspace_bytes(B, Hq, D, max_seq_len, window)
    if workspace is None and need > 0:
        workspace = ragged_workspace(B, Hq, D, max_seq_len, window, device)
    return workspace, (0 if workspace is None else workspace.numel() * workspace.element_size())


def mqa_decode_ragged(q: torch.Tensor, kv: KVView, seq_lens: torch.Tensor, max_seq_len: int, window: int,
                      softmax_scale: float | None = None, out: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """mqa_decode with work balanced over the compute units from the actual lengths."""
    lib = load_library()
    _need(q, torch.bfloat16, "q", 3)
    _need(seq_lens, torch.int32, "seq_lens", 1)
    B, Hq, D = (int(x) for x in q.shape)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    _need(out, torch.float32, "out", 3)
    workspace, ws_bytes = _ragged_ws(B, Hq, D, max_seq_len, window, workspace, q.device)
    scale = default_softmax_scale(D) if softmax_scale is None else float(softmax_scale)
    view = kv.c_view()
    _check(lib.mqa_decode_ragged(_ptr(q), ctypes.byref(view), _ptr(seq_lens), int(max_seq_len), B, Hq, D,
                                 int(window), scale, _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)),
           "mqa_decode_ragged")
    return out


def mqa_decode_append_ragged(q: torch.Tensor, kv: KVView, k_new: torch.Tensor, v_new: torch.Tensor,
                             seq_lens: torch.Tensor, max_seq_len: int, window: int,
                             softmax_scale: float | None = None, out: torch.Tensor | None = None,
                             workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """mqa_decode_append with work balanced over the compute units from the actual lengths."""
    lib = load_library()
    _need(q, torch.bfloat16, "q", 3)
    _need(seq_lens, torch.int32, "seq_lens", 1)
    B, Hq, D = (int(x) for x in q.shape)
    _need(k_new, torch.float32, "k_new", 2)
    _need(v_new, torch.float32, "v_new", 2)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    _need(out, torch.float32, "out", 3)
    workspace, ws_bytes = _ragged_ws(B, Hq, D, max_seq_len, window, workspace, q.device)
    scale = default_softmax_scale(D) if softmax_scale is None else float(softmax_scale)
    cache = kv.c_cache()
    _check(lib.mqa_decode_append_ragged(_ptr(q), ctypes.byref(cache), _ptr(k_new), _ptr(v_new), _ptr(seq_lens),
                                        int(max_seq_len), B, Hq, D, int(window), scale, _ptr(out),
                                        _ptr(workspace), ws_bytes, _stream(stream)),
           "mqa_decode_append_ragged")
    return out


def mqa_prefill_workspace_bytes(B: int, C: int, D: int, max_prefix_len: int) -> int:
    return int(load_library().mqa_prefill_workspace_bytes(B, C, D, max_prefix_len))


def prefill_workspace(B: int, C: int, D: int, max_prefix_len: int, device="cuda"):
    """A workspace for mqa_prefill_chunk, reusable by any later call it fits."""
    return torch.empty(mqa_prefill_workspace_bytes(B, C, D, max_prefix_len), dtype=torch.uint8,
                       device=device)


def mqa_prefill_chunk(q: torch.Tensor, kv: KVView, prefix_lens: torch.Tensor, max_prefix_len: int,
                      window: int, softmax_scale: float | None = None,
                      out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                      stream=None) -> torch.Tensor:
    """Causal chunk attention: q bf16 [B, C, Hq, D] -> out fp32 [B, C, Hq, D]."""
    lib = load_library()
    _need(q, torch.bfloat16, "q", 4)
    _need(prefix_lens, torch.int32, "prefix_lens", 1)
    B, C, Hq, D = (int(x) for x in q.shape)
    if out is None:
        out = torch.empty((B, C, Hq, D), dtype=torch.float32, device=q.device)
    _need(out, torch.float32, "out", 4)
    if workspace is None:
        workspace = prefill_workspace(B, C, D, max_prefix_len, q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    scale = default_softmax_scale(D) if softmax_scale is None else float(softmax_scale)
    view = kv.c_view()
    _check(lib.mqa_prefill_chunk(_ptr(q), ctypes.byref(view), _ptr(prefix_lens), int(max_prefix_len), B,
                                 C, Hq, D, int(window), scale, _ptr(out), _ptr(workspace), ws_bytes,
                                 _stream(stream)),
           "mqa_prefill_chunk")
    return out


class PagedKV:
    """One paged KV buffer: int8 pools K/V [num_blocks, block_size, D], fp32
    scale pools [num_blocks, block_size] and an int32 block table
    [B, table_len] mapping logical block j of sequence b to pool block
    table[b, j % table_len] (a short table makes a ring)."""

    def __init__(self, k: torch.Tensor, v: torch.Tensor, k_scale: torch.Tensor, v_scale: torch.Tensor,
                 block_table: torch.Tensor):
        for t, n in ((k, "k"), (v, "v")):
            _need(t, torch.int8, n, 3)
        for t, n in ((k_scale, "k_scale"), (v_scale, "v_scale")):
            _need(t, torch.float32, n, 2)
        _need(block_table, torch.int32, "block_table", 2)
        if k.shape != v.shape or k_scale.shape != v_scale.shape or tuple(k.shape[:2]) != tuple(k_scale.shape):
            raise ValueError("inconsistent paged pool shapes")
        self.k, self.v, self.k_scale, self.v_scale, self.block_table = k, v, k_scale, v_scale, block_table
        self.num_blocks, self.block_size, self.D = (int(x) for x in k.shape)
        self.B, self.table_len = (int(x) for x in block_table.shape)

    @classmethod
    def empty(cls, num_blocks: int, block_size: int, D: int, block_table: torch.Tensor, device="cuda"):
        return cls(torch.zeros((num_blocks, block_size, D), dtype=torch.int8, device=device),
                   torch.zeros((num_blocks, block_size, D), dtype=torch.int8, device=device),
                   torch.zeros((num_blocks, block_size), dtype=torch.float32, device=device),
                   torch.zeros((num_blocks, block_size), dtype=torch.float32, device=device),
                   block_table)

    def c_paged(self) -> mqa_kv_paged:
        return mqa_kv_paged(self.k.data_ptr(), self.v.data_ptr(), self.k_scale.data_ptr(), self.v_scale.data_ptr(),
                            self.block_table.data_ptr(), self.block_size, self.table_len, self.num_blocks)


def kv_quantize_int8_paged(k_src: torch.Tensor, v_src: torch.Tensor, kv: PagedKV, start_pos: torch.Tensor,
                           stream=None) -> None:
    """Quantize new K and V rows (fp32 [B, T, D]) into their pool rows."""
    lib = load_library()
    _need(k_src, torch.float32, "k_src", 3)
    _need(v_src, torch.float32, "v_src", 3)
    _need(start_pos, torch.int32, "start_pos", 1)
    B, T, D = (int(x) for x in k_src.shape)
    if tuple(v_src.shape) != (B, T, D) or D != kv.D or start_pos.shape[0] != B or B > kv.B:
        raise ValueError("kv_quantize_int8_paged: shape mismatch")
    c = kv.c_paged()
    _check(lib.kv_quantize_int8_paged(_ptr(k_src), _ptr(v_src), ctypes.byref(c), _ptr(start_pos), B, T, D,
                                      _stream(stream)), "kv_quantize_int8_paged")


def mqa_decode_paged_workspace_bytes(B: int, Hq: int, D: int, max_seq_len: int, window: int,
                                     block_size: int) -> int:
    return int(load_library().mqa_decode_paged_workspace_bytes(B, Hq, D, max_seq_len, window, block_size))


def _paged_decode_args(q, kv, seq_lens, max_seq_len, window, softmax_scale, out, workspace):
    _need(q, torch.bfloat16, "q", 3)
    _need(seq_lens, torch.int32, "seq_lens", 1)
    B, Hq, D = (int(x) for x in q.shape)
    if B > kv.B or D != kv.D:
        raise ValueError("paged decode: q does not match the buffer")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    _need(out, torch.float32, "out", 3)
    need = mqa_decode_paged_workspace_bytes(B, Hq, D, max_seq_len, window, kv.block_size)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    scale = default_softmax_scale(D) if softmax_scale is None else float(softmax_scale)
    return B, Hq, D, out, workspace, ws_bytes, scale


def mqa_decode_paged(q: torch.Tensor, kv: PagedKV, seq_lens: torch.Tensor, max_seq_len: int, window: int,
                     softmax_scale: float | None = None, out: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """mqa_decode over a paged buffer."""
    lib = load_library()
    B, Hq, D, out, workspace, ws_bytes, scale = _paged_decode_args(q, kv, seq_lens, max_seq_len, window,
                                                                   softmax_scale, out, workspace)
    c = kv.c_paged()
    _check(lib.mqa_decode_paged(_ptr(q), ctypes.byref(c), _ptr(seq_lens), int(max_seq_len), B, Hq, D,
                                int(window), scale, _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)),
           "mqa_decode_paged")
    return out


def mqa_decode_append_paged(q: torch.Tensor, kv: PagedKV, k_new: torch.Tensor, v_new: torch.Tensor,
                            seq_lens: torch.Tensor, max_seq_len: int, window: int,
                            softmax_scale: float | None = None, out: torch.Tensor | None = None,
                            workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """mqa_decode_append over a paged buffer."""
    lib = load_library()
    B, Hq, D, out, workspace, ws_bytes, scale = _paged_decode_args(q, kv, seq_lens, max_seq_len, window,
                                                                   softmax_scale, out, workspace)
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, torch.float32, n, 2)
        if tuple(t.shape) != (B, D):
            raise ValueError(f"{n} must have shape {(B, D)}")
    c = kv.c_paged()
    _check(lib.mqa_decode_append_paged(_ptr(q), ctypes.byref(c), _ptr(k_new), _ptr(v_new), _ptr(seq_lens),
                                       int(max_seq_len), B, Hq, D, int(window), scale, _ptr(out),
                                       _ptr(workspace), ws_bytes, _stream(stream)),
           "mqa_decode_append_paged")
    return out


def mqa_prefill_chunk_paged(q: torch.Tensor, kv: PagedKV, prefix_lens: torch.Tensor, max_prefix_len: int,
                            window: int, softmax_scale: float | None = None,
                            out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                            stream=None) -> torch.Tensor:
    """mqa_prefill_chunk over a paged buffer."""
    lib = load_library()
    _need(q, torch.bfloat16, "q", 4)
    _need(prefix_lens, torch.int32, "prefix_lens", 1)
    B, C, Hq, D = (int(x) for x in q.shape)
    if B > kv.B or D != kv.D:
        raise ValueError("mqa_prefill_chunk_paged: q does not match the buffer")
    if out is None:
        out = torch.empty((B, C, Hq, D), dtype=torch.float32, device=q.device)
    _need(out, torch.float32, "out", 4)
    if workspace is None:
        workspace = prefill_workspace(B, C, D, max_prefix_len, q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    scale = default_softmax_scale(D) if softmax_scale is None else float(softmax_scale)
    c = kv.c_paged()
    _check(lib.mqa_prefill_chunk_paged(_ptr(q), ctypes.byref(c), _ptr(prefix_lens), int(max_prefix_len), B, C,
                                       Hq, D, int(window), scale, _ptr(out), _ptr(workspace), ws_bytes,
                                       _stream(stream)),
           "mqa_prefill_chunk_paged")
    return out


def _q8_args(q8, q_scale, seq_lens, max_seq_len, window, softmax_scale, out, workspace):
    _need(q8, torch.int8, "q8", 3)
    _need(q_scale, torch.float32, "q_scale", 2)
    _need(seq_lens, torch.int32, "seq_lens", 1)
    B, Hq, D = (int(x) for x in q8.shape)
    if tuple(q_scale.shape) != (B, Hq):
        raise ValueError(f"q_scale must have shape {(B, Hq)}")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q8.device)
    _need(out, torch.float32, "out", 3)
    if workspace is None and mqa_decode_workspace_bytes(B, Hq, D, max_seq_len, window) > 0:
        workspace = decode_workspace(B, Hq, D, max_seq_len, window, q8.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    scale = default_softmax_scale(D) if softmax_scale is None else float(softmax_scale)
    return B, Hq, D, out, workspace, ws_bytes, scale


def mqa_decode_q8(q8: torch.Tensor, q_scale: torch.Tensor, kv: KVView, seq_lens: torch.Tensor, max_seq_len: int,
                  window: int, softmax_scale: float | None = None, out: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Decode step with int8 queries: q8 int8 [B, Hq, D], q_scale fp32 [B, Hq]."""
    lib = load_library()
    B, Hq, D, out, workspace, ws_bytes, scale = _q8_args(q8, q_scale, seq_lens, max_seq_len, window,
                                                         softmax_scale, out, workspace)
    view = kv.c_view()
    _check(lib.mqa_decode_q8(_ptr(q8), _ptr(q_scale), ctypes.byref(view), _ptr(seq_lens), int(max_seq_len), B, Hq,
                             D, int(window), scale, _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)),
           "mqa_decode_q8")
    return out


def mqa_decode_append_q8(q8: torch.Tensor, q_scale: torch.Tensor, kv: KVView, k_new: torch.Tensor,
                         v_new: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, window: int,
                         softmax_scale: float | None = None, out: torch.Tensor | None = None,
                         workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """mqa_decode_append with int8 queries."""
    lib = load_library()
    B, Hq, D, out, workspace, ws_bytes, scale = _q8_args(q8, q_scale, seq_lens, max_seq_len, window,
                                                         softmax_scale, out, workspace)
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, torch.float32, n, 2)
        if tuple(t.shape) != (B, D):
            raise ValueError(f"{n} must have shape {(B, D)}")
    cache = kv.c_cache()
    _check(lib.mqa_decode_append_q8(_ptr(q8), _ptr(q_scale), ctypes.byref(cache), _ptr(k_new), _ptr(v_new),
                                    _ptr(seq_lens), int(max_seq_len), B, Hq, D, int(window), scale, _ptr(out),
                                    _ptr(workspace), ws_bytes, _stream(stream)),
           "mqa_decode_append_q8")
    return out


class PrefixCache:
    """Host-memory prefix cache (control plane in libmqa_int8): which token
    prefixes are cached, block by block, in which slots of a host pool."""

    def __init__(self, block_size: int, capacity_blocks: int):
        self._lib = load_library()
        h = ctypes.c_void_p()
        _check(self._lib.mqa_prefix_cache_create(int(block_size), int(capacity_blocks), ctypes.byref(h)),
               "mqa_prefix_cache_create")
        self._h = h
        self.block_size = int(block_size)
        self.capacity_blocks = int(capacity_blocks)

    @staticmethod
    def _tokens(tokens):
        import numpy as np
        return np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))

    def match(self, tokens):
        """(matched_tokens, slots of the matched blocks)."""
        import numpy as np
        t = self._tokens(tokens)
        slots = np.zeros(max(1, len(t) // self.block_size), np.int64)
        m = ctypes.c_int64()
        _check(self._lib.mqa_prefix_cache_match(self._h, t.ctypes.data, len(t), ctypes.byref(m), slots.ctypes.data),
               "mqa_prefix_cache_match")
        return int(m.value), slots[: int(m.value) // self.block_size].copy()

    def insert(self, tokens):
        """(slots of the blocks, first new block, number of blocks cached)."""
        import numpy as np
        t = self._tokens(tokens)
        slots = np.zeros(max(1, len(t) // self.block_size), np.int64)
        first, n = ctypes.c_int64(), ctypes.c_int64()
        _check(self._lib.mqa_prefix_cache_insert(self._h, t.ctypes.data, len(t), slots.ctypes.data,
                                                 ctypes.byref(first), ctypes.byref(n)), "mqa_prefix_cache_insert")
        return slots[: n.value].copy(), int(first.value), int(n.value)

    def stats(self) -> dict:
        st = mqa_prefix_cache_stats()
        _check(self._lib.mqa_prefix_cache_get_stats(self._h, ctypes.byref(st)), "mqa_prefix_cache_get_stats")
        return {n: int(getattr(st, n)) for n, _ in mqa_prefix_cache_stats._fields_}

    def close(self):
        if getattr(self, "_h", None):
            self._lib.mqa_prefix_cache_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()


def kv_block_bytes(n_bufs: int, block_size: int, D: int) -> int:
    return n_bufs * block_size * (2 * D + 8)


def host_pool(n_slots: int, n_bufs: int, block_size: int, D: int) -> torch.Tensor:
    """Pinned host memory for n_slots cached blocks (allocated pinned)."""
    return torch.empty(n_slots * kv_block_bytes(n_bufs, block_size, D), dtype=torch.uint8, pin_memory=True)


def _pool_slots(pool: torch.Tensor, n_bufs: int, block_size: int, D: int) -> int:
    if pool.dtype != torch.uint8 or pool.is_cuda or not pool.is_pinned() or not pool.is_contiguous():
        raise ValueError("host_pool must be a contiguous pinned uint8 host tensor")
    return pool.numel() // kv_block_bytes(n_bufs, block_size, D)


def mqa_kv_blocks_to_host(bufs, b: int, first_block: int, slots, block_size: int, pool: torch.Tensor,
                          stream=None) -> None:
    """Copy blocks first_block.. of sequence b of every buffer into pool slots."""
    import numpy as np
    lib = load_library()
    views = (mqa_kv_view * len(bufs))(*[kv.c_view() for kv in bufs])
    s = np.ascontiguousarray(np.asarray(slots, np.int64))
    D = bufs[0].D
    if not 0 <= int(b) < bufs[0].B or any(kv.B != bufs[0].B or kv.D != D for kv in bufs):
        raise ValueError("mqa_kv_blocks_to_host: sequence index or buffer shapes")
    _check(lib.mqa_kv_blocks_to_host(views, len(bufs), bufs[0].B, int(b), int(first_block), len(s), int(block_size), D,
                                     s.ctypes.data, pool.data_ptr(), _pool_slots(pool, len(bufs), block_size, D),
                                     _stream(stream)), "mqa_kv_blocks_to_host")


def mqa_kv_blocks_to_device(bufs, b: int, first_block: int, slots, block_size: int, pool: torch.Tensor,
                            stream=None) -> None:
    """Copy pool slots back into blocks first_block.. of sequence b of every buffer."""
    import numpy as np
    lib = load_library()
    caches = (mqa_kv_cache * len(bufs))(*[kv.c_cache() for kv in bufs])
    s = np.ascontiguousarray(np.asarray(slots, np.int64))
    D = bufs[0].D
    if not 0 <= int(b) < bufs[0].B or any(kv.B != bufs[0].B or kv.D != D for kv in bufs):
        raise ValueError("mqa_kv_blocks_to_device: sequence index or buffer shapes")
    _check(lib.mqa_kv_blocks_to_device(caches, len(bufs), bufs[0].B, int(b), int(first_block), len(s), int(block_size), D,
                                       s.ctypes.data, pool.data_ptr(), _pool_slots(pool, len(bufs), block_size, D),
                                       _stream(stream)), "mqa_kv_blocks_to_device")


def hip_runtimes_mapped() -> list[str]:
    """Paths of the HIP runtime libraries mapped into this process (diagnostic)."""
    paths = set()
    with open("/proc/self/maps") as f:
        for ln in f:
            if "libamdhip64" in ln:
                paths.add(ln.split()[-1])
    return sorted(paths)
