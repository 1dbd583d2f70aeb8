"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

Holds no attention or quantization arithmetic: it only draws numbers.
Streams are numpy ``default_rng(SeedSequence([workload_id, tensor_id, extra]))``
so every tensor of every workload is reproducible on its own.

Distributions follow the workloads this library is measured on: queries are
N(0, 1) rounded to bf16 (stored as uint16 bit patterns), keys and values are
N(0, 1) fp32 rows that are quantized to int8 by whoever consumes them, ragged
sequence lengths are uniform integers in a closed range.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# tensor ids within a workload
T_Q, T_K, T_V, T_LENS, T_KNEW, T_VNEW = 1, 2, 3, 4, 5, 6


def rng(workload_id: int, tensor_id: int, extra: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(workload_id), int(tensor_id), int(extra)]))


def normal_f32(g: np.random.Generator, shape) -> np.ndarray:
    return g.standard_normal(size=shape, dtype=np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to the nearest bf16 (ties to even); returns uint16 patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def q_bf16(g: np.random.Generator, shape) -> np.ndarray:
    return f32_to_bf16_bits(normal_f32(g, shape))


def ragged_lens(g: np.random.Generator, B: int, lo: int, hi: int) -> np.ndarray:
    """Integers uniform on [lo, hi] inclusive."""
    return g.integers(lo, hi, size=B, endpoint=True).astype(np.int32)


@dataclass(frozen=True)
class DecodeWorkload:
    """A decode step: B sequences, Hq query heads, one shared KV head of width D."""
    wid: int
    name: str
    B: int
    Hq: int
    D: int
    seq_lens: tuple | None = None      # fixed lengths (all equal) or None for ragged
    ragged: tuple | None = None        # (lo, hi) inclusive for ragged lengths
    layers: tuple = ((None, 0),)       # (buffer name, window) per layer
    L_cap: int | None = None

    def lens(self) -> np.ndarray:
        if self.ragged is not None:
            return ragged_lens(rng(self.wid, T_LENS), self.B, *self.ragged)
        return np.asarray(self.seq_lens, dtype=np.int32)

    def capacity(self) -> int:
        if self.L_cap is not None:
            return self.L_cap
        return int(self.lens().max())


@dataclass(frozen=True)
class PrefillWorkload:
    wid: int
    name: str
    B: int
    C: int
    prefix: int
    Hq: int
    D: int
    windows: tuple = (0, 1024)


TINY = DecodeWorkload(1, "tiny_decode_B1_Hq8_D64_L256", B=1, Hq=8, D=64,
                      seq_lens=(256,), layers=(("G", 0),))
DECODE = DecodeWorkload(2, "decode_B64_Hq32_D128_L4096_global+w1024", B=64, Hq=32, D=128,
                        seq_lens=tuple([4096] * 64), layers=(("G", 0), ("G", 1024)))
HYBRID = DecodeWorkload(3, "hybrid6_B128_Hq32_D128_L1024-32768", B=128, Hq=32, D=128,
                        ragged=(1024, 32768),
                        layers=(("G", 0), ("A", 1024), ("A", 1024), ("A", 1024),
                                ("Bf", 1024), ("Bf", 1024)))
PREFILL = PrefillWorkload(4, "prefill_B16_C512_P8192_Hq32_D128", B=16, C=512, prefix=8192,
                          Hq=32, D=128)
LONG = DecodeWorkload(5, "long_decode_B8_Hq32_D128_L131072", B=8, Hq=32, D=128,
                      seq_lens=tuple([131072] * 8), layers=(("G", 0),))

WORKLOADS = {w.wid: w for w in (TINY, DECODE, HYBRID, PREFILL, LONG)}


def kv_rows_f32(wid: int, which: int, buffer_id: int, B: int, L: int, D: int) -> np.ndarray:
    """fp32 N(0,1) K (which=T_K) or V (which=T_V) rows of one buffer, [B, L, D]."""
    g = rng(wid, which, buffer_id)
    return normal_f32(g, (B, L, D))


def block_table(g: np.random.Generator, B: int, table_len: int, num_blocks: int) -> np.ndarray:
    """int32 [B, table_len]: distinct pool blocks drawn at random (a shuffled
    allocation, as a block allocator under churn would leave it)."""
    if B * table_len > num_blocks:
        raise ValueError("pool too small for distinct blocks")
    return g.permutation(num_blocks)[: B * table_len].reshape(B, table_len).astype(np.int32)

