"""Shared helpers of the GPU parity tests: seeded inputs built on the CPU.

Inputs come from ``synth`` (random numbers only) and, where the method's int8
encoding is needed, from the oracle's quantizer; they are then uploaded. No
input or expected value is ever read back from the HIP path.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import synth


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev(x: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


TILE_ROWS = 32   # decode calls take caches whose capacity is a multiple of 32 rows


def pad_rows(a: np.ndarray, rows: int) -> np.ndarray:
    """`a` [B, L, ...] with zero rows appended up to `rows` rows."""
    if a.shape[1] >= rows:
        return a
    pad = np.zeros((a.shape[0], rows - a.shape[1]) + a.shape[2:], a.dtype)
    return np.concatenate([a, pad], axis=1)


class HostKV:
    """int8 KV buffer made on the host: codes and scales from the oracle
    quantizer. The capacity is padded with zero rows (codes and scales) to a
    multiple of 32; no length used with it reaches the padding."""

    def __init__(self, kq, ks, vq, vs):
        rows = -(-kq.shape[1] // TILE_ROWS) * TILE_ROWS
        self.kq, self.ks, self.vq, self.vs = (pad_rows(a, rows) for a in (kq, ks, vq, vs))

    @classmethod
    def seeded(cls, wid: int, buffer_id: int, B: int, L: int, D: int, rows=None):
        """K/V = N(0,1) fp32 rows quantized per row. ``rows`` (list of (b, lo, hi))
        restricts the filled rows; the rest stay zero codes with zero scale."""
        kq = np.zeros((B, L, D), np.int8)
        vq = np.zeros((B, L, D), np.int8)
        ks = np.zeros((B, L), np.float32)
        vs = np.zeros((B, L), np.float32)
        gk = synth.rng(wid, synth.T_K, buffer_id)
        gv = synth.rng(wid, synth.T_V, buffer_id)
        spans = rows if rows is not None else [(b, 0, L) for b in range(B)]
        for b, lo, hi in spans:
            if hi <= lo:
                continue
            kq[b, lo:hi], ks[b, lo:hi] = oracle.quantize_rows(synth.normal_f32(gk, (hi - lo, D)))
            vq[b, lo:hi], vs[b, lo:hi] = oracle.quantize_rows(synth.normal_f32(gv, (hi - lo, D)))
        return cls(kq, ks, vq, vs)

    def to_device(self):
        from mqa_attention_int8_amd import KVView
        return KVView(dev(self.kq), dev(self.vq), dev(self.ks), dev(self.vs))

    def arrays(self):
        return self.kq, self.ks, self.vq, self.vs


def q_bits(wid: int, shape, extra: int = 0) -> np.ndarray:
    return synth.q_bf16(synth.rng(wid, synth.T_Q, extra), shape)


def q_dev(bits: np.ndarray) -> torch.Tensor:
    return dev(bits.view(np.int16), torch.bfloat16)


def max_abs(gpu: torch.Tensor, ref: np.ndarray) -> float:
    g = gpu.detach().cpu().numpy().astype(np.float64)
    return float(np.max(np.abs(g - ref))) if ref.size else 0.0


def assert_decode_close(gpu: torch.Tensor, ref: np.ndarray, tol: float = 1e-4, what: str = ""):
    g = gpu.detach().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = float(np.max(np.abs(g - ref))) if ref.size else 0.0
    log(f"  {what}: max |gpu - oracle| = {err:.3e} (tol {tol:.0e})")
    assert err <= tol, f"{what}: max abs error {err} > {tol}"
    return err


def assert_prefill_close(gpu: torch.Tensor, ref: np.ndarray, atol=5e-3, rtol=1e-2, what=""):
    g = gpu.detach().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    excess = np.abs(g - ref) - (atol + rtol * np.abs(ref))
    err = float(np.max(np.abs(g - ref))) if ref.size else 0.0
    log(f"  {what}: max |gpu - oracle| = {err:.3e}, worst margin {float(excess.max()):.3e}")
    assert np.all(excess <= 0), f"{what}: {int((excess > 0).sum())} elements outside atol+rtol*|ref|"
    return err


def block_copy_pool(cont: np.ndarray, table: np.ndarray, bs: int, num_blocks: int, fill=0) -> np.ndarray:
    """Pool [num_blocks, bs, ...] built from a contiguous cache [B, L, ...] by
    whole-block copies: logical block j of sequence b -> pool block table[b, j]
    (blocks past L // bs are left at ``fill``)."""
    B, L = cont.shape[:2]
    pool = np.full((num_blocks, bs) + cont.shape[2:], fill, cont.dtype)
    for b in range(B):
        for j in range(min(L // bs, table.shape[1])):
            pool[table[b, j]] = cont[b, j * bs:(j + 1) * bs]
    return pool


def paged_from_host(hkv: "HostKV", table: np.ndarray, bs: int, num_blocks: int):
    """PagedKV on the device holding the same rows as a host cache."""
    from mqa_attention_int8_amd import PagedKV
    kq, ks, vq, vs = hkv.arrays()
    return PagedKV(dev(block_copy_pool(kq, table, bs, num_blocks)), dev(block_copy_pool(vq, table, bs, num_blocks)),
                   dev(block_copy_pool(ks, table, bs, num_blocks)), dev(block_copy_pool(vs, table, bs, num_blocks)),
                   dev(np.ascontiguousarray(table, dtype=np.int32)))

