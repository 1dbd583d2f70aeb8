"""Plain CPU oracle for multi-query attention read from an int8 KV cache.

TEST INFRASTRUCTURE. This module is the checker, not the product: only the
test suite, the smoke check and the CPU-baseline leg of the benchmark may
import it. It shares no code, constants or helpers with the HIP path.

What it computes, and where that comes from:

* Multi-query attention: every query head of a layer attends to ONE shared
  K/V head.  [9c1h.cn news page on Character.AI's inference tricks
  (headline: which AI app handles 20,000 inference requests/s), section
  "秘訣1", item "全面采用MQA"; explinks.com page "Character.AI 的最佳实践",
  section "多查询注意力"; tubrief.io LLM-inference workshop transcript,
  00:44:29-00:45:08, where one 128-column block of the 4096-wide K/V
  projection serves all 32 query heads.]
* Hybrid attention horizons: local layers see a sliding window of 1024
  keys, one layer in six is global.  [9c1h.cn page, section "秘訣1", item
  "混合注意力視野"; explinks.com page, section "混合注意力范围".]
* Cross-layer KV sharing: several layers read one KV buffer.  [9c1h.cn
  page, section "秘訣1", item "跨層KV共享"; explinks.com page, section
  "跨层 KV 共享".]  In this oracle a shared buffer is literally the same
  array passed to several layers.
* int8 KV cache.  [explinks.com page, section "训练和服务的量化".]  The pages
  fix int8 but not the scheme; the reading used here is symmetric,
  per-token-row, absmax/127 scale in fp32, round half to even.
* Attention itself is the plain definition: scaled dot products, masked
  softmax, weighted sum of values.  [explinks.com page, section "代码块描述":
  energy = q.k, softmax of the scaled energy over keys, weighted sum of
  values; the scale there divides by the square root of the model width,
  here it is an explicit argument defaulting to 1/sqrt(head_dim).]
* Paged KV buffers: a sequence's KV is logically contiguous but stored in
  fixed-size blocks of a shared pool, mapped through a per-sequence table
  and allocated as tokens arrive.  [workshop transcript, 01:01:35-01:03:22
  (PagedAttention).]  A table shorter than the sequence wraps around, so a
  window-only buffer keeps just the recent blocks [9c1h.cn page, "秘訣1",
  item "混合注意力視野": local layers need only the last 1024 tokens];
  ``paged_rows`` / ``paged_gather`` / ``paged_scatter`` write the mapping out.
* The online-softmax / partition merge is an exact rewrite of softmax
  [workshop transcript, 00:48:02-00:49:13: tiles kept in fast memory with
  three running quantities for an online softmax]; ``lse_merge`` writes the
  combine rule out so the invariant can be tested.

Precision: attention in float64. The quantizer is an encoding, so it is
emulated bit-exactly in IEEE fp32 (each fp32 operation is done in float64
and rounded once to fp32; for division this double rounding is harmless
because 53 >= 2*24 + 2).
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# int8 KV encoding  [explinks.com "Character.AI 的最佳实践", 训练和服务的量化]
# ---------------------------------------------------------------------------

INT8_QMAX = 127


def _fl32(x64: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest fp32 (ties to even)."""
    return np.asarray(x64, dtype=np.float64).astype(np.float32)


def quantize_rows(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Quantize each row (last axis) of fp32 ``x`` to int8 with one fp32 scale.

    Steps, in fp32 as the encoding is defined:
      1. a = max_d |x_d|                      (exact)
      2. s = fl32(a / 127)                     (correctly rounded division)
      3. if s == 0: the row encodes as all zeros with scale 0
         (an all-zero row, or one so small that a/127 underflows)
      4. r_d = fl32(x_d / s)                   (correctly rounded division)
      5. q_d = clamp(round_half_even(r_d), -127, 127)

    Returns (q int8 [..., D], s float32 [...]).
    """
    x = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("quantize_rows: non-finite input")
    a = np.max(np.abs(x), axis=-1)
    s = _fl32(a.astype(np.float64) / float(INT8_QMAX))
    safe = np.where(s > 0, s, np.float32(1.0))
    r = _fl32(x.astype(np.float64) / safe.astype(np.float64)[..., None])
    q = np.clip(np.rint(r), -INT8_QMAX, INT8_QMAX)
    q = np.where((s > 0)[..., None], q, 0.0).astype(np.int8)
    return q, s.astype(np.float32)


def dequantize_rows(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """x_hat = q * s, exact in float64 (int8 times an fp32 fits 53 bits)."""
    return np.asarray(q, dtype=np.float64) * np.asarray(s, dtype=np.float64)[..., None]


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 numbers stored as their 16-bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def default_softmax_scale(head_dim: int) -> np.float32:
    """fl32(1/sqrt(D)): the head-dimension scale (see ``attend``)."""
    return np.float32(1.0 / np.sqrt(float(head_dim)))


# ---------------------------------------------------------------------------
# Visible keys  [9c1h.cn page 秘訣1 混合注意力視野: window of 1024 keys]
# ---------------------------------------------------------------------------

def decode_visible(n: int, window: int) -> tuple[int, int]:
    """Keys [lo, hi) seen by the newest token of a sequence holding n keys.

    ``n`` counts the current token (already written to the cache). A window
    W > 0 keeps the last W keys including the current one; W <= 0 is global.
    """
    n = int(n)
    if window > 0:
        return max(0, n - int(window)), n
    return 0, n


def prefill_visible(pos: int, window: int) -> tuple[int, int]:
    """Keys [lo, hi) seen by a query at absolute position ``pos`` (causal)."""
    pos = int(pos)
    if window > 0:
        return max(0, pos - int(window) + 1), pos + 1
    return 0, pos + 1


# ---------------------------------------------------------------------------
# Attention  [explinks.com page, 代码块描述; 9c1h.cn page 秘訣1 MQA]
# ---------------------------------------------------------------------------

def attend(qrows: np.ndarray, khat: np.ndarray, vhat: np.ndarray,
           allowed: np.ndarray, sigma: float) -> np.ndarray:
    """softmax over allowed keys of sigma * q.k, applied to the values.

    qrows [R, D], khat/vhat [n, D] (one shared K/V head), allowed [R, n] bool.
    A row with no allowed key outputs zeros. float64 throughout.
    """
    qrows = np.asarray(qrows, dtype=np.float64)
    R = qrows.shape[0]
    D = vhat.shape[1] if vhat.ndim == 2 else qrows.shape[1]
    if khat.shape[0] == 0:
        return np.zeros((R, D))
    z = float(sigma) * (qrows @ khat.T)
    z = np.where(allowed, z, -np.inf)
    m = np.max(z, axis=1, keepdims=True)
    has = np.isfinite(m)
    p = np.where(allowed, np.exp(z - np.where(has, m, 0.0)), 0.0)
    l = np.sum(p, axis=1, keepdims=True)
    out = (p @ vhat) / np.where(l > 0, l, 1.0)
    return np.where(has, out, 0.0)


def attention_weights(qrows, khat, allowed, sigma) -> np.ndarray:
    """The normalised softmax weights that ``attend`` applies (for invariants)."""
    z = float(sigma) * (np.asarray(qrows, np.float64) @ khat.T)
    z = np.where(allowed, z, -np.inf)
    m = np.max(z, axis=1, keepdims=True)
    p = np.where(allowed, np.exp(z - np.where(np.isfinite(m), m, 0.0)), 0.0)
    l = np.sum(p, axis=1, keepdims=True)
    return p / np.where(l > 0, l, 1.0)


def _sigma(softmax_scale, head_dim) -> float:
    if softmax_scale is None:
        softmax_scale = default_softmax_scale(head_dim)
    return float(np.float32(softmax_scale))


def decode_ref(q_bits, k_q, k_s, v_q, v_s, seq_lens, window, softmax_scale=None):
    """One decode step of one attention layer.

    q_bits uint16 (bf16) [B, Hq, D]; k_q/v_q int8 [B, L_cap, D];
    k_s/v_s fp32 [B, L_cap]; seq_lens [B] (keys including the new token);
    window <= 0 means global. Returns float64 [B, Hq, D].
    """
    return _decode_f64(bf16_bits_to_f64(q_bits), k_q, k_s, v_q, v_s, seq_lens, window, softmax_scale)


def decode_ref_q8(q8, q_scale, k_q, k_s, v_q, v_s, seq_lens, window, softmax_scale=None):
    """Decode step with int8 queries [explinks.com page, 训练和服务的量化:
    activations in int8 too; int8 内核实现: int8 attention kernels].

    q8 int8 [B, Hq, D] with one fp32 scale per (token, head) row, q_scale
    [B, Hq]: the query is the dequantized row q8 * q_scale, so every logit is
    softmax_scale * q_scale * k_scale * (q8 . k8). Otherwise as ``decode_ref``.
    """
    return _decode_f64(dequantize_rows(q8, q_scale), k_q, k_s, v_q, v_s, seq_lens, window, softmax_scale)


def _decode_f64(q, k_q, k_s, v_q, v_s, seq_lens, window, softmax_scale):
    B, Hq, D = q.shape
    sigma = _sigma(softmax_scale, D)
    out = np.zeros((B, Hq, D))
    for b in range(B):
        lo, hi = decode_visible(int(seq_lens[b]), window)
        if hi <= lo:
            continue
        khat = dequantize_rows(k_q[b, lo:hi], k_s[b, lo:hi])
        vhat = dequantize_rows(v_q[b, lo:hi], v_s[b, lo:hi])
        allowed = np.ones((Hq, hi - lo), dtype=bool)
        out[b] = attend(q[b], khat, vhat, allowed, sigma)
    return out


def decode_ref_rows(q_bits, k_q, k_s, v_q, v_s, seq_lens, window, picks,
                    softmax_scale=None):
    """decode_ref for selected (b, h) pairs only; returns [len(picks), D]."""
    q = bf16_bits_to_f64(q_bits)
    D = q.shape[-1]
    sigma = _sigma(softmax_scale, D)
    res = []
    for b, h in picks:
        lo, hi = decode_visible(int(seq_lens[b]), window)
        if hi <= lo:
            res.append(np.zeros(D))
            continue
        khat = dequantize_rows(k_q[b, lo:hi], k_s[b, lo:hi])
        vhat = dequantize_rows(v_q[b, lo:hi], v_s[b, lo:hi])
        res.append(attend(q[b, h][None, :], khat, vhat,
                          np.ones((1, hi - lo), bool), sigma)[0])
    return np.stack(res) if res else np.zeros((0, D))


def prefill_ref(q_bits, k_q, k_s, v_q, v_s, prefix_lens, window,
                softmax_scale=None, positions=None, row_block=32):
    """Attention of a new chunk of C tokens over a cached prefix plus itself.

    q_bits uint16 (bf16) [B, C, Hq, D]; the chunk's own K/V already sit in
    the int8 cache at rows prefix_lens[b] ... prefix_lens[b] + C - 1.
    Query i of sequence b is at absolute position prefix_lens[b] + i and
    attends causally (window W > 0: the last W keys up to itself).
    ``positions`` optionally restricts the computed chunk rows (list of i);
    others are left at zero. Returns float64 [B, C, Hq, D].
    """
    q = bf16_bits_to_f64(q_bits)
    B, C, Hq, D = q.shape
    sigma = _sigma(softmax_scale, D)
    out = np.zeros((B, C, Hq, D))
    rows = list(range(C)) if positions is None else list(positions)
    for b in range(B):
        P = int(prefix_lens[b])
        n = P + C
        khat = dequantize_rows(k_q[b, :n], k_s[b, :n])
        vhat = dequantize_rows(v_q[b, :n], v_s[b, :n])
        for s0 in range(0, len(rows), row_block):
            blk = rows[s0:s0 + row_block]
            allowed = np.zeros((len(blk), n), dtype=bool)
            for t, i in enumerate(blk):
                lo, hi = prefill_visible(P + i, window)
                allowed[t, lo:hi] = True
            qrows = q[b, blk].reshape(len(blk) * Hq, D)
            allowed_rows = np.repeat(allowed, Hq, axis=0)
            o = attend(qrows, khat, vhat, allowed_rows, sigma)
            out[b, blk] = o.reshape(len(blk), Hq, D)
    return out


# ---------------------------------------------------------------------------
# Partition merge  [workshop transcript 00:48:02-00:49:13, online softmax]
# ---------------------------------------------------------------------------

def lse_partial(qrows, khat, vhat, sigma):
    """Running quantities of one key subset: (m, l, o_unnormalised).

    m = max_j z_j, l = sum_j exp(z_j - m), o = sum_j exp(z_j - m) v_j.
    An empty subset is (-inf, 0, 0).
    """
    qrows = np.asarray(qrows, np.float64)
    R, D = qrows.shape[0], vhat.shape[1]
    if khat.shape[0] == 0:
        return np.full(R, -np.inf), np.zeros(R), np.zeros((R, D))
    z = float(sigma) * (qrows @ khat.T)
    m = np.max(z, axis=1)
    p = np.exp(z - m[:, None])
    return m, p.sum(axis=1), p @ vhat


def lse_merge(parts):
    """Combine partials: m = max m_p; l = sum l_p e^(m_p-m); o = sum o_p e^(m_p-m) / l."""
    ms = np.stack([p[0] for p in parts])
    m = np.max(ms, axis=0)
    R = m.shape[0]
    D = parts[0][2].shape[1]
    l = np.zeros(R)
    o = np.zeros((R, D))
    for pm, pl, po in parts:
        w = np.where(np.isfinite(pm), np.exp(pm - np.where(np.isfinite(m), m, 0.0)), 0.0)
        l += pl * w
        o += po * w[:, None]
    return np.where((l > 0)[:, None], o / np.where(l > 0, l, 1.0)[:, None], 0.0)


# ---------------------------------------------------------------------------
# Hybrid block with cross-layer KV sharing  [9c1h.cn page 秘訣1]
# ---------------------------------------------------------------------------

def hybrid_block_ref(q_layers, layer_spec, buffers, seq_lens, softmax_scale=None):
    """Decode step of a block of layers, each reading a (possibly shared) buffer.

    layer_spec: list of (buffer_name, window); buffers: name -> (k_q, k_s, v_q, v_s).
    Layers naming the same buffer read the same arrays.
    """
    outs = []
    for q_bits, (name, window) in zip(q_layers, layer_spec):
        k_q, k_s, v_q, v_s = buffers[name]
        outs.append(decode_ref(q_bits, k_q, k_s, v_q, v_s, seq_lens, window,
                               softmax_scale))
    return outs


# ---------------------------------------------------------------------------
# KV byte accounting  [workshop transcript 00:14:45-00:15:58]
# ---------------------------------------------------------------------------

def kv_bytes_per_token(head_dim, n_layers, n_kv_heads, bytes_per_elem):
    """Bytes of K and V kept per token: 2 (K and V) * D * layers * KV heads * bytes."""
    return 2 * head_dim * n_layers * n_kv_heads * bytes_per_elem


def int8_kv_bytes_per_key(head_dim):
    """One shared head stored as int8 plus an fp32 scale for each of K and V."""
    return 2 * head_dim + 2 * 4


def decode_visible_keys(seq_lens, window):
    return int(sum(decode_visible(int(n), window)[1] - decode_visible(int(n), window)[0]
                   for n in seq_lens))


def prefill_visible_pairs(prefix_lens, chunk, window):
    tot = 0
    for P in prefix_lens:
        for i in range(chunk):
            lo, hi = prefill_visible(int(P) + i, window)
            tot += hi - lo
    return tot


# ---------------------------------------------------------------------------
# Paged KV buffers  [workshop transcript 01:01:35-01:03:22 (logical blocks of
# a sequence mapped to physical blocks of a pool); 9c1h.cn "秘訣1" (a local
# layer only needs its window, so its blocks can be reused as a ring)]
# ---------------------------------------------------------------------------


def paged_rows(table: np.ndarray, block_size: int, b: int, positions) -> np.ndarray:
    """Pool rows of token positions of sequence ``b``: the logical block of a
    position is position // block_size; the table (row b, wrapping around its
    length) names the pool block; the offset inside the block is kept."""
    t = np.asarray(positions, dtype=np.int64)
    logical_block = t // block_size
    pool_block = np.asarray(table, dtype=np.int64)[b, logical_block % table.shape[1]]
    return pool_block * block_size + t % block_size


def paged_gather(pool: np.ndarray, table: np.ndarray, block_size: int, L: int) -> np.ndarray:
    """Logical view [B, L, ...] of a pool [num_blocks, block_size, ...]."""
    flat = pool.reshape((pool.shape[0] * block_size,) + pool.shape[2:])
    B = table.shape[0]
    return np.stack([flat[paged_rows(table, block_size, b, np.arange(L))] for b in range(B)])


def paged_scatter(pool: np.ndarray, table: np.ndarray, block_size: int, rows: np.ndarray,
                  start_pos) -> None:
    """Write rows[b, i] (in order of i) at position start_pos[b] + i of sequence b."""
    flat = pool.reshape((pool.shape[0] * block_size,) + pool.shape[2:])
    for b in range(rows.shape[0]):
        for i in range(rows.shape[1]):
            pos = int(start_pos[b]) + i
            if pos < 0:
                continue
            flat[paged_rows(table, block_size, b, [pos])[0]] = rows[b, i]


def paged_window_resident(window: int, table_len: int, block_size: int) -> bool:
    """Whether a wrapping table still holds the last ``window`` positions
    after positions are appended in order: position t and t + table_len *
    block_size share a pool row, so exactly the last table_len * block_size
    positions are kept."""
    return window <= table_len * block_size

