// mqa_decode: one decode step of multi-query attention over an int8 KV cache.
//
// What is computed (9c1h.cn news page on Character.AI's inference tricks,
// section 秘訣1; explinks.com "Character.AI 的最佳实践", sections 多查询注意力,
// 混合注意力范围, 跨层 KV 共享, 训练和服务的量化): for every sequence b and
// query head h,
//     z_j = scale * s_k[j] * (q_h . k_j)             j in the visible keys
//     out_h = sum_j softmax(z)_j * s_v[j] * v_j
// where k_j, v_j are int8 rows of the ONE shared KV head and the visible keys
// are [max(0, n-W), n) for a window W > 0, else [0, n).
//
// Design for gfx950 (decode is bound by HBM reads of the cache):
//  * One work-group = one sequence x one contiguous range of 32-key tiles
//    (a "partition") x up to 32 query heads (more heads: more head groups
//    in grid z). Each K/V byte is read from HBM once per call and head group
//    and feeds all its heads: this is where MQA's reuse lives. Short visible
//    ranges (sliding windows) instead run 16-head groups over the whole
//    range, with no partitions to merge (plan_decode).
//  * Eight waves per work-group, one work-group per compute unit. The
//    work-group's tiles are handed to its waves from an LDS counter, so the
//    waves finish together whatever the SIMD arbiter favours (which wave sums
//    which tile, and so the last bits of the result, depends on timing; the
//    deterministic setting assigns them in a fixed order instead).
//  * Ragged batches (mqa_decode_ragged): a planner kernel cuts the list of
//    all sequences' visible tiles into ranges of equal cost, one per
//    work-group (a tile costs one unit, the start of a sequence a fixed
//    number); a work-group walks the sequence segments inside its range.
//  * Per 32-key tile a wave runs S^T = K Q^T and O^T += V^T P''^T on fp16
//    MFMA (v_mfma_f32_16x16x32_f16): 32 heads x 128 dims x 2 flops per key
//    per product is far above what the vector ALUs can sustain at HBM rate.
//  * int8 -> fp16 is exact and costs one instruction per element (an SDWA
//    sign-extended byte convert, inline asm with its own MFMA wait states).
//    q is scaled per wave by a power of two into fp16's top binade; the
//    scale is folded into the per-key logit factor.
//  * The contraction index d is permuted consistently in Q and K so that a
//    lane's K bytes are one contiguous run of a key row; the key index is
//    permuted consistently in P'' and V so that the accumulator layout of S^T
//    is directly the B operand of the PV product (no shuffles), and V's
//    column mapping makes each lane's V bytes contiguous within a row.
//  * P'' (below) is split into fp16 hi + lo parts (two MFMAs), so the PV
//    product carries 22 significant bits instead of 11.
//  * Loads are software-pipelined through LDS: each wave owns two slots that
//    direct-to-LDS buffer loads fill (1 KB of contiguous rows per
//    instruction); a slot is read into registers and refilled with the
//    wave's next tile before that tile's arithmetic, so two tiles are in
//    flight while one is computed.
//  * Online softmax (running offset m, sum l, rescaled accumulator) in the
//    log2 domain per head. The waves of a work-group combine through LDS.
//    With several partitions per sequence, each work-group writes its
//    normalised (m, l, o) state and a small second kernel combines them with
//    a log-sum-exp merge (workshop transcript 00:48:02-00:49:13: tiles plus
//    three running quantities give the exact softmax). A kernel boundary is
//    the cheap way to make the states written on one XCD visible to another.
//  * Tiles wholly outside the window are never loaded; only the tiles that
//    straddle a window end are masked per key.
//  * Optionally (mqa_decode_append) the wave that draws the tile holding the
//    sequence's last row first encodes the new token's K and V into it.
#include <math.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "common.h"
#include "launch.h"

namespace mqa {

namespace {

constexpr int kTileKeys = 32;
// Waves per work-group: eight, two per SIMD (a wave's state for up to 32
// heads fits in 256 registers). One work-group per compute unit.
constexpr int kWavesPerWG = 8;
// Heads per work-group: a layer with more query heads is split into groups of
// 32 (grid z), each of which reads the key/value tiles itself. Short key
// ranges (sliding windows) use groups of 16 instead (see plan_decode).
constexpr int kHeadsPerGroup = 32;
// Visible ranges of at most this many tiles run as 16-head work-groups over
// the whole range when those fit on the chip at once: no partition states and
// no merge kernel. Work-group (b, z) has linear id b + B*z, so with B a
// multiple of 8 the head groups of a sequence share an XCD and all but the
// first read the tiles from its L2. (Measured on 64 sequences, window 1024:
// 14.3 us against 16.2 us for four 32-head partitions and the merge.)
constexpr int kShortRangeTiles = 40;

// The PV product takes P'' = 2^(z - m) s_v 2^-vexp in fp16 (hi + lo; largest
// finite fp16 is 65504 < 2^16), with two independent power-of-two scales:
//  * m, the softmax offset per head, is raised lazily, only when a logit
//    exceeds it by more than 2^kLazy (and on the first keys, m = -inf);
//  * vexp, per wave, only rises: it is kept at (largest s_v exponent seen) - 7,
//    so every s_v 2^-vexp < 2^7.
// Hence P'' < 2^(kLazy + 7) = 2^15 for every key, for any scales; the
// accumulator is rescaled when either scale moves (rare).
constexpr float kLazy = 8.0f;
// Paged layout: block-table entries of one partition kept in LDS (the plan
// bounds a partition's tiles so that they span fewer blocks).
constexpr int kMaxTableSlice = 1024;
constexpr int kValueHeadroom = 7;

struct DecodeParams {
  const uint16_t* q;
  // int8 queries (q == nullptr): codes [B, Hq, D] and one fp32 scale per
  // (token, head) row.
  const int8_t* q8;
  const float* q_scale;
  const int8_t* k;
  const int8_t* v;
  const float* ks;
  const float* vs;
  const int32_t* seq_lens;
  float* out;
  // Fused append (k_new != nullptr): the new token's K and V rows, fp32 [B, D],
  // are encoded into row seq_lens[b] - 1 of the (writable) cache.
  const float* k_new;
  const float* v_new;
  int8_t* k_w;
  int8_t* v_w;
  float* ks_w;
  float* vs_w;
  // Paged layout (table != nullptr): k, v, ks, vs are block pools and token
  // position t of sequence b is row table[b][(t >> log2_bs) % table_len]
  // << log2_bs | (t & (2^log2_bs - 1)).
  const int32_t* table;
  int32_t table_len;
  int32_t log2_bs;
  int32_t num_blocks;
  float* ws_o;       // [slots, Hq, D] partition outputs, normalised (natural d order)
  float2* ws_ml;     // [slots, Hq] (offset m in log2 units, sum l of 2^(z - m))
  // Balanced plan of a ragged batch, written by decode_plan_kernel (layout
  // there); plan_G work-groups per head group.
  int32_t* plan;
  int32_t plan_G;
  int32_t plan_inline;      // != 0: each work-group derives its own range of the plan (B <= kInlinePlanMaxB)
  int32_t fixed_tiles;      // != 0: wave w takes tiles w, w + 8, ... (bitwise repeatable)
  int32_t B;
  int32_t L_cap;
  int32_t max_len;          // lengths are clamped to [0, max_len]: the host's max_seq_len (<= L_cap)
  int32_t Hq;
  int32_t heads_per_group;  // 16 or 32 (grid z = ceil(Hq / heads_per_group))
  int32_t window;
  int32_t tiles_per_part;
  int32_t num_parts;
  float scale_log2;  // softmax_scale * log2(e)
};

// Raw bytes of one 32-key tile as one lane needs them.
template <int D>
struct Tile {
  static constexpr int KV4 = D / 64;  // 16-byte K chunks per lane per 16 keys
  static constexpr int VW = D / 64;   // V words per lane per key
  u32x4 k[2][KV4];
  uint32_t v[8][VW];
  f32x4 ks[2];
  f32x4 vs[2];
};

struct SeqBuffers {
  __amdgpu_buffer_rsrc_t k, v, ks, vs;
};

// A tile is staged in LDS: each wave has two slots of its own, filled by
// direct-to-LDS buffer loads (no registers held while in flight). Every load
// instruction reads 1 KB of K or V rows contiguous in memory (a wave reading
// 16 scattered bytes per lane per row measured ~30% slower on the same
// bytes); within each row the 16-byte chunks are stored XOR-swizzled by the
// row index, so that the reads that put the rows into the MFMA operand
// layout are free of bank conflicts. Slot layout: K rows [32][D], V rows
// [32][D], then the 32 K scales and the 32 V scales (each stored twice, lane
// l holding the scale of key l % 32).
template <int D>
struct Slot {
  static constexpr int kCh = D / 16;              // 16-byte chunks per row
  static constexpr int kKV = kTileKeys * D;       // bytes of K (and of V) per tile
  static constexpr int kOffV = kKV;
  static constexpr int kOffKs = 2 * kKV;
  static constexpr int kOffVs = 2 * kKV + 256;
  static constexpr int kBytes = 2 * kKV + 512;
  static constexpr int kDma = 2 * (kKV / 1024) + 2;  // load instructions per tile
};

// Loads are issued unconditionally so the compiler can count them (a load
// under a runtime branch makes it wait for every outstanding load); a tile
// that does not exist is pointed past the buffer ends through the per-lane
// offset, where buffer loads return zero without a memory access (and the
// slot receives zeros).
constexpr uint32_t kNowhere = 0x80000000u;

// The tiles of a sequence's visible keys [lo, n): tile t covers rows
// org + 32 t .. org + 32 t + 31 for t in [begin, end). A full window whose
// length is a multiple of 32 (and a contiguous buffer: paged blocks need
// aligned tiles) is tiled from its first key, so every tile is whole and
// visible (1024 keys: 32 tiles instead of 33, none masked); otherwise tiles
// are aligned to 32 rows and the first and last may be partly visible. Every
// row of a tile lies below max(n, the aligned end) <= the cache capacity.
struct TileRange {
  int org, begin, end;
};
__device__ __forceinline__ TileRange tile_range(int n, int window, bool exact_ok) {
  const int lo = window > 0 ? max(0, n - window) : 0;
  if (exact_ok && window > 0 && window % kTileKeys == 0 && n >= window) return {lo, 0, window / kTileKeys};
  const int b = lo / kTileKeys;
  return {0, b, n > lo ? (n + kTileKeys - 1) / kTileKeys : b};
}

// Per-lane offsets of the staging loads: lane l of a 1 KB load takes chunk
// (l % kCh) ^ (row % kCh) of row l / kCh of that kilobyte, so that LDS chunk
// position p holds chunk (p % kCh) ^ (row % kCh) of row p / kCh.
template <int D>
__device__ __forceinline__ uint32_t stage_lane_offset(int lane) {
  constexpr int CH = Slot<D>::kCh;
  const int r = lane / CH;
  return (uint32_t)(r * D + (((lane % CH) ^ (r % CH)) * 16));
}

// Direct-to-LDS buffer loads: each lane's 16 (or 4) bytes land at
// lds + 16 * lane (or 4 * lane); the 16-byte form optionally non-temporal.
template <bool NT>
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, voff, soff, 0, NT ? kCachePolicyNT : 0);
}
__device__ __forceinline__ void lds_load4(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 4, voff, soff, 0, 0);
}

// Issue the loads of the tile whose first row is `base` (scalar offset) into
// `slot`. The tile base enters as the scalar offset, which the range check of
// a buffer load does not cover: only tiles wholly inside the buffer exist.
template <int D, bool NT>
__device__ __forceinline__ void stage_tile(char* slot, const SeqBuffers& sb, uint32_t lane_kv, uint32_t lane_sc,
                                           int base, bool exists) {
  const uint32_t vk = exists ? lane_kv : kNowhere;
  const uint32_t vs = exists ? lane_sc : kNowhere;
  const uint32_t kv_s = __builtin_amdgcn_readfirstlane(exists ? (uint32_t)base * D : 0u);
  const uint32_t sc_s = __builtin_amdgcn_readfirstlane(exists ? (uint32_t)base * 4 : 0u);
#pragma unroll
  for (int j = 0; j < Slot<D>::kKV / 1024; ++j) lds_load16<NT>(sb.k, slot + j * 1024, vk + j * 1024, kv_s);
#pragma unroll
  for (int j = 0; j < Slot<D>::kKV / 1024; ++j) lds_load16<NT>(sb.v, slot + Slot<D>::kOffV + j * 1024, vk + j * 1024, kv_s);
  lds_load4(sb.ks, slot + Slot<D>::kOffKs, vs, sc_s);
  lds_load4(sb.vs, slot + Slot<D>::kOffVs, vs, sc_s);
}

// The staged tile in the register layout the MFMAs take (see Tile). The
// reads are written out in one asm block that waits for them: the compiler
// cannot tell which slot a staging load in flight writes, and before a read
// of either slot it would wait for all of them (the caller waits for the
// slot's own loads). Lane (g, c) reads K rows c and 16 + c (chunks
// g*KV4 + w, swizzled by the row), V rows 16(i/4) + 4g + i%4 at byte
// c*D/16, and the scales of keys 16hf + 4g .. +3. The same block adds 1 to
// the LDS word at each lane's `claim_addr` and returns its old value in
// `claimed` (the work-group's tile counter for lane 0, a lane-private
// dummy word for the others), so the claim of the wave's next tile shares
// the reads' single wait.
template <int D>
__device__ __forceinline__ void read_slot(Tile<D>& t, const char* slot, int g, int c, uint32_t claim_addr,
                                          int& claimed) {
  constexpr int CH = Slot<D>::kCh;
  constexpr int HALF = 16 * D;  // bytes of 16 rows: rows r and r + 16 share the swizzle
  const uint32_t base = (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)slot);
  uint32_t ak[Tile<D>::KV4], av[4];
#pragma unroll
  for (int w = 0; w < Tile<D>::KV4; ++w) ak[w] = base + (c * CH + ((g * Tile<D>::KV4 + w) ^ (c % CH))) * 16;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * g + i;
    av[i] = base + Slot<D>::kOffV + r * D + (((D == 128 ? c >> 1 : c >> 2) ^ (r % CH)) * 16) +
            (D == 128 ? (c & 1) * 8 : (c & 3) * 4);
  }
  const uint32_t as = base + Slot<D>::kOffKs + 16 * g;
  static_assert(Slot<D>::kOffVs - Slot<D>::kOffKs == 256, "scale layout");
  const uint32_t one = 1;
  if constexpr (D == 128) {
    u32x2 v[8];
    asm volatile(
        "ds_add_rtn_u32 %[cl], %[ca], %[one]\n\t"
        "ds_read_b128 %[k00], %[ak0]\n\t"
        "ds_read_b128 %[k10], %[ak0] offset:2048\n\t"
        "ds_read_b128 %[k01], %[ak1]\n\t"
        "ds_read_b128 %[k11], %[ak1] offset:2048\n\t"
        "ds_read_b64 %[v0], %[av0]\n\t"
        "ds_read_b64 %[v1], %[av1]\n\t"
        "ds_read_b64 %[v2], %[av2]\n\t"
        "ds_read_b64 %[v3], %[av3]\n\t"
        "ds_read_b64 %[v4], %[av0] offset:2048\n\t"
        "ds_read_b64 %[v5], %[av1] offset:2048\n\t"
        "ds_read_b64 %[v6], %[av2] offset:2048\n\t"
        "ds_read_b64 %[v7], %[av3] offset:2048\n\t"
        "ds_read_b128 %[ks0], %[as]\n\t"
        "ds_read_b128 %[ks1], %[as] offset:64\n\t"
        "ds_read_b128 %[vs0], %[as] offset:256\n\t"
        "ds_read_b128 %[vs1], %[as] offset:320\n\t"
        "s_waitcnt lgkmcnt(0)"
        : [k00] "=&v"(t.k[0][0]), [k10] "=&v"(t.k[1][0]), [k01] "=&v"(t.k[0][1]), [k11] "=&v"(t.k[1][1]),
          [v0] "=&v"(v[0]), [v1] "=&v"(v[1]), [v2] "=&v"(v[2]), [v3] "=&v"(v[3]), [v4] "=&v"(v[4]),
          [v5] "=&v"(v[5]), [v6] "=&v"(v[6]), [v7] "=&v"(v[7]), [ks0] "=&v"(t.ks[0]), [ks1] "=&v"(t.ks[1]),
          [vs0] "=&v"(t.vs[0]), [vs1] "=&v"(t.vs[1]), [cl] "=&v"(claimed)
        : [ak0] "v"(ak[0]), [ak1] "v"(ak[1]), [av0] "v"(av[0]), [av1] "v"(av[1]), [av2] "v"(av[2]),
          [av3] "v"(av[3]), [as] "v"(as), [ca] "v"(claim_addr), [one] "v"(one)
        : "memory");
    static_assert(HALF == 2048, "offsets above assume D = 128");
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      t.v[i][0] = v[i][0];
      t.v[i][1] = v[i][1];
    }
  } else {
    static_assert(D == 64 && HALF == 1024, "offsets below assume D = 64");
    uint32_t v[8];
    asm volatile(
        "ds_add_rtn_u32 %[cl], %[ca], %[one]\n\t"
        "ds_read_b128 %[k00], %[ak0]\n\t"
        "ds_read_b128 %[k10], %[ak0] offset:1024\n\t"
        "ds_read_b32 %[v0], %[av0]\n\t"
        "ds_read_b32 %[v1], %[av1]\n\t"
        "ds_read_b32 %[v2], %[av2]\n\t"
        "ds_read_b32 %[v3], %[av3]\n\t"
        "ds_read_b32 %[v4], %[av0] offset:1024\n\t"
        "ds_read_b32 %[v5], %[av1] offset:1024\n\t"
        "ds_read_b32 %[v6], %[av2] offset:1024\n\t"
        "ds_read_b32 %[v7], %[av3] offset:1024\n\t"
        "ds_read_b128 %[ks0], %[as]\n\t"
        "ds_read_b128 %[ks1], %[as] offset:64\n\t"
        "ds_read_b128 %[vs0], %[as] offset:256\n\t"
        "ds_read_b128 %[vs1], %[as] offset:320\n\t"
        "s_waitcnt lgkmcnt(0)"
        : [k00] "=&v"(t.k[0][0]), [k10] "=&v"(t.k[1][0]), [v0] "=&v"(v[0]), [v1] "=&v"(v[1]), [v2] "=&v"(v[2]),
          [v3] "=&v"(v[3]), [v4] "=&v"(v[4]), [v5] "=&v"(v[5]), [v6] "=&v"(v[6]), [v7] "=&v"(v[7]),
          [ks0] "=&v"(t.ks[0]), [ks1] "=&v"(t.ks[1]), [vs0] "=&v"(t.vs[0]), [vs1] "=&v"(t.vs[1]),
          [cl] "=&v"(claimed)
        : [ak0] "v"(ak[0]), [av0] "v"(av[0]), [av1] "v"(av[1]), [av2] "v"(av[2]), [av3] "v"(av[3]),
          [as] "v"(as), [ca] "v"(claim_addr), [one] "v"(one)
        : "memory");
#pragma unroll
    for (int i = 0; i < 8; ++i) t.v[i][0] = v[i];
  }
}

// Running state of one wave: online-softmax quantities of its NT*16 heads.
template <int D, int NT>
struct WaveState {
  f32x4 oacc[D / 16][NT];  // sum of P'' v over the keys seen, P'' = 2^(z - m) s_v 2^-vexp
  float m_run[NT];         // softmax offset per head (log2 units)
  float l_run[NT];         // sum of 2^(z - m), per lane (summed over the 4 key groups at the end)
  int vexp;                // value exponent of the wave (uniform)
};

// Rare path of the online softmax for one head group: some logit of the tile
// exceeds the offset m by more than 2^kLazy (or m = -inf). m becomes the
// largest logit seen; the accumulated state is scaled by 2^(m_old - m_new) and
// t is recomputed. Lanes that did not ask keep m (alpha = 1).
template <int D, int NT>
__device__ __forceinline__ void rebase(WaveState<D, NT>& st, int nt, const f32x4 (&s)[2][NT],
                                       const float (&kscl)[8], const bool (&ok)[8], bool masked, float (&t)[8]) {
  float z[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    z[i] = s[i >> 2][nt][i & 3] * kscl[i];
    if (masked) z[i] = ok[i] ? z[i] : -INFINITY;
  }
  const float zmax = quad_max(max8(z));
  const float m_old = st.m_run[nt];
  const float m_new = fmaxf(m_old, zmax);
  const float alpha = (m_old == -INFINITY) ? 0.f : fast_exp2(m_old - m_new);
  st.m_run[nt] = m_new;
  st.l_run[nt] *= alpha;
#pragma unroll
  for (int mt = 0; mt < D / 16; ++mt) st.oacc[mt][nt] *= alpha;
#pragma unroll
  for (int i = 0; i < 8; ++i) t[i] = (m_new == -INFINITY) ? -INFINITY : z[i] - m_new;
}

// One 32-key tile. A tile that straddles an end of the visible range [lo, hi)
// (at most two per sequence) gives the keys outside it weight zero; the
// branch is wave-uniform and the empty asm keeps the compiler from turning it
// into selects executed for every tile.
// Q^T as an MFMA B operand. Q8 = false: q in fp16, scaled per wave by a
// power of two. Q8 = true: the int8 codes of each (token, head) row as 16-byte
// slices matching the K bytes a lane holds, and the row's scale per lane.
template <int D, int NT, bool Q8>
struct QOperand {
  f16x8 h[NT][D / 32];
};
template <int D, int NT>
struct QOperand<D, NT, true> {
  u32x4 b[NT][D / 64];
  float scale[NT];
};

template <int D, int NT, bool Q8>
__device__ __forceinline__ void compute_tile(Tile<D>& cur, WaveState<D, NT>& st,
                                             const QOperand<D, NT, Q8>& qop,
                                             float kscale, int base, int lo, int hi, int g) {
  constexpr int KK = D / 32;
  constexpr int DPL = D / 16;
  const bool masked = (base < lo) || (base + kTileKeys > hi);  // wave-uniform

  f32x4 s[2][NT];
  if constexpr (!Q8) {
    // ---- S^T = K Q'^T (fp16 operands, exact products, fp32 sums) ----------
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) s[hf][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const u32x4 w = cur.k[hf][kk >> 1];
        const f16x8 kop = as_f16x8(i8x8_to_f16(w[2 * (kk & 1)], w[2 * (kk & 1) + 1]));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) s[hf][nt] = mfma16_f16(kop, qop.h[nt][kk], s[hf][nt]);
      }
    }
  } else {
    // ---- S^T = K8 Q8^T on int8 MFMA: the raw K bytes are the A operand; the
    // int32 sums (|sum| <= D * 127 * 127 < 2^24) convert to fp32 exactly and
    // take the row's q scale.
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        i32x4 acc = {0, 0, 0, 0};
#pragma unroll
        for (int w = 0; w < D / 64; ++w) acc = mfma16_i8(cur.k[hf][w], qop.b[nt][w], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) s[hf][nt][r] = (float)acc[r] * qop.scale[nt];
      }
  }

  // ---- online softmax (log2 domain); P'' = 2^(z - m) s_v as fp16 hi + lo ----
  float kscl[8], vscl[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    kscl[i] = cur.ks[0][i] * kscale;
    kscl[4 + i] = cur.ks[1][i] * kscale;
    vscl[i] = cur.vs[0][i];
    vscl[4 + i] = cur.vs[1][i];
  }
  bool ok[8];
  if (masked) {
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = base + 16 * (i >> 2) + 4 * g + (i & 3);
      ok[i] = (j >= lo) && (j < hi);
      vscl[i] = ok[i] ? vscl[i] : 0.f;
    }
  }
  // Value exponent: every s_v of the tile is below 2^(x - 126), x the largest
  // biased exponent (s_v >= 0, so the bits compare as integers). Each lane
  // checks its own keys; only when one of them needs a larger exponent is
  // the tile's maximum formed (uniform).
  {
    uint32_t xb = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) xb = max(xb, __float_as_uint(vscl[i]));
    int x = (int)(xb >> 23) - 126 - kValueHeadroom;
    if (__builtin_amdgcn_ballot_w64(x > st.vexp) != 0) {  // rare: the accumulator moves to the new value scale
      x = __builtin_amdgcn_readfirstlane(quad_max_i(x));
      const float f = __builtin_ldexpf(1.f, max(st.vexp - x, -200));
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < DPL; ++mt) st.oacc[mt][nt] *= f;
      st.vexp = x;
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) vscl[i] = __builtin_ldexpf(vscl[i], -st.vexp);  // < 2^7
  f16x8 phi[NT], plo[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = fmaf(s[i >> 2][nt][i & 3], kscl[i], -st.m_run[nt]);
    if (masked) {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int i = 0; i < 8; ++i) t[i] = ok[i] ? t[i] : -INFINITY;
    }
    // any lane over the lazy bound (or m = -inf) sends the whole wave to rebase
    const float tmax = max8(t);
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(tmax > kLazy) != 0, 0))
      rebase<D, NT>(st, nt, s, kscl, ok, masked, t);
    u32x4 hw, lw;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const float e0 = fast_exp2(t[i]);
      const float e1 = fast_exp2(t[i + 1]);
      st.l_run[nt] += e0 + e1;
      const u32x2 hl = split_f16(e0 * vscl[i], e1 * vscl[i + 1]);
      hw[i >> 1] = hl[0];
      lw[i >> 1] = hl[1];
    }
    phi[nt] = as_f16x8(hw);
    plo[nt] = as_f16x8(lw);
  }

  // ---- O^T += V^T P''^T -------------------------------------------------------
  static_for<0, DPL>([&](auto MT) {
    constexpr int mt = decltype(MT)::value;
    uint32_t vw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) vw[i] = cur.v[i][mt >> 2];
    const f16x8 vop = as_f16x8(f16_pairs_of_bytes<mt & 3>(vw));
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      st.oacc[mt][nt] = mfma16_f16(vop, phi[nt], st.oacc[mt][nt]);
      st.oacc[mt][nt] = mfma16_f16(vop, plo[nt], st.oacc[mt][nt]);
    }
  });
}

// Fused append: the tile holding the new key (row r of the tile) was loaded
// from the cache, possibly before the row was written; its bytes and scales
// are replaced in registers by the encoded row kept in LDS (K codes at nk[0,D),
// V codes at nk[D, 2D), scales at ns[0..1]). Selects only: no divergence.
template <int D>
__device__ __forceinline__ void patch_new_row(Tile<D>& t, const int8_t* nk, const float* ns, int r, int g, int c) {
  const int hfr = r >> 4, cr = r & 15, gr = cr >> 2, ir = cr & 3;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int w = 0; w < Tile<D>::KV4; ++w) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(nk + g * (D / 4) + 16 * w);
      if (hf == hfr && c == cr) t.k[hf][w] = v;
    }
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int w = 0; w < Tile<D>::VW; ++w) {
      const uint32_t v = *reinterpret_cast<const uint32_t*>(nk + D + c * (D / 16) + 4 * w);
      if (i == 4 * hfr + ir && g == gr) t.v[i][w] = v;
    }
  const float sk = ns[0], sv = ns[1];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (hf == hfr && e == ir && g == gr) {
        t.ks[hf][e] = sk;
        t.vs[hf][e] = sv;
      }
}

// Fused append, done by the wave that draws the tile holding the new key
// (row r of the tile): it encodes the new K and V rows (lane holds elements
// [D/64 * lane, D/64 * (lane + 1)) of each in xk, xv) with the same arithmetic
// as kv_quantize_int8, writes them to the cache row (first head group only),
// and patches the tile registers, which may hold what the cache had before.
template <int D>
__device__ __forceinline__ void encode_new_row(Tile<D>& t, const float (&xk)[D / 64], const float (&xv)[D / 64],
                                               int8_t* row_lds, int r, int g, int c, int lane, bool write,
                                               int8_t* krow, int8_t* vrow, float* ks, float* vs) {
  constexpr int E = D / 64;  // elements per lane
  float ak = 0.f, av = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    ak = fmaxf(ak, fabsf(xk[e]));
    av = fmaxf(av, fabsf(xv[e]));
  }
  ak = wave_max(ak);
  av = wave_max(av);
  const float sk = kv_row_scale(ak), sv = kv_row_scale(av);
  uint32_t ck = 0, cv = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    ck |= ((uint32_t)kv_code(xk[e], sk) & 0xffu) << (8 * e);
    cv |= ((uint32_t)kv_code(xv[e], sv) & 0xffu) << (8 * e);
  }
  // the codes in order in the wave's LDS row buffer: K at [0, D), V at [D, 2D)
  if constexpr (E == 2) {
    reinterpret_cast<uint16_t*>(row_lds)[lane] = (uint16_t)ck;
    reinterpret_cast<uint16_t*>(row_lds + D)[lane] = (uint16_t)cv;
    if (write) {
      reinterpret_cast<uint16_t*>(krow)[lane] = (uint16_t)ck;
      reinterpret_cast<uint16_t*>(vrow)[lane] = (uint16_t)cv;
    }
  } else {
    row_lds[lane] = (int8_t)ck;
    row_lds[D + lane] = (int8_t)cv;
    if (write) {
      krow[lane] = (int8_t)ck;
      vrow[lane] = (int8_t)cv;
    }
  }
  if (write && lane == 0) {
    *ks = sk;
    *vs = sv;
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's own LDS writes are done
  __builtin_amdgcn_wave_barrier();
  const float ns[2] = {sk, sv};
  patch_new_row<D>(t, row_lds, ns, r, g, c);
}

// The work-group's tiles [0, count) (rows row0 + 32 i ..) are handed out to its waves from an
// LDS counter, so waves that run ahead (the SIMDs favour older waves) take
// more tiles and all finish close together. Which wave sums which tile then
// depends on timing, so results can differ between runs in the last bits;
// with `fixed` (the deterministic setting) wave w takes tiles w, w + 8, ...
// instead, and every sum has a fixed order.
// Each wave stages two tiles in its LDS slots: on entry s0 receives its tile
// ia and s1 its tile ib (> ia). A slot is read into the register tile (and
// the slot's next tile claimed in the same LDS round trip), the tile is
// computed, then the slot is refilled: one tile per wave is in flight while
// it computes, two while it waits. (Refilling before the arithmetic, with two
// tiles always in flight, measured ~1 us slower on a 64 x 4096-key global
// call and ~2 us on 8 x 131072 keys: the chip then holds ~36 MB of requests,
// and every load, a segment's q rows and first tiles included, queues behind
// them.)
template <int D, int NT, bool Q8, typename Stage>
__device__ __forceinline__ void run_tiles(char* s0, char* s1, Tile<D>& cur, WaveState<D, NT>& st,
                                          const Stage& stage, const QOperand<D, NT, Q8>& qop, float kscale,
                                          int row0, int count, int ia, int ib, uint32_t claim_addr, int lane,
                                          int lo, int hi,
                                          int g, int new_tile, const float (&xk)[D / 64], const float (&xv)[D / 64],
                                          int8_t* row_lds, bool write, int8_t* krow, int8_t* vrow, float* ks,
                                          float* vs, bool fixed) {
  constexpr int NDMA = Slot<D>::kDma;
  const int c = lane & 15;
  // One tile from `slot`: wait for its loads (only the other slot's may still
  // be in flight), read it and claim the slot's next tile (the counter's, or
  // with a fixed assignment the slot's next one: the wave's two slots
  // alternate), compute, refill the slot.
  const auto step = [&](char* slot, int& i) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(NDMA));
    int claimed;
    read_slot<D>(cur, slot, g, c, claim_addr, claimed);
    const int in = fixed ? i + 2 * kWavesPerWG : __builtin_amdgcn_readfirstlane(claimed);
    if (i == new_tile) {
      encode_new_row<D>(cur, xk, xv, row_lds, hi - 1 - (row0 + i * kTileKeys), g, c, lane, write, krow, vrow, ks,
                        vs);
      // the row's stores count with the staging loads: let them drain so the
      // counts above keep meaning "the other slot's loads"
      __builtin_amdgcn_s_waitcnt(0);
    }
    compute_tile<D, NT, Q8>(cur, st, qop, kscale, row0 + i * kTileKeys, lo, hi, g);
    stage(slot, in);
    i = in;
  };
  // ia < ib at the top of the loop and handed-out indices only grow, so once
  // ia is past the end so is ib (and vice versa in the middle).
  while (ia < count) {
    step(s0, ia);
    if (ib >= count) break;
    step(s1, ib);
  }
}

// ---------------------------------------------------------------------------
// Balanced plan of a ragged batch: up to kInlinePlanMaxB sequences each
// work-group of the attention kernel derives its own part of it; larger
// batches get it from decode_plan_kernel (one work-group of NTH threads: 256
// up to 1024 sequences, measured ~1 us faster than 1024 there, else 1024).
// Work is counted in tile units: a sequence with t_b > 0 visible tiles costs
// kSegmentCost + t_b, the first kSegmentCost units standing for the fixed
// work of starting a segment (the length and q loads before its first tile,
// the combine and state stores after its last). Laid end to end in sequence
// order these costs form one line of C units; with G the work-groups that
// fill the chip once, chunk c = max(8, ceil(C / G)) and work-group j takes
// the tiles whose unit lies in [j c, (j + 1) c), so no work-group's tiles
// plus the segment starts inside its range cost more than c, whatever the
// lengths. (Equal tile counts alone left the work-groups that start several
// short sequences well behind the rest.) Sequence b's tiles occupy units
// A_b .. A_b + t_b - 1, A_b = Q_b + kSegmentCost with Q_b the cost of the
// sequences before it; the part of it in work-group j's range is a segment;
// a work-group's segments are consecutive in (sequence, work-group) order,
// which is also the order of the partial-state slots: sequence b spans
// work-groups A_b / c .. (A_b + t_b - 1) / c and owns that many consecutive
// slots. Written (int32 words): header {c, T, segments, ceil(C / c)}; per
// work-group (G) {first segment, segments} (segments = 0: no work, the first
// word is then -1); per segment (at most G + B) {b, first tile, tiles, length
// of b}; per sequence (B) {first segment, segments}. Lengths are clamped to
// [0, max_len] as the attention kernel clamps them; the attention kernel takes
// a segment's length from the plan, so its first tiles go out at once.
// ---------------------------------------------------------------------------
constexpr int kMinChunk = kWavesPerWG;  // at least one tile per wave
// Batches up to this size are planned inside the attention kernel (one
// sequence per thread of a work-group; no planning kernel, whose launch and
// round trips cost ~5 us per call); larger ones by decode_plan_kernel.
constexpr int kInlinePlanMaxB = 64 * kWavesPerWG;
// On the hybrid block's global layer (128 sequences of 1024..32768 keys, 256
// work-groups) the call took 142, 134, 127, 125, 129 and 132 us with a
// segment cost of 0, 16, 32, 48, 64 and 96 tiles; once a segment's length
// came from the plan and its first tiles went out at once, 40 measured
// ~2.7 us faster than 48 (and 32 ~1 us, 24 no faster).
constexpr int kSegmentCost = kRaggedSegmentCost;

// The tiles the attention kernel computes for a sequence (balanced plans are
// contiguous-buffer plans, so full windows are tiled from their first key).
__device__ __forceinline__ int visible_tiles(int n, int window, int max_len) {
  n = n < 0 ? 0 : (n > max_len ? max_len : n);
  const TileRange tr = tile_range(n, window, true);
  return tr.end - tr.begin;
}
__device__ __forceinline__ int sequence_cost(int t) { return t > 0 ? t + kSegmentCost : 0; }
// Words of the balanced plan's area (layout above).
__host__ __device__ constexpr size_t ragged_plan_words(size_t G, size_t B) { return 4 + 2 * G + 4 * (G + B) + 2 * B; }

// Inclusive prefix sum over the block; `total` receives the block's sum.
template <int NTH>
__device__ __forceinline__ int block_inclusive_sum(int v, int* sm, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  if (lane == 63) sm[w] = v;
  __syncthreads();
  if (w == 0) {
    int x = lane < NTH / 64 ? sm[lane] : 0;
#pragma unroll
    for (int o = 1; o < NTH / 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane < NTH / 64) sm[lane] = x;
  }
  __syncthreads();
  const int add = w > 0 ? sm[w - 1] : 0;
  total = sm[NTH / 64 - 1];
  __syncthreads();  // sm is reused by the next call
  return v + add;
}

// WINDOWED: the layer attends to the last `window` keys (the partition's
// tiles then depend on the sequence length); otherwise to all of them.
// PAGED: the cache is a block pool addressed through p.table.
// Q8: int8 queries (p.q8, p.q_scale) and int8 MFMA for Q K^T.
// RAGGED: balanced plan (a range of the batch's tiles per work-group, one or
// more sequence segments; see decode_plan_kernel).
template <int D, int NT, bool WINDOWED, bool PAGED, bool Q8, bool RAGGED>
__global__ __launch_bounds__(64 * kWavesPerWG) __attribute__((amdgpu_waves_per_eu(2)))
void decode_partition_kernel(DecodeParams p) {
  static_assert(!RAGGED || (!PAGED && !Q8), "balanced plans serve contiguous bf16-query calls");
  static_assert(NT == 1 || NT == 2, "a work-group serves at most 32 heads");
  constexpr int WV = kWavesPerWG;
  constexpr int NTHR = 64 * WV;
  constexpr int KK = D / 32;   // MFMAs along d per 16 keys
  constexpr int DPL = D / 16;  // PV m-tiles; V bytes per lane per key
  constexpr int HP = NT * 16;  // padded head count
  constexpr int NK = NT * DPL; // accumulator tiles per lane

  // Each wave's two staging slots (separate arrays, so the compiler can tell
  // a slot being read from the one being filled). After its last tile a wave
  // parks its accumulators in its own slots: tile nt*DPL+mt of the state,
  // 1 KB per tile in lane order, the first half of the tiles in slot 0.
  __shared__ __attribute__((aligned(16))) char sm_s0[WV][Slot<D>::kBytes];
  __shared__ __attribute__((aligned(16))) char sm_s1[WV][Slot<D>::kBytes];
  static_assert((NK / 2) * kWave * 16 <= Slot<D>::kBytes, "parked state fits the slots");
  const auto parked = [&](int w, int t) -> float* {
    char* base = t < NK / 2 ? sm_s0[w] : sm_s1[w];
    return reinterpret_cast<float*>(base + (t % (NK / 2)) * (kWave * 16));
  };
  __shared__ float sm_m[WV][HP];
  __shared__ float sm_l[WV][HP];
  __shared__ int sm_next;  // next tile (relative to the partition's first) to hand out
  __shared__ int sm_dummy[kWave];  // targets of the claim adds of lanes other than 0
  __shared__ __attribute__((aligned(16))) int8_t sm_new[WV][2 * D];  // fused append: per-wave row buffer
  __shared__ int sm_tab[PAGED ? kMaxTableSlice : 1];  // physical blocks of the partition's tiles
  // Balanced plan derived in the kernel: this work-group's segments.
  __shared__ int4 sm_plan_segs[RAGGED ? kInlinePlanMaxB : 1];
  __shared__ int sm_plan_scan[kWavesPerWG];
  __shared__ int sm_plan_first, sm_plan_n;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int g = lane >> 4;
  const int c = lane & 15;
  const int Hq = p.Hq;                     // heads of the layer (row stride of q and out)
  const int h0 = p.heads_per_group * (int)blockIdx.z;   // first head of this group
  const int Hg = min(Hq - h0, min(p.heads_per_group, NT * 16));    // heads of this group

  // A global layer's K and V are read once per call: non-temporal loads
  // (measured faster). A window's keys are read again by the next layer that
  // shares the buffer, in the same step, and by the next step: default
  // policy, so they may stay in the caches.
  constexpr bool kStreamKV = !WINDOWED;
  const uint32_t lane_kv = stage_lane_offset<D>(lane);
  const uint32_t lane_sc = (uint32_t)(lane & 31) * 4;

  // One segment: sequence b, its visible tiles [seg_lo, seg_lo + seg_len)
  // (relative to the first visible tile; tiles past the visible range are
  // dropped). The states go to partial-state slot `slot`, or straight to the
  // output when the segment is the whole sequence (`direct`).
  // (n_plan: the sequence's clamped length as the balanced plan recorded it;
  // other plans load it here.)
  const auto segment = [&](const int b, const int seg_lo, const int seg_len, const int64_t slot,
                           const bool direct, const int n_plan) {
  // Contiguous layout: one buffer resource per tensor of this sequence (the
  // rows of tiles past the length but inside the capacity are masked).
  // Paged layout: resources are made per tile (below).
  SeqBuffers sb;
  if (!PAGED) {
    sb.k = make_rsrc(p.k + (int64_t)b * p.L_cap * D, (uint32_t)p.L_cap * D);
    sb.v = make_rsrc(p.v + (int64_t)b * p.L_cap * D, (uint32_t)p.L_cap * D);
    sb.ks = make_rsrc(p.ks + (int64_t)b * p.L_cap, (uint32_t)p.L_cap * 4);
    sb.vs = make_rsrc(p.vs + (int64_t)b * p.L_cap, (uint32_t)p.L_cap * 4);
  }
  // Loads go out first: the sequence length, the q rows this lane needs and
  // the new K/V row elements (fused append). A compute unit's vector memory
  // requests are served in order, so every wave issues these before any wave
  // of the work-group issues a tile load (the barrier orders issue, it does
  // not wait for data): behind the tile stream they would return only after
  // most of the unit's first burst of tile loads. They are then waited for
  // while the first tile is in flight. Lane (g, c) takes
  // q[h = 16nt + c][d = g*D/4 + 8kk + 0..7] (bf16), loaded unconditionally
  // through a buffer resource (heads past Hq read as zero).
  // The length goes through the vector memory path: a scalar load would be
  // waited for at the barrier below (it shares a counter with the LDS write
  // before it).
  int n_raw;
  if constexpr (RAGGED) n_raw = n_plan;
  else n_raw = (int)buf_load4(make_rsrc(p.seq_lens + b, 4), 0, 0);
  u32x4 qraw[NT][KK];
  QOperand<D, NT, Q8> qop;
  if constexpr (!Q8) {
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(uniform_ptr(p.q + ((int64_t)b * Hq + h0) * D),
                                                __builtin_amdgcn_readfirstlane((uint32_t)(Hg * D * 2)));
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        qraw[nt][kk] = buf_load16(qr, (uint32_t)(((16 * nt + c) * D + g * (D / 4) + 8 * kk) * 2), 0);
  } else {
    // lane (g, c): bytes g*D/4 + 16w .. +15 of row 16nt + c, the same
    // contraction indices as the K bytes it holds
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(uniform_ptr(p.q8 + ((int64_t)b * Hq + h0) * D),
                                                __builtin_amdgcn_readfirstlane((uint32_t)(Hg * D)));
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(uniform_ptr(p.q_scale + (int64_t)b * Hq + h0),
                                                __builtin_amdgcn_readfirstlane((uint32_t)(Hg * 4)));
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int w = 0; w < D / 64; ++w)
        qop.b[nt][w] = buf_load16(qr, (uint32_t)((16 * nt + c) * D + g * (D / 4) + 16 * w), 0);
      qop.scale[nt] = __uint_as_float(buf_load4(sr, (uint32_t)(16 * nt + c) * 4, 0));
    }
  }
  // fused append: lane holds elements [D/64 * lane, D/64 * (lane + 1)) of the new K and V rows
  const bool appending = p.k_new != nullptr;
  float xk[D / 64], xv[D / 64];
#pragma unroll
  for (int e = 0; e < D / 64; ++e) {
    xk[e] = appending ? p.k_new[(int64_t)b * D + (D / 64) * lane + e] : 0.f;
    xv[e] = appending ? p.v_new[(int64_t)b * D + (D / 64) * lane + e] : 0.f;
  }
  if (threadIdx.x == 0) sm_next = 2 * WV;
  __syncthreads();

  // A global layer's first tile per wave does not depend on the sequence
  // length: it is loaded before the length arrives if it lies inside the
  // cache capacity (a tile past the length is never computed).
  // A windowed layer needs the length to place its tiles. (Issuing the second
  // tile this early too measured slower: the first work-groups' loads then
  // delay the q loads of those dispatched last.)
  char* const s0 = sm_s0[wave];
  char* const s1 = sm_s1[wave];
  if (!WINDOWED && !PAGED && !RAGGED) {
    const int t0 = seg_lo + wave;
    stage_tile<D, kStreamKV>(s0, sb, lane_kv, lane_sc, t0 * kTileKeys, wave < seg_len && (t0 + 1) * kTileKeys <= p.L_cap);
  }

  int n = __builtin_amdgcn_readfirstlane(n_raw);  // same for the whole work-group
  // A length beyond the host's max_seq_len (a caller error) is read as
  // max_seq_len: the plan's partitions cover exactly those keys (the
  // balanced planner clamps the same way).
  n = n < 0 ? 0 : (n > p.max_len ? p.max_len : n);
  const int lo = WINDOWED ? max(0, n - p.window) : 0;
  const int hi = n;
  const TileRange tr = tile_range(n, WINDOWED ? p.window : 0, !PAGED);
  const int org = tr.org;  // row of tile 0 (0 unless a full window is tiled from its first key)
  const int pt0 = tr.begin + seg_lo;
  const int pt1 = min(pt0 + seg_len, tr.end);
  const int count = pt1 - pt0;  // tiles of this segment (may be <= 0)
  // Fused append: the wave that draws the tile holding row n - 1 encodes it.
  const int new_tile = (appending && n > 0) ? (n - 1 - org) / kTileKeys - pt0 : -1;  // outside [0, count): none here

  // Paged: the physical blocks of this partition's tiles, read once into LDS
  // (entries clamped into the pool, so no access can leave it).
  const int blk0 = PAGED ? (pt0 * kTileKeys) >> p.log2_bs : 0;
  if (PAGED) {
    const int nblk = count > 0 ? (((pt0 + count) * kTileKeys - 1) >> p.log2_bs) - blk0 + 1 : 0;
    const int32_t* trow = p.table + (int64_t)b * p.table_len;
    for (int i = threadIdx.x; i < nblk; i += NTHR) {
      const int e = trow[(blk0 + i) % p.table_len];
      sm_tab[i] = e < 0 ? 0 : (e >= p.num_blocks ? p.num_blocks - 1 : e);
    }
    __syncthreads();
  }
  // Physical row of token position `pos` (a position of this partition).
  const auto phys_row = [&](int pos) -> int64_t {
    if (!PAGED) return (int64_t)b * p.L_cap + pos;
    const int e = sm_tab[(pos >> p.log2_bs) - blk0];
    return ((int64_t)e << p.log2_bs) | (pos & ((1 << p.log2_bs) - 1));
  };
  const int64_t new_row = (new_tile >= 0 && new_tile < count) ? phys_row(n - 1) : 0;
  // Staging loads of tile i of the partition (i >= count: nothing is read).
  const auto stage = [&](char* slot, int i) {
    if (!PAGED) {
      stage_tile<D, kStreamKV>(slot, sb, lane_kv, lane_sc, org + (pt0 + i) * kTileKeys, i < count);
    } else {
      SeqBuffers tsb;
      const int64_t row = i < count ? phys_row((pt0 + i) * kTileKeys) : 0;
      const uint32_t kvb = i < count ? (uint32_t)(kTileKeys * D) : 0u, scb = i < count ? (uint32_t)(kTileKeys * 4) : 0u;
      tsb.k = make_rsrc(p.k + row * D, kvb);
      tsb.v = make_rsrc(p.v + row * D, kvb);
      tsb.ks = make_rsrc(p.ks + row, scb);
      tsb.vs = make_rsrc(p.vs + row, scb);
      stage_tile<D, kStreamKV>(slot, tsb, lane_kv, lane_sc, 0, i < count);
    }
  };
  if (WINDOWED || PAGED || RAGGED) stage(s0, wave);
  stage(s1, wave + WV);

  // Q^T as the B operand in fp16: the wave scales q by an exact power of two
  // that puts its largest |q| in [2^14, 2^15) and folds the scale into its
  // per-key logit factor (waves may differ; each works with true logits).
  float kscale = p.scale_log2;
  if constexpr (!Q8) {
    float qmax = 0.f;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          qmax = fmaxf(qmax, fmaxf(fabsf(bf16_lo_to_f32(qraw[nt][kk][e])), fabsf(bf16_hi_to_f32(qraw[nt][kk][e]))));
    qmax = wave_max(qmax);
    int eq = qmax > 0.f ? __builtin_amdgcn_frexp_expf(qmax) : 0;  // qmax < 2^eq
    eq = eq < -100 ? -100 : eq;
    const float qup = __builtin_ldexpf(1.f, 15 - eq);
    kscale = p.scale_log2 * __builtin_ldexpf(1.f, eq - 15);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w[e] = cvt_pk_f16(bf16_lo_to_f32(qraw[nt][kk][e]) * qup, bf16_hi_to_f32(qraw[nt][kk][e]) * qup);
        qop.h[nt][kk] = as_f16x8(w);
      }
  }

  WaveState<D, NT> st;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    st.m_run[nt] = -INFINITY;
    st.l_run[nt] = 0.f;
#pragma unroll
    for (int mt = 0; mt < DPL; ++mt) st.oacc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  st.vexp = -1000;

  Tile<D> cur;
  const auto lds_addr = [](int* p_) {
    return (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) int*)p_);
  };
  const uint32_t claim_addr =
      (lane == 0 && p.fixed_tiles == 0) ? lds_addr(&sm_next) : lds_addr(&sm_dummy[lane]);
  run_tiles<D, NT, Q8>(s0, s1, cur, st, stage, qop, kscale, org + pt0 * kTileKeys, count, wave, wave + WV, claim_addr,
                       lane, lo, hi, g,
                   new_tile, xk, xv, sm_new[wave], blockIdx.z == 0, p.k_w + new_row * D, p.v_w + new_row * D,
                   p.ks_w + new_row, p.vs_w + new_row, p.fixed_tiles != 0);

  // ---- combine the waves of the work-group -----------------------------------
  // Each wave parks its raw accumulators and (m, l) per head in LDS (lane-ordered
  // 16-byte stores, conflict free) once its own staging loads have landed (the
  // last ones, of tiles past the end, write zeros into its slots); after one
  // barrier, job (nt, g', c, r)
  // combines all waves' values of head 16nt + c at dims DPL*(4g' + r) + 0..DPL-1,
  // which are contiguous in the output row.
  // Parked states are normalised, o / l with the value scale folded back
  // (2^vexp), so that no partial sum can overflow fp32.
  __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float l = quad_sum(st.l_run[nt]);
    if (g == 0) {
      sm_m[wave][16 * nt + c] = st.m_run[nt];
      sm_l[wave][16 * nt + c] = l;
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int mt = 0; mt < DPL; ++mt) {
      f32x4 o = st.oacc[mt][nt] * inv;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = __builtin_ldexpf(o[r], st.vexp);
      *reinterpret_cast<f32x4*>(parked(wave, nt * DPL + mt) + lane * 4) = o;
    }
  }
  __syncthreads();

  // NT * 256 jobs over the work-group's threads: with 16 heads two threads
  // share a job, each combining half of its dims.
  constexpr int SPLIT = NTHR / (NT * 256);
  constexpr int DPS = DPL / SPLIT;
  static_assert(SPLIT * NT * 256 == NTHR && DPS * SPLIT == DPL && DPS % 2 == 0, "combine split");
  {
    const int job = threadIdx.x / SPLIT, part = threadIdx.x % SPLIT;
    const int nt = job >> 8;
    const int gq = (job >> 6) & 3;
    const int cc = (job >> 2) & 15;
    const int rr = job & 3;
    const int h = 16 * nt + cc;
    const int d0 = DPL * (4 * gq + rr) + DPS * part;
    float mw[WV], f[WV];
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < WV; ++w) {
      mw[w] = sm_m[w][h];
      M = fmaxf(M, mw[w]);
    }
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < WV; ++w) {
      f[w] = (mw[w] == -INFINITY) ? 0.f : fast_exp2(mw[w] - M) * sm_l[w][h];  // empty wave: no weight
      L += f[w];
    }
    const float invL = L > 0.f ? 1.f / L : 0.f;
    float o[DPS];
#pragma unroll
    for (int mi = 0; mi < DPS; ++mi) {
      const int mt = DPS * part + mi;
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < WV; ++w)
        acc += f[w] * parked(w, nt * DPL + mt)[(16 * gq + cc) * 4 + rr];
      o[mi] = acc * invL;  // normalised: the output itself, or this partition's share
    }
    if (h < Hg) {
      float* dst;
      if (direct) {
        dst = p.out + ((int64_t)b * Hq + h0 + h) * D + d0;
      } else {
        dst = p.ws_o + (slot * Hq + h0 + h) * D + d0;
        if (part == 0 && gq == 0 && rr == 0) p.ws_ml[slot * Hq + h0 + h] = make_float2(M, L);
      }
      if constexpr (DPS % 4 == 0) {
#pragma unroll
        for (int u = 0; u < DPS; u += 4)
          *reinterpret_cast<f32x4*>(dst + u) = f32x4{o[u], o[u + 1], o[u + 2], o[u + 3]};
      } else {
#pragma unroll
        for (int u = 0; u < DPS; u += 2) *reinterpret_cast<float2*>(dst + u) = make_float2(o[u], o[u + 1]);
      }
    }
  }
  };

  if constexpr (!RAGGED) {
    const int part = blockIdx.x, tpp = p.tiles_per_part;
    segment(blockIdx.y, part * tpp, tpp, (int64_t)blockIdx.y * p.num_parts + part, p.num_parts == 1, 0);
  } else {
    // the segments of this work-group's range of the balanced plan, in order
    // (each segment begins with a barrier, so the previous one's combine is
    // over before its LDS is reused)
    int first, nseg, seg0;
    const int4* segs;
    if (p.plan_inline) {
      // This work-group's range of the plan decode_plan_kernel would write
      // (same integer arithmetic, one sequence per thread): its segments go
      // to LDS, and the per-sequence words the merge kernel reads are written
      // by the work-group holding each sequence's first segment (work-group 0
      // for sequences with no visible tile).
      const int b = threadIdx.x;
      const int nb = b < p.B ? min(max(p.seq_lens[b], 0), p.max_len) : 0;
      const int t = b < p.B ? visible_tiles(nb, WINDOWED ? p.window : 0, p.max_len) : 0;
      const int cost = sequence_cost(t);
      if (threadIdx.x == 0) {
        sm_plan_first = 0x7fffffff;
        sm_plan_n = 0;
      }
      int total_c, total_s;
      const int Q = block_inclusive_sum<NTHR>(cost, sm_plan_scan, total_c) - cost;
      const int chunk = (int)max<int64_t>(kMinChunk, ((int64_t)total_c + p.plan_G - 1) / p.plan_G);
      const int A = Q + kSegmentCost;
      const int j1 = A / chunk, j2 = (int)(((int64_t)A + t - 1) / chunk);
      const int ns = t > 0 ? j2 - j1 + 1 : 0;
      const int S = block_inclusive_sum<NTHR>(ns, sm_plan_scan, total_s) - ns;
      const int j = blockIdx.x;
      const bool mine = t > 0 && j1 <= j && j <= j2;
      int lo = 0, hi = 0;
      if (mine) {
        const int64_t start = (int64_t)j * chunk;
        lo = (int)max(start, (int64_t)A);
        hi = (int)min(start + chunk, (int64_t)A + t);
        atomicMin(&sm_plan_first, S + j - j1);
        atomicAdd(&sm_plan_n, 1);
      }
      if (blockIdx.z == 0 && b < p.B && (t > 0 ? j1 == j : j == 0)) {
        int32_t* seqs = p.plan + ragged_plan_words(p.plan_G, p.B) - 2 * p.B;
        *reinterpret_cast<int2*>(seqs + 2 * b) = make_int2(S, ns);
      }
      __syncthreads();
      first = __builtin_amdgcn_readfirstlane(sm_plan_first);
      nseg = __builtin_amdgcn_readfirstlane(sm_plan_n);
      if (mine) sm_plan_segs[S + j - j1 - first] = make_int4(b, lo - A, hi - lo, nb);
      __syncthreads();
      segs = sm_plan_segs;
      seg0 = 0;
    } else {
      const int2 wg = *reinterpret_cast<const int2*>(p.plan + 4 + 2 * blockIdx.x);
      first = __builtin_amdgcn_readfirstlane(wg.x);
      nseg = __builtin_amdgcn_readfirstlane(wg.y);
      segs = reinterpret_cast<const int4*>(p.plan + 4 + 2 * p.plan_G);
      seg0 = first;
    }
    for (int k = 0; k < nseg; ++k) {
      const int4 sg = segs[seg0 + k];
      const int seg_lo = __builtin_amdgcn_readfirstlane(sg.y), seg_len = __builtin_amdgcn_readfirstlane(sg.z);
      const int n = __builtin_amdgcn_readfirstlane(sg.w);
      // a segment holding all of the sequence's tiles writes the output directly
      const TileRange tr = tile_range(n, WINDOWED ? p.window : 0, true);
      segment(__builtin_amdgcn_readfirstlane(sg.x), seg_lo, seg_len, (int64_t)(first + k),
              seg_lo == 0 && seg_len == tr.end - tr.begin, n);
    }
  }
}

// Log-sum-exp merge of the partition states of one sequence and a group of
// heads, o_p normalised: m = max_p m_p; w_p = l_p 2^(m_p - m);
// out = sum_p w_p o_p / sum_p w_p.
// 256 threads = 8 heads x 32 float4 columns (D = 128) or 16 heads x 16
// columns (D = 64), times S partition slices (block = 256 S threads, S <= 4):
// slice s merges partitions s, s + S, ... with eight loads in flight at a
// time and a running rescale, then slice 0 combines the S slices through LDS.
// A long context (tens of partitions per sequence) thus needs one or two
// dependent memory round trips instead of one per eight partitions.
constexpr int kMergeMaxSlices = 4;
template <int D>
__global__ __launch_bounds__(256 * kMergeMaxSlices) void decode_merge_kernel(const float* __restrict__ ws_o,
                                                                             const float2* __restrict__ ws_ml,
                                                                             float* __restrict__ out, int Hq, int P,
                                                                             const int32_t* __restrict__ plan,
                                                                             int seq_off) {
  constexpr int D4 = D / 4;
  constexpr int HPB = 256 / D4;  // heads per block
  __shared__ f32x4 s_acc[kMergeMaxSlices - 1][256];
  __shared__ float2 s_ml[kMergeMaxSlices - 1][256];
  const int S = blockDim.x / 256;
  const int slice = threadIdx.x / 256;
  const int t = threadIdx.x % 256;
  const int b = blockIdx.y;
  const int h = blockIdx.x * HPB + t / D4;
  const int d0 = 4 * (t % D4);
  const bool live_h = h < Hq;
  // States of sequence b: slots s0 .. s0 + P - 1. Balanced plan: the
  // sequence's segments wrote consecutive slots; a sequence in one segment was
  // written to the output directly, one with no visible key gets zeros.
  int64_t s0 = (int64_t)b * P;
  if (plan != nullptr) {
    const int2 sq = *reinterpret_cast<const int2*>(plan + seq_off + 2 * b);
    if (sq.y == 1) return;
    s0 = sq.x;
    P = sq.y;
  }
  const float2* ml = ws_ml + s0 * Hq + h;
  const float* wo = ws_o + (s0 * Hq + h) * D + d0;
  float M = -INFINITY, L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int q0 = slice; q0 < P; q0 += 8 * S) {
    float2 st[8];
    f32x4 o[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int pp = q0 + u * S;
      const bool live = live_h && pp < P;
      st[u] = live ? ml[(int64_t)pp * Hq] : make_float2(-INFINITY, 0.f);
      o[u] = live ? *reinterpret_cast<const f32x4*>(wo + (int64_t)pp * Hq * D) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float Mc = M;
#pragma unroll
    for (int u = 0; u < 8; ++u) Mc = fmaxf(Mc, st[u].x);
    if (Mc == -INFINITY) continue;
    const float a = exp2f(M - Mc);  // 0 while nothing has been seen
    acc *= a;
    L *= a;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float w = exp2f(st[u].x - Mc) * st[u].y;  // 0 for an empty partition
      L += w;
      acc += w * o[u];
    }
    M = Mc;
  }
  if (S > 1) {
    if (slice > 0) {
      s_acc[slice - 1][t] = acc;
      s_ml[slice - 1][t] = make_float2(M, L);
    }
    __syncthreads();
    if (slice > 0) return;
    for (int j = 0; j < S - 1; ++j) {
      const float2 x = s_ml[j][t];
      const float Mc = fmaxf(M, x.x);
      if (Mc == -INFINITY) continue;
      const float a = exp2f(M - Mc), w = exp2f(x.x - Mc);
      acc = acc * a + s_acc[j][t] * w;
      L = L * a + x.y * w;
      M = Mc;
    }
  }
  if (!live_h) return;
  const float inv = L > 0.f ? 1.f / L : 0.f;
  *reinterpret_cast<f32x4*>(out + ((int64_t)b * Hq + h) * D + d0) = acc * inv;
}

template <int NTH>
__global__ __launch_bounds__(NTH) void decode_plan_kernel(const int32_t* __restrict__ seq_lens,
                                                                   int32_t* __restrict__ plan, int B, int window,
                                                                   int max_len, int G) {
  __shared__ int sm[NTH / 64];
  const int tid = threadIdx.x;
  int part_t = 0, part_c = 0;
  for (int b = tid; b < B; b += NTH) {
    const int t = visible_tiles(seq_lens[b], window, max_len);
    part_t += t;
    part_c += sequence_cost(t);
  }
  int total_t, total_c;
  (void)block_inclusive_sum<NTH>(part_t, sm, total_t);
  (void)block_inclusive_sum<NTH>(part_c, sm, total_c);
  const int chunk = (int)max<int64_t>(kMinChunk, ((int64_t)total_c + G - 1) / G);
  int32_t* wg = plan + 4;
  int32_t* segs = plan + 4 + 2 * G;
  int32_t* seqs = segs + 4 * (G + B);
  for (int j = tid; j < G; j += NTH) *reinterpret_cast<int2*>(wg + 2 * j) = make_int2(-1, 0);
  __syncthreads();
  int carry_c = 0, carry_s = 0;
  for (int base = 0; base < B; base += NTH) {
    const int b = base + tid;
    const int nb = b < B ? min(max(seq_lens[b], 0), max_len) : 0;   // clamped as the attention kernel clamps
    const int t = visible_tiles(nb, window, max_len);
    const int cost = sequence_cost(t);
    int tot_c, tot_s;
    const int Q = carry_c + block_inclusive_sum<NTH>(cost, sm, tot_c) - cost;  // cost of the sequences before b
    const int A = Q + kSegmentCost;                                              // unit of its first tile
    const int j1 = A / chunk, j2 = (int)(((int64_t)A + t - 1) / chunk);
    const int n = t > 0 ? j2 - j1 + 1 : 0;
    const int S = carry_s + block_inclusive_sum<NTH>(n, sm, tot_s) - n;  // segments before sequence b
    if (b < B) {
      *reinterpret_cast<int2*>(seqs + 2 * b) = make_int2(S, n);
      // the previous sequence with tiles ends at unit Q - 1: is it in j1's range?
      const bool shares_j1 = Q > 0 && (Q - 1) / chunk == j1;
      for (int k = 0; k < n; ++k) {
        const int j = j1 + k;
        const int64_t start = (int64_t)j * chunk;  // 64-bit: (j + 1) c may pass 2^31
        const int lo = (int)max(start, (int64_t)A), hi = (int)min(start + chunk, (int64_t)A + t);
        *reinterpret_cast<int4*>(segs + 4 * (S + k)) = make_int4(b, lo - A, hi - lo, nb);
        if (k > 0 || !shares_j1) wg[2 * j] = S + k;  // the first segment of work-group j's range
      }
    }
    carry_c += tot_c;
    carry_s += tot_s;
  }
  __syncthreads();  // every work-group's first segment is written
  for (int j = tid; j < G; j += NTH) {
    const int first = wg[2 * j];
    if (first < 0) continue;  // no tile in this range
    int next = carry_s;
    for (int i = j + 1; i < G; ++i) {
      const int f = wg[2 * i];
      if (f >= 0) {
        next = f;
        break;
      }
    }
    wg[2 * j + 1] = next - first;
  }
  if (tid == 0) {
    plan[0] = chunk;
    plan[1] = total_t;
    plan[2] = carry_s;
    plan[3] = (int)(((int64_t)total_c + chunk - 1) / chunk);
  }
}


template <int D, int NT, bool PAGED, bool Q8, bool RAGGED>
void launch_partitions(const DecodeParams& prm, int B, int G, hipStream_t stream) {
  const dim3 block(64 * kWavesPerWG);
  const int groups = (prm.Hq + prm.heads_per_group - 1) / prm.heads_per_group;
  // balanced plan: G work-groups per head group, each over its range of the plan
  const dim3 grid = RAGGED ? dim3(G, 1, groups) : dim3(prm.num_parts, B, groups);
  if (prm.window > 0)
    hipLaunchKernelGGL((decode_partition_kernel<D, NT, true, PAGED, Q8, RAGGED>), grid, block, 0, stream, prm);
  else
    hipLaunchKernelGGL((decode_partition_kernel<D, NT, false, PAGED, Q8, RAGGED>), grid, block, 0, stream, prm);
}

template <int D>
void launch_by_heads(const DecodeParams& prm, int B, int G, hipStream_t stream) {
  // int8 queries are served on contiguous buffers only; balanced plans on
  // contiguous buffers with bf16 queries
  const bool paged = prm.table != nullptr, q8 = prm.q8 != nullptr, ragged = prm.plan != nullptr;
  if (prm.Hq <= 16 || prm.heads_per_group <= 16) {
    if (q8) launch_partitions<D, 1, false, true, false>(prm, B, G, stream);
    else if (paged) launch_partitions<D, 1, true, false, false>(prm, B, G, stream);
    else if (ragged) launch_partitions<D, 1, false, false, true>(prm, B, G, stream);
    else launch_partitions<D, 1, false, false, false>(prm, B, G, stream);
  } else {
    if (q8) launch_partitions<D, 2, false, true, false>(prm, B, G, stream);
    else if (paged) launch_partitions<D, 2, true, false, false>(prm, B, G, stream);
    else if (ragged) launch_partitions<D, 2, false, false, true>(prm, B, G, stream);
    else launch_partitions<D, 2, false, false, false>(prm, B, G, stream);
  }
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }


}  // namespace

DecodePlan plan_decode(int32_t B, int32_t Hq, int32_t D, int32_t max_seq_len, int32_t window,
                       int num_cus, int32_t block_size) {
  DecodePlan pl{1, 1, 0, kHeadsPerGroup, max_seq_len, 0};
  // Upper bound of 32-key tiles a sequence's visible range can touch.
  int64_t ntiles;
  if (window > 0 && window < max_seq_len)
    ntiles = (window + kTileKeys - 1) / kTileKeys + 1;  // window start may be unaligned
  else
    ntiles = ((int64_t)max_seq_len + kTileKeys - 1) / kTileKeys;
  if (ntiles < 1) ntiles = 1;
  // Aim at one work-group per compute unit, with at least one tile per wave.
  const int64_t target = num_cus > 0 ? num_cus : 256;
  if (Hq > 16 && ntiles <= kShortRangeTiles && (int64_t)B * ((Hq + 15) / 16) <= target) {
    pl.tiles_per_part = (int)ntiles;
    pl.heads_per_group = 16;
    return pl;
  }
  const int64_t wv = kWavesPerWG;
  const int64_t groups = (Hq + kHeadsPerGroup - 1) / kHeadsPerGroup;
  int64_t tpp = ((int64_t)B * groups * ntiles + target - 1) / target;
  if (tpp < wv) tpp = wv;
  if (tpp > ntiles) tpp = ntiles;
  // Paged: a partition's tiles must span at most kMaxTableSlice blocks.
  if (block_size > 0) {
    const int64_t cap = (int64_t)(kMaxTableSlice - 2) * block_size / kTileKeys;
    if (tpp > cap) tpp = cap;
  }
  const int64_t parts = (ntiles + tpp - 1) / tpp;
  pl.tiles_per_part = (int)tpp;
  pl.num_parts = (int)parts;
  if (parts > 1) {
    const size_t slots = (size_t)B * (size_t)parts * (size_t)Hq;
    pl.ws_bytes = align_up(slots * sizeof(float2), 256) + align_up(slots * (size_t)D * sizeof(float), 256);
  }
  return pl;
}

DecodePlan plan_decode_ragged(int32_t B, int32_t Hq, int32_t D, int32_t max_seq_len, int32_t window,
                              int num_cus) {
  // Sliding windows short enough for the whole-range plan keep it: every
  // sequence's work is then at most one window.
  DecodePlan pl = plan_decode(B, Hq, D, max_seq_len, window, num_cus);
  if (pl.heads_per_group == 16) return pl;
  const int64_t groups = (Hq + kHeadsPerGroup - 1) / kHeadsPerGroup;
  const int64_t target = num_cus > 0 ? num_cus : 256;
  const int64_t G = std::max<int64_t>(1, target / groups);
  pl.ragged_groups = (int)G;
  pl.heads_per_group = kHeadsPerGroup;
  pl.tiles_per_part = 0;
  pl.num_parts = 0;
  const size_t plan_words = ragged_plan_words((size_t)G, (size_t)B);
  const size_t slots = ((size_t)G + (size_t)B) * (size_t)Hq;
  pl.ws_bytes = align_up(plan_words * sizeof(int32_t), 256) + align_up(slots * sizeof(float2), 256) +
                align_up(slots * (size_t)D * sizeof(float), 256);
  return pl;
}

// Device memory of the allocation-free decode entry point: the partition
// states of one call (each GPU holds its own copy for the life of the
// process). In host code `scratch` names a host-side stand-in, never the
// device array: its device address is looked up once per device.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxScratchDevices];
std::mutex g_scratch_mu;
}  // namespace

void* static_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  void* ptr = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (ptr != nullptr) return ptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ptr = g_scratch_addr[dev].load(std::memory_order_relaxed);
  if (ptr == nullptr) {
    // the current device is `dev`: the address returned is its copy's
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_addr[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}

namespace {
std::atomic<bool> g_fixed_tiles{false};
}  // namespace

bool set_deterministic(bool on) { return g_fixed_tiles.exchange(on); }

int launch_decode(const uint16_t* q, const mqa_kv_view& kv, const KVLayout& layout, const int32_t* seq_lens,
                  int32_t B, int32_t Hq, int32_t D, int32_t window, float softmax_scale, float* out,
                  void* workspace, const DecodePlan& plan, hipStream_t stream, const AppendRows* append,
                  const QueryInt8* q8) {
  DecodeParams prm;
  prm.q8 = q8 ? q8->codes : nullptr;
  prm.q_scale = q8 ? q8->scale : nullptr;
  prm.table = layout.table;
  prm.table_len = layout.table_len;
  prm.log2_bs = layout.log2_bs;
  prm.num_blocks = layout.num_blocks;
  prm.k_new = append ? append->k_new : nullptr;
  prm.v_new = append ? append->v_new : nullptr;
  prm.k_w = append ? append->k : nullptr;
  prm.v_w = append ? append->v : nullptr;
  prm.ks_w = append ? append->k_scale : nullptr;
  prm.vs_w = append ? append->v_scale : nullptr;
  prm.q = q;
  prm.k = kv.k;
  prm.v = kv.v;
  prm.ks = kv.k_scale;
  prm.vs = kv.v_scale;
  prm.seq_lens = seq_lens;
  prm.out = out;
  prm.L_cap = layout.table ? layout.L_cap : kv.L_cap;
  prm.max_len = std::min(plan.max_seq_len, prm.L_cap);
  prm.Hq = Hq;
  prm.heads_per_group = plan.heads_per_group;
  prm.window = window;
  prm.tiles_per_part = plan.tiles_per_part;
  prm.num_parts = plan.num_parts;
  prm.scale_log2 = softmax_scale * 1.4426950408889634f;
  prm.ws_o = nullptr;
  prm.ws_ml = nullptr;
  prm.plan = nullptr;
  prm.plan_G = 0;
  prm.plan_inline = 0;
  prm.fixed_tiles = g_fixed_tiles.load(std::memory_order_relaxed) ? 1 : 0;
  prm.B = B;
  const int G = plan.ragged_groups;
  if (G > 0) {
    // balanced plan: plan area, then the states of G + B slots
    const size_t plan_words = ragged_plan_words((size_t)G, (size_t)B);
    const size_t slots = ((size_t)G + (size_t)B) * (size_t)Hq;
    char* ws = static_cast<char*>(workspace);
    int32_t* plan_area = reinterpret_cast<int32_t*>(ws);
    ws += align_up(plan_words * sizeof(int32_t), 256);
    prm.ws_ml = reinterpret_cast<float2*>(ws);
    ws += align_up(slots * sizeof(float2), 256);
    prm.ws_o = reinterpret_cast<float*>(ws);
    prm.plan = plan_area;
    prm.plan_G = G;
    // small batches are planned inside the attention kernel
    prm.plan_inline = B <= kInlinePlanMaxB ? 1 : 0;
    if (!prm.plan_inline) {
      if (B <= 1024)
        hipLaunchKernelGGL(decode_plan_kernel<256>, dim3(1), dim3(256), 0, stream, seq_lens, plan_area, B, window,
                           prm.max_len, G);
      else
        hipLaunchKernelGGL(decode_plan_kernel<1024>, dim3(1), dim3(1024), 0, stream, seq_lens, plan_area, B,
                           window, prm.max_len, G);
      if (hipGetLastError() != hipSuccess) return MQA_ERR_HIP;
    }
  } else if (plan.num_parts > 1) {
    const size_t slots = (size_t)B * (size_t)plan.num_parts * (size_t)Hq;
    char* ws = static_cast<char*>(workspace);
    prm.ws_ml = reinterpret_cast<float2*>(ws);
    ws += align_up(slots * sizeof(float2), 256);
    prm.ws_o = reinterpret_cast<float*>(ws);
  }
  if (D == 128)
    launch_by_heads<128>(prm, B, G, stream);
  else
    launch_by_heads<64>(prm, B, G, stream);
  if (hipGetLastError() != hipSuccess) return MQA_ERR_HIP;
  if (G > 0 || plan.num_parts > 1) {
    const int hpb = 256 / (D / 4);
    const dim3 grid((Hq + hpb - 1) / hpb, B);
    // A balanced plan over at least G / 2 sequences leaves each a few
    // partial states, which one slice merges in one round of loads (hybrid
    // block, 128 sequences: 116.9 vs 118.1 us per global-layer call with four
    // slices); fewer sequences may be cut into many pieces.
    const int slices = G > 0 ? (B >= G / 2 ? 1 : kMergeMaxSlices)
                             : std::min(kMergeMaxSlices, (plan.num_parts + 7) / 8);
    const dim3 block(256 * slices);
    if (D == 128)
      hipLaunchKernelGGL(decode_merge_kernel<128>, grid, block, 0, stream, prm.ws_o, prm.ws_ml, out, Hq,
                         plan.num_parts, prm.plan, (int)(ragged_plan_words((size_t)G, (size_t)B) - 2 * (size_t)B));
    else
      hipLaunchKernelGGL(decode_merge_kernel<64>, grid, block, 0, stream, prm.ws_o, prm.ws_ml, out, Hq,
                         plan.num_parts, prm.plan, (int)(ragged_plan_words((size_t)G, (size_t)B) - 2 * (size_t)B));
    if (hipGetLastError() != hipSuccess) return MQA_ERR_HIP;
  }
  return MQA_OK;
}

}  // namespace mqa
