// mqa_prefill_chunk: causal attention of a new chunk over a cached prefix,
// multi-query, int8 KV cache.
//
// What is computed: for sequence b with P = prefix_lens[b] cached tokens and
// a chunk of C new tokens (already appended to the int8 cache), the query of
// chunk token i sits at absolute position P + i and, for every head h,
//     out[b, i, h] = sum_j softmax_j(scale * s_k[j] * q.k_j) * s_v[j] * v_j
// over keys j in [max(0, P+i-W+1), P+i] (window W > 0) or [0, P+i].
// Sources: 9c1h.cn news page on Character.AI's inference tricks, sections
// 秘訣1 (MQA, sliding windows) and 秘訣2 (a cached prefix is reused, only the
// new turn is processed); explinks.com "Character.AI 的最佳实践", section
// 训练和服务的量化 (int8 KV); tubrief.io workshop transcript 00:20:54-00:22:12
// (prefill is the compute-bound phase) and 00:48:02-00:49:13 (tiles in fast
// on-chip memory with an online softmax).
//
// Design for gfx950 (prefill is a dense contraction, so it runs on MFMA):
//  * Heads are folded into rows: a sequence's chunk is a [C*Hq, D] query
//    matrix against ONE K/V head, so every K/V tile serves C*Hq rows (the
//    MQA reuse on the compute side).
//  * Stage pass: each 64-key tile a sequence needs is converted ONCE (instead
//    of once per work-group that reads it) into a workspace: K as bf16
//    [key][d]; V pre-multiplied by its row scale, V'' = fp16(v * s_v * 2^-E),
//    transposed [d][key] with the keys in the order the PV product consumes
//    them; both with 16-byte chunks XOR-swizzled so the MFMA operand reads
//    from LDS are free of bank conflicts; plus s_k * scale * log2(e) per key.
//    E is a per-sequence power of two with 2^E >= max s_v (a small first
//    pass, or for a window the stage work-groups themselves), which keeps
//    V'' in fp16's range; it is undone on the output.
//  * Attention pass: work-group = 8 waves x 32 rows, one per compute unit;
//    staged tiles stream global -> LDS with direct-to-LDS loads (no
//    registers) through four buffers, two tiles ahead of the one being
//    computed (with one tile ahead, the L2 round trip was exposed: 12% of the
//    kernel); each wave waits only for its own copies of the next tile. The
//    two waves of each SIMD run half a tile apart, and LDS operand reads are
//    issued one MFMA block ahead.
//    S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (q and K exact in bf16);
//    O^T += V''^T P^T on v_mfma_f32_16x16x32_f16 with P = 2^(z - m) in fp16
//    (relative rounding 2^-11 on V'' and on P, inside the prefill
//    tolerance), and the row sums l come from one more MFMA against an
//    all-ones block, so they use exactly the rounded P of the product.
//  * Softmax per element is one FMA (t = s * kscl - m_old), a max and an
//    exp: the running max is only moved when a tile exceeds it by more than
//    2^8 (rare path, which recomputes), so normally exp2(t) is the weight.
//  * Tiles outside every row's causal/window range are skipped, boundary
//    tiles are masked per element; work-groups of one sequence share an XCD.
#include <math.h>

#include <algorithm>

#include "common.h"
#include "launch.h"

namespace mqa {

namespace {

constexpr int kKeys = 64;        // keys per tile
constexpr int kRowsPerWave = 32;
constexpr int kWavesP = 8;
constexpr int kStages = 4;
constexpr int kRowsPerWG = kRowsPerWave * kWavesP;
constexpr float kLazyP = 8.0f;

// Staged tile: [K bf16 64 x D][V''^T fp16 D x 64][kscl 64 f32][pad to 1 KB]
// K row `key` keeps its 16-byte chunk c at c ^ (key & kSwzK): one MFMA
// operand read (16 keys x 4 chunks) then touches every LDS bank equally.
template <int D>
constexpr int kSwzK = D / 8 - 1;
template <int D>
struct StagedTile {
  static constexpr int kBytesK = kKeys * D * 2;
  static constexpr int kBytesV = kKeys * D * 2;
  static constexpr int kOffScl = kBytesK + kBytesV;
  static constexpr int kBytes = kOffScl + 1024;  // 256 B of scales + pad to 1 KB
};

struct PrefillParams {
  const uint16_t* q;
  const int8_t* k;
  const int8_t* v;
  const float* ks;
  const float* vs;
  const int32_t* prefix_lens;
  float* out;
  char* stage;          // [B][ntiles][StagedTile]
  float* seq_e;         // [B] exponent E of each sequence (as float)
  int32_t L_cap;         // contiguous: rows per sequence; paged: position bound
  // Paged layout (table != nullptr): k, v, ks, vs are block pools.
  const int32_t* table;
  int32_t table_len;
  int32_t log2_bs;
  int32_t num_blocks;
  int32_t C;
  int32_t Hq;
  int32_t window;
  int32_t ntiles;       // tiles per sequence in the workspace
  int32_t P_max;        // prefix lengths are clamped to [0, P_max] (workspace and cache bounds)
  int32_t row_tiles;    // attention work-groups per sequence
  int32_t inline_e;     // != 0: each stage work-group derives E itself (short visible ranges)
  float scale_log2;
};

// Physical row of key position j of sequence b.
__device__ __forceinline__ int64_t key_row(const PrefillParams& p, int b, int j) {
  if (p.table == nullptr) return (int64_t)b * p.L_cap + j;
  return paged_row(p.table, p.table_len, p.log2_bs, p.num_blocks, b, j);
}

__device__ __forceinline__ int clampP(int P, int P_max) {
  return P < 0 ? 0 : (P > P_max ? P_max : P);
}

__device__ __forceinline__ int first_needed_key(int P, int window) {
  return window > 0 ? max(0, P - window + 1) : 0;
}

// ---------------------------------------------------------------------------
// Exponent pass: grid (B), kExpThreads threads. E = smallest e with
// 2^e >= max s_v over the keys the chunk can see. Each thread keeps four
// loads in flight (one load per thread at a time left the pass bound by
// dozens of dependent memory round trips).
// ---------------------------------------------------------------------------
constexpr int kExpThreads = 1024;
constexpr int kExpUnroll = 4;
// Visible ranges up to this many keys get E from the stage pass itself.
constexpr int kInlineExpKeys = 4096;
__global__ __launch_bounds__(kExpThreads) void prefill_exponent_kernel(PrefillParams p) {
  const int b = blockIdx.x, tid = threadIdx.x;
  __shared__ float red[kExpThreads / kWave];
  const int P = clampP(__builtin_amdgcn_readfirstlane(p.prefix_lens[b]), p.P_max);
  const int lo = first_needed_key(P, p.window), hi = P + p.C;
  float m = 0.f;
  for (int j0 = lo + tid; j0 < hi; j0 += kExpUnroll * kExpThreads) {
    float v[kExpUnroll];
#pragma unroll
    for (int u = 0; u < kExpUnroll; ++u) {
      const int j = j0 + u * kExpThreads;
      v[u] = j < hi ? fabsf(p.vs[key_row(p, b, j)]) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kExpUnroll; ++u) m = fmaxf(m, v[u]);
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) m = fmaxf(m, __shfl_xor(m, s, kWave));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) {
    m = 0.f;
#pragma unroll
    for (int w = 0; w < kExpThreads / kWave; ++w) m = fmaxf(m, red[w]);
    int e = 0;
    if (m > 0.f && m < INFINITY) (void)frexpf(m, &e);
    p.seq_e[b] = (float)e;
  }
}

// Row of key j of sequence b, with the layout fixed at compile time.
template <bool PAGED>
__device__ __forceinline__ int64_t key_row_of(const PrefillParams& p, int b, int j) {
  if constexpr (!PAGED) return (int64_t)b * p.L_cap + j;
  else return paged_row(p.table, p.table_len, p.log2_bs, p.num_blocks, b, j);
}

// ---------------------------------------------------------------------------
// Stage pass: grid (tiles, B), 256 threads, one 64-key tile per work-group
// (a window: only the tiles its needed keys can span, from the first).
// Keys past the last one (kend) are read at row kend - 1 and zeroed after the
// load, so every load of a thread is issued before the first wait (loads
// under per-key conditions each waited for the previous one).
// ---------------------------------------------------------------------------
template <int D, bool PAGED>
__global__ __launch_bounds__(256) void prefill_stage_kernel(PrefillParams p) {
  const int b = blockIdx.y, tid = threadIdx.x;
  const int P = clampP(__builtin_amdgcn_readfirstlane(p.prefix_lens[b]), p.P_max);
  const int kend = P + p.C;                            // keys [0, kend) exist
  const int kbeg = first_needed_key(P, p.window);      // no query of the chunk sees a key before it
  const int t_lo = kbeg / kKeys;
  const int t_hi = (kend + kKeys - 1) / kKeys;
  // A window's grid covers only the tiles one window and the chunk can span,
  // counted from the sequence's first needed tile.
  const int t = p.window > 0 ? t_lo + (int)blockIdx.x : (int)blockIdx.x;
  if (t < t_lo || t >= t_hi) return;
  const int base = t * kKeys;
  char* tile = p.stage + ((int64_t)b * p.ntiles + t) * StagedTile<D>::kBytes;

  // E for the value scaling: from the exponent pass, or (a visible range of
  // at most kInlineExpKeys keys) the same maximum formed here by every
  // work-group of the sequence, the one of its first tile writing it for the
  // attention pass.
  float e_seq;
  if (p.inline_e) {
    __shared__ float red[256 / kWave];
    float m = 0.f;
    for (int j = kbeg + tid; j < kend; j += 256) m = fmaxf(m, fabsf(p.vs[key_row_of<PAGED>(p, b, j)]));
#pragma unroll
    for (int s_ = 32; s_ >= 1; s_ >>= 1) m = fmaxf(m, __shfl_xor(m, s_, kWave));
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    int e = 0;
    if (m > 0.f && m < INFINITY) (void)frexpf(m, &e);
    e_seq = (float)e;
    if (t == t_lo && tid == 0) p.seq_e[b] = e_seq;
  } else {
    e_seq = p.seq_e[b];
  }

  // K: thread = (key, quarter of the row); 16-byte chunk c of row `key` is
  // stored at chunk c ^ (key & kSwzK).
  {
    constexpr int QB = D / 4;   // bytes of the row per thread (32 or 16)
    const int key = tid >> 2, qtr = tid & 3;
    const int j = base + key;
    const bool ok = j < kend;
    const int64_t krow = key_row_of<PAGED>(p, b, ok ? j : kend - 1);
    u32x4 w[QB / 16];
#pragma unroll
    for (int u = 0; u < QB / 16; ++u) w[u] = *reinterpret_cast<const u32x4*>(p.k + krow * D + qtr * QB + 16 * u);
#pragma unroll
    for (int u = 0; u < QB / 16; ++u) w[u] = ok ? w[u] : u32x4{0u, 0u, 0u, 0u};
    uint16_t* row = reinterpret_cast<uint16_t*>(tile) + key * D;
#pragma unroll
    for (int u = 0; u < QB / 16; ++u)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int chunk = (qtr * QB) / 8 + 2 * u + h;   // 8 bf16 per chunk
        const u32x4 o = cat(i8x4_to_bf16(w[u][2 * h]), i8x4_to_bf16(w[u][2 * h + 1]));
        *reinterpret_cast<u32x4*>(row + 8 * (chunk ^ (key & kSwzK<D>))) = o;
      }
  }
  // V''^T: thread = (key group (ks, g), 4 columns). Chunk (ks, g) of row d
  // holds the 8 keys 32ks + 16(i/4) + 4g + i%4 (i = 0..7), stored at chunk
  // (4ks + g) ^ (d & 7) of the 64-key row; values fp16(v * s_v * 2^-E).
  // Keys outside [kbeg, kend) are stored as zero: the exponent E only bounds
  // the scales of the keys some query sees, so an unseen key's V'' could
  // overflow fp16, and its zero weight times infinity would be NaN.
  {
    constexpr int DQ = D / 4;   // 4-column groups
    const float rE = exp2f(-e_seq);
    for (int it = tid; it < 8 * DQ; it += 256) {
      const int grp = it / DQ, dq = it % DQ;
      const int ks = grp >> 2, g = grp & 3;
      uint32_t w[8];
      float f[8];
      int64_t row[8];
      bool ok[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = base + 32 * ks + 16 * (i >> 2) + 4 * g + (i & 3);
        ok[i] = j >= kbeg && j < kend;
        row[i] = key_row_of<PAGED>(p, b, j < kend ? j : kend - 1);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        w[i] = *reinterpret_cast<const uint32_t*>(p.v + row[i] * D + 4 * dq);
        f[i] = p.vs[row[i]];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        w[i] = ok[i] ? w[i] : 0u;
        f[i] = ok[i] ? f[i] * rE : 0.f;   // exact: a power-of-two rescale
      }
      uint16_t* vt = reinterpret_cast<uint16_t*>(tile + StagedTile<D>::kBytesK);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = 4 * dq + e;
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 8; i += 2)
          o[i >> 1] = cvt_pk_f16(i8_byte(w[i], e) * f[i], i8_byte(w[i + 1], e) * f[i + 1]);
        *reinterpret_cast<u32x4*>(vt + d * kKeys + 8 * ((4 * ks + g) ^ (d & 7))) = o;
      }
    }
  }
  // Per-key s_k * scale * log2(e).
  if (tid < kKeys) {
    const int j = base + tid;
    const float skr = p.ks[key_row_of<PAGED>(p, b, j < kend ? j : kend - 1)];
    const float sk = j < kend ? skr * p.scale_log2 : 0.f;
    reinterpret_cast<float*>(tile + StagedTile<D>::kOffScl)[tid] = sk;
  }
}

// One 64-key tile of one wave in three parts: S^T = K Q^T (tile_qk), the
// online softmax of one 16-row block (tile_softmax, once per block), and
// O^T += V''^T P^T (tile_pv). Split so that a wave can run the parts of
// consecutive tiles in a rotated order (see the attention pass).
// Scales s_k * scale * log2(e) of this lane's keys 16kb + 4g + r.
template <int D>
__device__ __forceinline__ void load_kscl(const char* tl, f32x4 (&kscl)[4], int g) {
  const float* scl = reinterpret_cast<const float*>(tl + StagedTile<D>::kOffScl);
#pragma unroll
  for (int kb4 = 0; kb4 < 4; ++kb4) kscl[kb4] = *reinterpret_cast<const f32x4*>(scl + 16 * kb4 + 4 * g);
}

// The K operand reads of each 16-key block are issued one block ahead of
// its MFMAs (scheduling barriers keep that order), so the LDS latency hides
// behind the previous block's MFMAs.
template <int D>
__device__ __forceinline__ void tile_qk(const char* tl, const bf16x8 (&qop)[2][D / 32], f32x4 (&s)[4][2], int g,
                                        int c) {
  constexpr int KK = D / 32;
  u32x4 kc[4][KK];
  const auto read = [&](int kb4) {
    const int key = 16 * kb4 + c;
    const uint16_t* krow = reinterpret_cast<const uint16_t*>(tl) + key * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int chunk = (4 * kk + g) ^ (key & kSwzK<D>);
      kc[kb4][kk] = *reinterpret_cast<const u32x4*>(krow + 8 * chunk);
    }
  };
  read(0);
#pragma unroll
  for (int kb4 = 0; kb4 < 4; ++kb4) {
    if (kb4 + 1 < 4) read(kb4 + 1);
    __builtin_amdgcn_sched_barrier(0);
    s[kb4][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    s[kb4][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const bf16x8 kop = as_bf16x8(kc[kb4][kk]);
      s[kb4][0] = mfma16(kop, qop[0][kk], s[kb4][0]);
      s[kb4][1] = mfma16(kop, qop[1][kk], s[kb4][1]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Online softmax of row block RT (rows 16RT + c of the wave) over one tile:
// t = s * kscl - m, weight 2^t as fp16 P (two 32-key halves), row sums by
// an MFMA against an all-ones block. `masked`: the tile straddles a row's
// causal or window limit. One body for both cases (a runtime branch that
// only rewrites the logits): with a separate masked copy, the joins of the
// two copies and their rare rescale paths cost ~24 register-pair moves of
// the accumulators per row block and tile on the common path.
template <int D, int RT>
__device__ __forceinline__ void tile_softmax(const char* tl, const f32x4 (&s)[4][2], f16x8 (&pop)[2][2],
                                             f32x4 (&oacc)[D / 16][2], f32x4 (&lacc)[2], float (&m_run)[2],
                                             const f16x8& ones, int base, const int (&row_lo)[2],
                                             const int (&row_pos)[2], int g, bool masked) {
  constexpr int MT = D / 16;
  f32x4 kscl[4];
  load_kscl<D>(tl, kscl, g);
  float tz[16];
#pragma unroll
  for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
    for (int r = 0; r < 4; ++r) tz[4 * kb4 + r] = fmaf(s[kb4][RT][r], kscl[kb4][r], -m_run[RT]);
  if (masked) {   // boundary tiles only (wave-uniform; only the logits change)
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = base + 16 * (i >> 2) + 4 * g + (i & 3);
      tz[i] = (j >= row_lo[RT] && j <= row_pos[RT]) ? tz[i] : -INFINITY;
    }
  }
  float tmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, tz[i]);
  tmax = quad_max(tmax);
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(tmax > kLazyP) != 0, 0)) {
    // Rare: move the running max to this tile's max and rescale.
    // (m_run = -inf makes every visible t = +inf; recompute from s.)
    float zmax = -INFINITY;
#pragma unroll
    for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * kb4 + r;
        const float z = s[kb4][RT][r] * kscl[kb4][r];
        tz[i] = (tz[i] == -INFINITY) ? -INFINITY : z;   // keep the mask
        zmax = fmaxf(zmax, tz[i]);
      }
    zmax = quad_max(zmax);
    const float m_new = fmaxf(m_run[RT], zmax);
    // rows of the wave may differ in position: a row with no visible key
    // yet keeps m = -inf and must not form 2^(-inf - -inf)
    const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run[RT] - m_new);
    m_run[RT] = m_new;
    lacc[RT] *= alpha;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) oacc[mt][RT] *= alpha;
    const float msub = (m_new == -INFINITY) ? 0.f : m_new;
#pragma unroll
    for (int i = 0; i < 16; ++i) tz[i] -= msub;
  }
#pragma unroll
  for (int ks2 = 0; ks2 < 2; ++ks2) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const int zi = 8 * ks2 + i;
      w[i >> 1] = cvt_pk_f16(fast_exp2(tz[zi]), fast_exp2(tz[zi + 1]));
    }
    pop[RT][ks2] = __builtin_bit_cast(f16x8, w);
    lacc[RT] = mfma16_f16(ones, pop[RT][ks2], lacc[RT]);
  }
}

// As in tile_qk, the V operand reads of each pair of 16-column blocks are
// issued one pair ahead of their MFMAs.
template <int D>
__device__ __forceinline__ void tile_pv(const char* tl, const f16x8 (&pop)[2][2], f32x4 (&oacc)[D / 16][2], int g,
                                        int c) {
  constexpr int MT = D / 16;
  const uint16_t* vt = reinterpret_cast<const uint16_t*>(tl + StagedTile<D>::kBytesK);
  u32x4 vc[MT][2];
  const auto read = [&](int mt) {
    const int d = 16 * mt + c;
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      const int chunk = (4 * ks2 + g) ^ (d & 7);
      vc[mt][ks2] = *reinterpret_cast<const u32x4*>(vt + d * kKeys + 8 * chunk);
    }
  };
  read(0);
  read(1);
#pragma unroll
  for (int mp = 0; mp < MT; mp += 2) {
    if (mp + 2 < MT) {
      read(mp + 2);
      read(mp + 3);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mt = mp; mt < mp + 2; ++mt)
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        const f16x8 vop = __builtin_bit_cast(f16x8, vc[mt][ks2]);
        oacc[mt][0] = mfma16_f16(vop, pop[0][ks2], oacc[mt][0]);
        oacc[mt][1] = mfma16_f16(vop, pop[1][ks2], oacc[mt][1]);
      }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---------------------------------------------------------------------------
// Attention pass.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64 * kWavesP) __attribute__((amdgpu_waves_per_eu(2))) void prefill_attn_kernel(
    PrefillParams p) {
  constexpr int TB = StagedTile<D>::kBytes;
  constexpr int NCH = TB / 1024;    // 1 KB copies per tile, spread over the waves
  constexpr int KK = D / 32;        // QK MFMAs along d
  constexpr int MT = D / 16;        // PV m-tiles
  // Four separate buffers (not one indexed array), named statically in an
  // unrolled loop, so the compiler can tell a buffer being read from the one
  // being filled and does not wait for the copy in flight.
  __shared__ __attribute__((aligned(16))) char lds0[TB];
  __shared__ __attribute__((aligned(16))) char lds1[TB];
  __shared__ __attribute__((aligned(16))) char lds2[TB];
  __shared__ __attribute__((aligned(16))) char lds3[TB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;
  const int c = lane & 15;
  // Work-group -> (sequence, row tile); consecutive work-groups are spread
  // over the 8 XCDs, so give each XCD whole sequences (shared K/V in its L2).
  const int nwg = gridDim.x;
  const int lin = blockIdx.x;
  const int B = nwg / p.row_tiles;
  int b, mtile;
  if ((B & 7) == 0) {
    const int flat = (lin & 7) * (nwg >> 3) + (lin >> 3);
    b = flat / p.row_tiles;
    mtile = flat % p.row_tiles;
  } else {
    b = lin / p.row_tiles;
    mtile = lin % p.row_tiles;
  }
  const int C = p.C, Hq = p.Hq;
  const int rows_total = C * Hq;
  const int P = clampP(__builtin_amdgcn_readfirstlane(p.prefix_lens[b]), p.P_max);

  const int wg_r0 = mtile * kRowsPerWG;
  const int wg_r1 = min(wg_r0 + kRowsPerWG, rows_total);
  const int w_r0 = wg_r0 + wave * kRowsPerWave;
  const int w_r1 = min(w_r0 + kRowsPerWave, rows_total);
  const bool wave_live = w_r0 < w_r1;
  auto key_lo = [&](int pos) { return p.window > 0 ? max(0, pos - p.window + 1) : 0; };
  const int wg_klo = key_lo(P + wg_r0 / Hq);
  const int wg_khi = P + (wg_r1 - 1) / Hq + 1;
  const int w_klo = wave_live ? key_lo(P + w_r0 / Hq) : 0;
  const int w_khi = wave_live ? P + (w_r1 - 1) / Hq + 1 : 0;
  const int t0 = wg_klo / kKeys;
  const int t1 = (wg_khi + kKeys - 1) / kKeys;
  const char* stage_b = p.stage + (int64_t)b * p.ntiles * TB;

  // Direct-to-LDS copy of staged tile t into buffer `buf`: 1 KB per
  // instruction per wave; the waves split the tile (wave w copies chunks
  // w, w + kWavesP, ...: kLoadsHi copies for the first NCH % kWavesP waves,
  // kLoadsLo for the others).
  constexpr int kLoadsLo = NCH / kWavesP;
  constexpr int kLoadsHi = kLoadsLo + (NCH % kWavesP != 0);
  const bool more_loads = wave < NCH % kWavesP;
  const __amdgpu_buffer_rsrc_t stage_r = make_rsrc(stage_b, (uint32_t)(p.ntiles * TB));
  auto issue_tile = [&](int t, char* dst) {
    const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)(t * TB));
#pragma unroll
    for (int i = 0; i < kLoadsHi; ++i) {
      const int ch = wave + i * kWavesP;
      if (i < kLoadsLo || more_loads)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(stage_r, dst + ch * 1024, 16, (uint32_t)(ch * 1024 + lane * 16),
                                                 soff, 0, 0);
    }
  };
  if (t0 < t1) issue_tile(t0, lds0);
  if (t0 + 1 < t1) issue_tile(t0 + 1, lds1);

  const float E = p.seq_e[b];   // output scale 2^E undoes the V'' shift

  // Rows held by this lane: 16*rt + c of the wave's 32; Q^T B operand.
  int row_pos[2], row_lo[2];
  bool row_ok[2];
  bf16x8 qop[2][KK];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int r = w_r0 + 16 * rt + c;
    row_ok[rt] = r < w_r1;
    const int rr = row_ok[rt] ? r : (wave_live ? w_r0 : 0);
    row_pos[rt] = P + rr / Hq;
    row_lo[rt] = key_lo(row_pos[rt]);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (row_ok[rt])
        w = *reinterpret_cast<const u32x4*>(p.q + ((int64_t)b * rows_total + r) * D + 32 * kk + 8 * g);
      qop[rt][kk] = as_bf16x8(w);
    }
  }

  f32x4 oacc[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    oacc[mt][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    oacc[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  f32x4 lacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};   // row sums (MFMA)
  float m_run[2] = {-INFINITY, -INFINITY};
  const f16x8 ones = __builtin_bit_cast(f16x8, u32x4{0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u});

  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Tile steps, each in two halves with a barrier after each: half 1 = issue
  // the copies of tile t + 2, QK and the softmax of row block 0; half 2 = the
  // softmax of row block 1 and PV. Waves 4-7 (one per SIMD beside waves 0-3)
  // pass one extra barrier first and so run half a step behind: while one
  // wave of a SIMD issues MFMAs the other runs its softmax on the vector
  // ALUs. Between two barriers the waves read tiles t - 1 and t (tile t from
  // the first barrier before its QK to the third after), so tile t + 2 goes
  // into the buffer of tile t - 2, of four. Before each barrier a wave waits
  // for its own copies of tile t + 1, which the half-step-late waves need
  // landed one barrier earlier than the others do.
  const bool late = wave >= kWavesP / 2;
  if (late && t0 < t1) __syncthreads();
  const auto wait_next = [&](int t) {
    if (t + 2 < t1) {   // only tile t+2's copies may still be in flight
      if (more_loads)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoadsHi));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoadsLo));
    } else {
      __builtin_amdgcn_s_waitcnt(0);
    }
  };
  f32x4 s[4][2];
  f16x8 pop[2][2];
  const auto step = [&](int t, const char* tl, char* fill) {
    if (t + 2 < t1) issue_tile(t + 2, fill);
    const int base = t * kKeys;
    const bool live = wave_live && base < w_khi && base + kKeys > w_klo;
    const bool masked = (base < w_klo) || (base + kKeys > P + w_r0 / Hq + 1) ||
                        (p.window > 0 && base < key_lo(P + (w_r1 - 1) / Hq));
    if (live) {
      tile_qk<D>(tl, qop, s, g, c);
      tile_softmax<D, 0>(tl, s, pop, oacc, lacc, m_run, ones, base, row_lo, row_pos, g, masked);
    }
    wait_next(t);
    __syncthreads();
    if (live) {
      tile_softmax<D, 1>(tl, s, pop, oacc, lacc, m_run, ones, base, row_lo, row_pos, g, masked);
      tile_pv<D>(tl, pop, oacc, g, c);
    }
    if (!(late && t + 1 == t1)) {   // the late waves passed their extra barrier first
      wait_next(t);
      __syncthreads();
    }
  };
  for (int t = t0; t < t1; t += kStages) {
    step(t, lds0, lds2);
    if (t + 1 >= t1) break;
    step(t + 1, lds1, lds3);
    if (t + 2 >= t1) break;
    step(t + 2, lds2, lds0);
    if (t + 3 >= t1) break;
    step(t + 3, lds3, lds1);
  }

  // ---- normalise and write: lane holds out[row 16rt + c][16mt + 4g + 0..3] ----
  const float oscale = exp2f(E);
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const float l = lacc[rt][0];   // every row of the all-ones block holds the sum
    if (!row_ok[rt]) continue;
    const float inv = l > 0.f ? oscale / l : 0.f;
    const int r = w_r0 + 16 * rt + c;
    float* dst = p.out + ((int64_t)b * rows_total + r) * D + 4 * g;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) *reinterpret_cast<f32x4*>(dst + 16 * mt) = oacc[mt][rt] * inv;
  }
}

}  // namespace

size_t prefill_workspace_bytes(int32_t B, int32_t C, int32_t D, int32_t max_prefix_len) {
  const int64_t ntiles = ((int64_t)max_prefix_len + C + kKeys - 1) / kKeys;
  const size_t tb = (D == 128) ? StagedTile<128>::kBytes : StagedTile<64>::kBytes;
  const size_t stage = (size_t)B * ntiles * tb;
  const size_t expo = ((size_t)B * sizeof(float) + 255) / 256 * 256;
  return stage + expo;
}

int launch_prefill(const uint16_t* q, const mqa_kv_view& kv, const KVLayout& layout, const int32_t* prefix_lens,
                   int32_t max_prefix_len, int32_t B, int32_t C, int32_t Hq, int32_t D,
                   int32_t window, float softmax_scale, float* out, void* workspace,
                   hipStream_t stream) {
  PrefillParams prm;
  prm.q = q;
  prm.k = kv.k;
  prm.v = kv.v;
  prm.ks = kv.k_scale;
  prm.vs = kv.v_scale;
  prm.prefix_lens = prefix_lens;
  prm.out = out;
  prm.L_cap = layout.table ? layout.L_cap : kv.L_cap;
  prm.table = layout.table;
  prm.table_len = layout.table_len;
  prm.log2_bs = layout.log2_bs;
  prm.num_blocks = layout.num_blocks;
  prm.C = C;
  prm.Hq = Hq;
  prm.window = window;
  prm.scale_log2 = softmax_scale * 1.4426950408889634f;
  prm.ntiles = (int)(((int64_t)max_prefix_len + C + kKeys - 1) / kKeys);
  // A prefix longer than max_prefix_len would reach past this sequence's
  // staged tiles; one past the cache capacity past the cache.
  prm.P_max = (int)((int64_t)max_prefix_len < (int64_t)prm.L_cap - C ? max_prefix_len : prm.L_cap - C);
  const size_t tb = (D == 128) ? StagedTile<128>::kBytes : StagedTile<64>::kBytes;
  // the attention pass addresses a sequence's staged tiles with 32-bit signed offsets
  if ((int64_t)prm.ntiles * (int64_t)tb > (int64_t)0x7fffffff) return MQA_ERR_SHAPE;
  prm.stage = static_cast<char*>(workspace);
  prm.seq_e = reinterpret_cast<float*>(prm.stage + (size_t)B * prm.ntiles * tb);
  const int64_t rows = (int64_t)C * Hq;
  prm.row_tiles = (int)((rows + kRowsPerWG - 1) / kRowsPerWG);
  const int64_t grid = (int64_t)prm.row_tiles * B;
  if (grid > 0x7fffffff) return MQA_ERR_SHAPE;
  // a window's needed keys [P - W + 1, P + C) span at most this many tiles
  const int64_t win_tiles = window > 0 ? ((int64_t)window - 1 + C + kKeys - 1) / kKeys + 1 : prm.ntiles;
  const dim3 sgrid((unsigned)std::min<int64_t>(prm.ntiles, win_tiles), B);
  // A short visible range (a window) is scanned by the stage work-groups
  // themselves: one kernel launch less.
  prm.inline_e = (window > 0 && (int64_t)window + C <= kInlineExpKeys) ? 1 : 0;
  if (!prm.inline_e) hipLaunchKernelGGL(prefill_exponent_kernel, dim3(B), dim3(kExpThreads), 0, stream, prm);
  if (D == 128) {
    if (prm.table)
      hipLaunchKernelGGL((prefill_stage_kernel<128, true>), sgrid, dim3(256), 0, stream, prm);
    else
      hipLaunchKernelGGL((prefill_stage_kernel<128, false>), sgrid, dim3(256), 0, stream, prm);
    hipLaunchKernelGGL(prefill_attn_kernel<128>, dim3((unsigned)grid), dim3(64 * kWavesP), 0, stream, prm);
  } else {
    if (prm.table)
      hipLaunchKernelGGL((prefill_stage_kernel<64, true>), sgrid, dim3(256), 0, stream, prm);
    else
      hipLaunchKernelGGL((prefill_stage_kernel<64, false>), sgrid, dim3(256), 0, stream, prm);
    hipLaunchKernelGGL(prefill_attn_kernel<64>, dim3((unsigned)grid), dim3(64 * kWavesP), 0, stream, prm);
  }
  return hipGetLastError() == hipSuccess ? MQA_OK : MQA_ERR_HIP;
}

}  // namespace mqa
