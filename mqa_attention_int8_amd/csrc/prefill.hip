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
//    matrix against ONE K/V head, so every K/V tile staged in LDS serves
//    C*Hq rows (the MQA reuse on the compute side).
//  * Work-group = 4 waves = 128 consecutive rows; a wave owns 32 rows.
//  * Per 64-key tile: the work-group converts the int8 K rows to bf16 into
//    LDS ([key][d], padded rows), and the int8 V rows to bf16 TRANSPOSED
//    ([d][key]) so that both MFMA operands are contiguous LDS reads; the
//    per-key scales go to LDS as well (s_k pre-multiplied by scale*log2 e).
//  * S^T = K Q^T and O^T += V^T P'^T on v_mfma_f32_16x16x32_bf16 with fp32
//    accumulation; P' = p * s_v is split into bf16 hi + lo parts: one bf16
//    rounding (2^-9 relative) is too coarse when a short window averages a
//    few nearly cancelling values.
//  * Tiles outside every row's causal/window range are skipped for the whole
//    work-group; a wave skips tiles outside its own rows' range; only the
//    boundary tiles apply the per-element mask.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace mqa {

namespace {

constexpr int kKeys = 64;       // keys per LDS tile
constexpr int kRowsPerWave = 32;
constexpr int kWavesP = 4;
constexpr int kRowsPerWG = kRowsPerWave * kWavesP;

struct PrefillParams {
  const uint16_t* q;
  const int8_t* k;
  const int8_t* v;
  const float* ks;
  const float* vs;
  const int32_t* prefix_lens;
  float* out;
  int32_t L_cap;
  int32_t C;
  int32_t Hq;
  int32_t window;
  int32_t row_tiles;  // work-groups per sequence
  float scale_log2;
};

template <int D>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillParams p) {
  constexpr int KSTR = D + 8;       // bf16 elements per K row in LDS
  constexpr int VSTR = kKeys + 8;   // bf16 elements per V^T row in LDS
  constexpr int KK = D / 32;        // MFMAs along d
  constexpr int MT = D / 16;        // PV m-tiles (16 output columns each)
  __shared__ __attribute__((aligned(16))) uint16_t sK[kKeys * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[D * VSTR];
  __shared__ float sKs[kKeys];
  __shared__ float sVs[kKeys];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int c = lane & 15;
  // Work-group -> (sequence, row tile). Consecutive work-groups land on
  // different XCDs (round-robin dispatch), so map the XCD index to the
  // sequence to keep one sequence's K/V in one L2.
  const int nwg = gridDim.x;
  const int lin = blockIdx.x;
  const int B = nwg / p.row_tiles;
  int b, mtile;
  {
    const int xcd = lin & 7;
    const int slot = lin >> 3;
    const int per_xcd = nwg >> 3;  // nwg is a multiple of 8 when B % 8 == 0
    if ((B & 7) == 0) {
      const int flat = xcd * per_xcd + slot;
      b = flat / p.row_tiles;
      mtile = flat % p.row_tiles;
    } else {
      b = lin / p.row_tiles;
      mtile = lin % p.row_tiles;
    }
  }
  const int C = p.C, Hq = p.Hq;
  const int rows_total = C * Hq;
  int P = p.prefix_lens[b];
  // keep every access inside the cache even for out-of-range lengths
  P = P < 0 ? 0 : (P > p.L_cap - C ? p.L_cap - C : P);

  const int wg_r0 = mtile * kRowsPerWG;
  const int wg_r1 = min(wg_r0 + kRowsPerWG, rows_total);
  const int w_r0 = wg_r0 + wave * kRowsPerWave;
  const int w_r1 = min(w_r0 + kRowsPerWave, rows_total);
  const bool wave_live = w_r0 < w_r1;

  auto key_lo = [&](int pos) { return p.window > 0 ? max(0, pos - p.window + 1) : 0; };
  // work-group key range
  const int wg_klo = key_lo(P + wg_r0 / Hq);
  const int wg_khi = P + (wg_r1 - 1) / Hq + 1;
  // wave key range
  const int w_klo = wave_live ? key_lo(P + w_r0 / Hq) : 0;
  const int w_khi = wave_live ? P + (w_r1 - 1) / Hq + 1 : 0;

  // rows held by this lane: 16*rt + c of the wave's 32
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
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};

  const int8_t* kb = p.k + (int64_t)b * p.L_cap * D;
  const int8_t* vb = p.v + (int64_t)b * p.L_cap * D;
  const float* ksb = p.ks + (int64_t)b * p.L_cap;
  const float* vsb = p.vs + (int64_t)b * p.L_cap;
  const int klast = wg_khi - 1;

  const int t0 = wg_klo / kKeys;
  const int t1 = (wg_khi + kKeys - 1) / kKeys;
  for (int t = t0; t < t1; ++t) {
    const int base = t * kKeys;
    __syncthreads();  // previous tile fully consumed
    // ---- stage K (bf16, [key][d]) ----
    constexpr int KSEG = D / 16;                  // 16-byte segments per row
    for (int it = tid; it < kKeys * KSEG; it += 256) {
      const int key = it / KSEG, seg = it % KSEG;
      const int j = min(base + key, klast);
      const u32x4 x = *reinterpret_cast<const u32x4*>(kb + (int64_t)j * D + 16 * seg);
      const u32x4 a = cat(i8x4_to_bf16(x[0]), i8x4_to_bf16(x[1]));
      const u32x4 bb = cat(i8x4_to_bf16(x[2]), i8x4_to_bf16(x[3]));
      u32x4* dst = reinterpret_cast<u32x4*>(&sK[key * KSTR + 16 * seg]);
      dst[0] = a;
      dst[1] = bb;
    }
    // ---- stage V transposed (bf16, [d][key]) ----
    constexpr int DQD = D / 4;                    // 4-column groups
    for (int it = tid; it < (kKeys / 4) * DQD; it += 256) {
      const int kq = it / DQD, dq = it % DQD;
      uint32_t w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = min(base + 4 * kq + u, klast);
        w[u] = *reinterpret_cast<const uint32_t*>(vb + (int64_t)j * D + 4 * dq);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        u32x2 o;
        o[0] = pack_hi16(i8_byte(w[0], e), i8_byte(w[1], e));
        o[1] = pack_hi16(i8_byte(w[2], e), i8_byte(w[3], e));
        *reinterpret_cast<u32x2*>(&sVt[(4 * dq + e) * VSTR + 4 * kq]) = o;
      }
    }
    if (tid < kKeys) {
      const int j = base + tid;
      const bool ok = j >= wg_klo && j < wg_khi;
      sKs[tid] = ok ? ksb[j] * p.scale_log2 : 0.f;
      sVs[tid] = ok ? vsb[j] : 0.f;
    }
    __syncthreads();

    if (!wave_live || base >= w_khi || base + kKeys <= w_klo) continue;
    const bool need_mask = (base < w_klo) || (base + kKeys > P + w_r0 / Hq + 1) ||
                           (p.window > 0 && base < key_lo(P + (w_r1 - 1) / Hq));

    // ---- S^T = K Q^T : 4 key blocks x 2 row blocks ----
    f32x4 s[4][2];
#pragma unroll
    for (int kb4 = 0; kb4 < 4; ++kb4) {
      s[kb4][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      s[kb4][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const bf16x8 kop =
            as_bf16x8(*reinterpret_cast<const u32x4*>(&sK[(16 * kb4 + c) * KSTR + 32 * kk + 8 * g]));
        s[kb4][0] = mfma16(kop, qop[0][kk], s[kb4][0]);
        s[kb4][1] = mfma16(kop, qop[1][kk], s[kb4][1]);
      }
    }

    // ---- online softmax per row ----
    bf16x8 phi[2][2], plo[2][2];  // [row block][32-key step], P' = hi + lo
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      float z[16];
      float tmax = -INFINITY;
#pragma unroll
      for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = 16 * kb4 + 4 * g + r;
          float zz = s[kb4][rt][r] * sKs[key];
          if (need_mask) {
            const int j = base + key;
            zz = (j >= row_lo[rt] && j <= row_pos[rt]) ? zz : -INFINITY;
          }
          z[4 * kb4 + r] = zz;
          tmax = fmaxf(tmax, zz);
        }
      tmax = wave_max_xor(tmax, 16);
      tmax = wave_max_xor(tmax, 32);
      const float m_new = fmaxf(m_run[rt], tmax);
      if (__builtin_amdgcn_ballot_w64(m_new > m_run[rt]) != 0) {
        const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_run[rt] - m_new);
        l_run[rt] *= alpha;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) oacc[mt][rt] *= alpha;
      }
      m_run[rt] = m_new;
      const float msub = (m_new == -INFINITY) ? 0.f : m_new;
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        u32x4 wh, wl;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {       // key block 2*ks2 + hh
#pragma unroll
          for (int r = 0; r < 4; r += 2) {
            const int zi = 4 * (2 * ks2 + hh) + r;
            const float e0 = exp2f(z[zi] - msub);
            const float e1 = exp2f(z[zi + 1] - msub);
            l_run[rt] += e0 + e1;
            const int key = 16 * (2 * ks2 + hh) + 4 * g + r;
            const float p0 = e0 * sVs[key], p1 = e1 * sVs[key + 1];
            const uint32_t h01 = cvt_pk_bf16(p0, p1);
            wh[2 * hh + (r >> 1)] = h01;
            wl[2 * hh + (r >> 1)] = cvt_pk_bf16(p0 - bf16_lo_to_f32(h01), p1 - bf16_hi_to_f32(h01));
          }
        }
        phi[rt][ks2] = as_bf16x8(wh);
        plo[rt][ks2] = as_bf16x8(wl);
      }
    }

    // ---- O^T += V^T P'^T ----
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        const uint16_t* row = &sVt[(16 * mt + c) * VSTR + 32 * ks2 + 4 * g];
        const u32x2 lo2 = *reinterpret_cast<const u32x2*>(row);
        const u32x2 hi2 = *reinterpret_cast<const u32x2*>(row + 16);
        const u32x4 a = {lo2[0], lo2[1], hi2[0], hi2[1]};
        const bf16x8 vop = as_bf16x8(a);
        oacc[mt][0] = mfma16(vop, phi[0][ks2], oacc[mt][0]);
        oacc[mt][0] = mfma16(vop, plo[0][ks2], oacc[mt][0]);
        oacc[mt][1] = mfma16(vop, phi[1][ks2], oacc[mt][1]);
        oacc[mt][1] = mfma16(vop, plo[1][ks2], oacc[mt][1]);
      }
    }
  }

  // ---- normalise and write: lane holds out[row 16rt + c][16mt + 4g + 0..3] ----
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    float l = l_run[rt];
    l += __shfl_xor(l, 16, kWave);
    l += __shfl_xor(l, 32, kWave);
    if (!row_ok[rt]) continue;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int r = w_r0 + 16 * rt + c;
    float* dst = p.out + ((int64_t)b * rows_total + r) * D + 4 * g;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const f32x4 o = oacc[mt][rt] * inv;
      *reinterpret_cast<f32x4*>(dst + 16 * mt) = o;
    }
  }
}

}  // namespace

int launch_prefill(const uint16_t* q, const mqa_kv_view& kv, const int32_t* prefix_lens,
                   int32_t max_prefix_len, int32_t B, int32_t C, int32_t Hq, int32_t D,
                   int32_t window, float softmax_scale, float* out, hipStream_t stream) {
  (void)max_prefix_len;
  PrefillParams prm;
  prm.q = q;
  prm.k = kv.k;
  prm.v = kv.v;
  prm.ks = kv.k_scale;
  prm.vs = kv.v_scale;
  prm.prefix_lens = prefix_lens;
  prm.out = out;
  prm.L_cap = kv.L_cap;
  prm.C = C;
  prm.Hq = Hq;
  prm.window = window;
  prm.scale_log2 = softmax_scale * 1.4426950408889634f;
  const int64_t rows = (int64_t)C * Hq;
  prm.row_tiles = (int)((rows + kRowsPerWG - 1) / kRowsPerWG);
  const int64_t grid = (int64_t)prm.row_tiles * B;
  if (grid > 0x7fffffff) return MQA_ERR_SHAPE;
  if (D == 128)
    hipLaunchKernelGGL(prefill_kernel<128>, dim3((unsigned)grid), dim3(256), 0, stream, prm);
  else
    hipLaunchKernelGGL(prefill_kernel<64>, dim3((unsigned)grid), dim3(256), 0, stream, prm);
  return hipGetLastError() == hipSuccess ? MQA_OK : MQA_ERR_HIP;
}

}  // namespace mqa
