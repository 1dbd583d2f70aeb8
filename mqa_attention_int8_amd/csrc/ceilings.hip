// Ceiling kernels for the measurements that the attention kernels are held
// against: how fast this GPU streams a buffer from HBM in one pass, and how
// many bf16 matrix-core flops it sustains. Not part of the attention
// library (libmqa_int8.so); built as libmqa_ceilings.so for the benchmark.
//
//  * Streaming read: work-groups sweep the buffer in contiguous 16 KB chunks
//    with 16-byte non-temporal loads, four in flight per lane (faster here
//    than a sweep whose four loads per lane lie a whole grid apart). Each
//    work-group writes the 32-bit wrapping sum
//    of the words it read, so the caller can check that every byte was read
//    exactly once.
//  * Matrix loop: every wave runs eight independent accumulator chains of
//    v_mfma_f32_16x16x32_bf16 (16 x 16 x 32 multiply-adds each), enough
//    independent work to keep the unit issuing; the sums go to a sink so the
//    loop cannot be removed.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"
#include "mqa_ceilings.h"

namespace mqa {
namespace {

constexpr int kStreamThreads = 256;
constexpr int kMfmaThreads = 512;  // 8 waves: two per SIMD
constexpr int kMfmaChains = 8;

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                                     uint32_t* __restrict__ partial) {
  // 16 KB chunks: a work-group reads chunk blockIdx.x, then every gridDim.x-th
  // one; lane t reads its words t, t + 256, t + 512, t + 768 of the chunk
  constexpr size_t kChunk = 4 * kStreamThreads;
  const size_t stride = (size_t)gridDim.x * kChunk;
  size_t i = (size_t)blockIdx.x * kChunk + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * kStreamThreads < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + kStreamThreads);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * kStreamThreads);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * kStreamThreads);
    acc += (a.x + a.y + a.z + a.w) + (b.x + b.y + b.z + b.w) + (c.x + c.y + c.z + c.w) + (d.x + d.y + d.z + d.w);
  }
  // the chunk that holds the end of the buffer (later chunks start past it)
  for (int u = 0; u < 4; ++u) {
    if (i + u * kStreamThreads < n16) {
      const u32x4 a = __builtin_nontemporal_load(src + i + u * kStreamThreads);
      acc += a.x + a.y + a.z + a.w;
    }
  }
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  __shared__ uint32_t red[kStreamThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t s = 0;
    for (int w = 0; w < kStreamThreads / 64; ++w) s += red[w];
    partial[blockIdx.x] = s;
  }
}

__global__ __launch_bounds__(kMfmaThreads) void mfma_loop_kernel(int iters, float* __restrict__ sink) {
  // operands depend on the lane so nothing folds; small values keep the sums finite
  u32x4 wa, wb;
  for (int e = 0; e < 4; ++e) {
    const uint32_t v = (uint32_t)((threadIdx.x + 3 * e) & 7);
    wa[e] = 0x3c003c00u + (v << 16) + v;  // bf16 bit patterns near 2^-7
    wb[e] = 0x3c803c80u - (v << 16) - v;
  }
  const bf16x8 a = as_bf16x8(wa), b = as_bf16x8(wb);
  f32x4 acc[kMfmaChains];
  for (int k = 0; k < kMfmaChains; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < kMfmaChains; ++k) acc[k] = mfma16(a, b, acc[k]);
  }
  float s = 0.f;
  for (int k = 0; k < kMfmaChains; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
  sink[(size_t)blockIdx.x * kMfmaThreads + threadIdx.x] = s;
}

}  // namespace
}  // namespace mqa

extern "C" {

int mqa_ceiling_stream_read(const void* src, size_t bytes, int32_t blocks, uint32_t* partial, void* stream) {
  if (!src || !partial) return 1;
  if (bytes == 0 || (bytes & 15) || ((uintptr_t)src & 15) || blocks <= 0) return 2;
  hipLaunchKernelGGL(mqa::stream_read_kernel, dim3(blocks), dim3(mqa::kStreamThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const mqa::u32x4*>(src), bytes / 16, partial);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

int mqa_ceiling_mfma_bf16(int32_t blocks, int32_t iters, float* sink, void* stream) {
  if (!sink) return 1;
  if (blocks <= 0 || iters <= 0) return 2;
  hipLaunchKernelGGL(mqa::mfma_loop_kernel, dim3(blocks), dim3(mqa::kMfmaThreads), 0, static_cast<hipStream_t>(stream), iters,
                     sink);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

double mqa_ceiling_mfma_bf16_flops(int32_t blocks, int32_t iters) {
  return (double)blocks * (mqa::kMfmaThreads / 64) * (double)iters * mqa::kMfmaChains * (16.0 * 16.0 * 32.0 * 2.0);
}

}  // extern "C"
