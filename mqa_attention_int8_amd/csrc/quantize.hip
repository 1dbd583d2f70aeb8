// kv_quantize_int8: per-token-row absmax/127 int8 encoding of new K or V rows.
//
// The int8 KV cache follows explinks.com "Character.AI 的最佳实践", section
// 训练和服务的量化. The scheme (the pages leave it open): scale
// s = fl32(absmax/127); a row whose scale is 0 is stored as zeros; otherwise
// code = clamp(rint(fl32(x/s)), -127, 127). Both divisions are IEEE
// correctly rounded fp32 divisions (hipcc's default for '/', denormals kept)
// and rintf rounds half to even, so the result is bit-exact and
// reproducible on any IEEE machine.
//
// Launch: one group of D/4 lanes per row; each lane owns four consecutive
// elements (one 16-byte load, one 4-byte store), the group reduces absmax
// with xor-shuffles. Rows are independent; this is a tiny, HBM-bound kernel.
#include "common.h"
#include "launch.h"

namespace mqa {

// Encoding of one row by a group of D/4 lanes: lane_in_row holds elements
// [4*lane_in_row, 4*lane_in_row + 4); returns the four codes packed and the
// row scale (the same in every lane of the group).
template <int D>
__device__ __forceinline__ uint32_t encode_row_part(const float4 x, float& s) {
  constexpr int LPR = D / 4;
  float a = fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w)));
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) a = fmaxf(a, __shfl_xor(a, m, kWave));
  s = kv_row_scale(a);
  uint32_t packed = 0;
  const float v[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) packed |= ((uint32_t)kv_code(v[i], s) & 0xffu) << (8 * i);
  return packed;
}

template <int D>
__global__ __launch_bounds__(256) void quantize_rows_kernel(
    const float* __restrict__ src, int8_t* __restrict__ dst, float* __restrict__ dst_scale,
    const int32_t* __restrict__ start_pos, int32_t B, int32_t T, int32_t L_cap) {
  constexpr int LPR = D / 4;             // lanes per row (16 or 32)
  constexpr int RPB = 256 / LPR;         // rows per block
  const int lane_in_row = threadIdx.x % LPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const bool live = row < (int64_t)B * T;
  const int64_t r = live ? row : 0;
  const int b = (int)(r / T);
  const int t = (int)(r % T);

  const float4 x = *reinterpret_cast<const float4*>(src + r * D + 4 * lane_in_row);
  float s;
  const uint32_t packed = encode_row_part<D>(x, s);
  if (!live) return;
  const int64_t pos = (int64_t)start_pos[b] + t;
  if (pos < 0 || pos >= L_cap) return;
  const int64_t drow = (int64_t)b * L_cap + pos;
  *reinterpret_cast<uint32_t*>(dst + drow * D + 4 * lane_in_row) = packed;
  if (lane_in_row == 0) dst_scale[drow] = s;
}

// Paged buffer: grid.y selects K (0) or V (1); position start_pos[b] + t of
// sequence b goes to its physical row through the block table. Negative
// positions are skipped.
template <int D>
__global__ __launch_bounds__(256) void quantize_rows_paged_kernel(
    const float* __restrict__ k_src, const float* __restrict__ v_src, int8_t* __restrict__ k,
    int8_t* __restrict__ v, float* __restrict__ k_scale, float* __restrict__ v_scale, const int32_t* table,
    int32_t table_len, int32_t log2_bs, int32_t num_blocks, const int32_t* __restrict__ start_pos, int32_t B,
    int32_t T) {
  constexpr int LPR = D / 4;
  constexpr int RPB = 256 / LPR;
  const bool is_v = blockIdx.y == 1;
  const float* src = is_v ? v_src : k_src;
  int8_t* dst = is_v ? v : k;
  float* dst_scale = is_v ? v_scale : k_scale;
  const int lane_in_row = threadIdx.x % LPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const bool live = row < (int64_t)B * T;
  const int64_t r = live ? row : 0;
  const int b = (int)(r / T);
  const int t = (int)(r % T);
  const float4 x = *reinterpret_cast<const float4*>(src + r * D + 4 * lane_in_row);
  float s;
  const uint32_t packed = encode_row_part<D>(x, s);
  if (!live) return;
  const int64_t pos = (int64_t)start_pos[b] + t;
  if (pos < 0 || pos >= kPagedPositionLimit) return;
  const int64_t drow = paged_row(table, table_len, log2_bs, num_blocks, b, (int)pos);
  *reinterpret_cast<uint32_t*>(dst + drow * D + 4 * lane_in_row) = packed;
  if (lane_in_row == 0) dst_scale[drow] = s;
}

int launch_quantize_paged(const float* k_src, const float* v_src, int8_t* k, int8_t* v, float* k_scale,
                          float* v_scale, const KVLayout& layout, const int32_t* start_pos, int32_t B,
                          int32_t T, int32_t D, hipStream_t stream) {
  const int64_t rows = (int64_t)B * T;
  const int rpb = 256 / (D / 4);
  const int64_t grid = (rows + rpb - 1) / rpb;
  if (grid > 0x7fffffff) return MQA_ERR_SHAPE;
  const dim3 g((unsigned)grid, 2);
  if (D == 128)
    hipLaunchKernelGGL(quantize_rows_paged_kernel<128>, g, dim3(256), 0, stream, k_src, v_src, k, v, k_scale,
                       v_scale, layout.table, layout.table_len, layout.log2_bs, layout.num_blocks, start_pos, B, T);
  else
    hipLaunchKernelGGL(quantize_rows_paged_kernel<64>, g, dim3(256), 0, stream, k_src, v_src, k, v, k_scale,
                       v_scale, layout.table, layout.table_len, layout.log2_bs, layout.num_blocks, start_pos, B, T);
  return hipGetLastError() == hipSuccess ? MQA_OK : MQA_ERR_HIP;
}

int launch_quantize(const float* src, int8_t* dst, float* dst_scale, const int32_t* start_pos,
                    int32_t B, int32_t T, int32_t D, int32_t L_cap, hipStream_t stream) {
  const int64_t rows = (int64_t)B * T;
  const int rpb = 256 / (D / 4);
  const int64_t grid = (rows + rpb - 1) / rpb;
  if (grid > 0x7fffffff) return MQA_ERR_SHAPE;
  if (D == 128)
    hipLaunchKernelGGL(quantize_rows_kernel<128>, dim3((unsigned)grid), dim3(256), 0, stream,
                       src, dst, dst_scale, start_pos, B, T, L_cap);
  else
    hipLaunchKernelGGL(quantize_rows_kernel<64>, dim3((unsigned)grid), dim3(256), 0, stream,
                       src, dst, dst_scale, start_pos, B, T, L_cap);
  return hipGetLastError() == hipSuccess ? MQA_OK : MQA_ERR_HIP;
}

}  // namespace mqa
