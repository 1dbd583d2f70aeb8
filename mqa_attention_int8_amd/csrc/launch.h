// Internal launchers of libmqa_int8 (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/mqa_int8.h"

namespace mqa {

// Sequence-partition plan of one decode call (host side, pure function).
struct DecodePlan {
  int tiles_per_part;  // 32-key tiles per work-group
  int num_parts;       // work-groups per sequence
  size_t ws_bytes;     // workspace for partial states (0 when num_parts == 1)
};
DecodePlan plan_decode(int32_t B, int32_t Hq, int32_t D, int32_t max_seq_len, int32_t window,
                       int num_cus);

int launch_quantize(const float* src, int8_t* dst, float* dst_scale, const int32_t* start_pos,
                    int32_t B, int32_t T, int32_t D, int32_t L_cap, hipStream_t stream);

// Fused append of one new token per sequence (writable view of the cache the
// attention reads, and the new fp32 rows).
struct AppendRows {
  const float* k_new;
  const float* v_new;
  int8_t* k;
  int8_t* v;
  float* k_scale;
  float* v_scale;
};

int launch_decode(const uint16_t* q, const mqa_kv_view& kv, const int32_t* seq_lens, int32_t B,
                  int32_t Hq, int32_t D, int32_t window, float softmax_scale, float* out,
                  void* workspace, const DecodePlan& plan, hipStream_t stream,
                  const AppendRows* append = nullptr);

size_t prefill_workspace_bytes(int32_t B, int32_t C, int32_t D, int32_t max_prefix_len);

int launch_prefill(const uint16_t* q, const mqa_kv_view& kv, const int32_t* prefix_lens,
                   int32_t max_prefix_len, int32_t B, int32_t C, int32_t Hq, int32_t D,
                   int32_t window, float softmax_scale, float* out, void* workspace,
                   hipStream_t stream);

}  // namespace mqa
