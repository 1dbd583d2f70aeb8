// Internal launchers of libmqa_int8 (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/mqa_int8.h"

namespace mqa {

// Where the token rows of a KV buffer live. Contiguous (table == nullptr):
// row b * L_cap + t. Paged: row table[b][(t >> log2_bs) % table_len] <<
// log2_bs | (t mod 2^log2_bs), with entries clamped into [0, num_blocks);
// L_cap then bounds token positions.
struct KVLayout {
  const int32_t* table = nullptr;
  int32_t table_len = 0;
  int32_t log2_bs = 0;
  int32_t num_blocks = 0;
  int32_t L_cap = 0;
};
// Position bound of a paged buffer (positions wrap around a short table).
constexpr int32_t kPagedPositionLimit = 1 << 30;

// Sequence-partition plan of one decode call (host side, pure function).
struct DecodePlan {
  int tiles_per_part;  // 32-key tiles per work-group
  int num_parts;       // work-groups per sequence
  size_t ws_bytes;     // workspace for partial states (0 when num_parts == 1)
  int heads_per_group; // query heads per work-group (grid z = ceil(Hq / heads_per_group))
  int max_seq_len;     // the host's bound on seq_lens; longer lengths are read as this
  int ragged_groups;   // > 0: balanced plan of a ragged batch with this many work-groups per head group
};
// block_size > 0: paged layout (bounds the tiles of a partition).
DecodePlan plan_decode(int32_t B, int32_t Hq, int32_t D, int32_t max_seq_len, int32_t window,
                       int num_cus, int32_t block_size = 0);
// Balanced plan for a batch of ragged lengths (contiguous buffers, bf16
// queries): a planner kernel splits the visible tiles of all sequences into
// ranges of equal cost per work-group (tiles plus a fixed cost per sequence
// start); windows short enough for the whole-range plan keep it
// (ragged_groups == 0 then).
DecodePlan plan_decode_ragged(int32_t B, int32_t Hq, int32_t D, int32_t max_seq_len, int32_t window,
                              int num_cus);
// Cost of a sequence start in the balanced plan, in tiles (the plan cuts
// tiles plus these costs into equal ranges).
constexpr int kRaggedSegmentCost = 40;

int launch_quantize(const float* src, int8_t* dst, float* dst_scale, const int32_t* start_pos,
                    int32_t B, int32_t T, int32_t D, int32_t L_cap, hipStream_t stream);
// K and V rows of T new tokens per sequence into a paged buffer (one launch).
int launch_quantize_paged(const float* k_src, const float* v_src, int8_t* k, int8_t* v, float* k_scale,
                          float* v_scale, const KVLayout& layout, const int32_t* start_pos, int32_t B,
                          int32_t T, int32_t D, hipStream_t stream);

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

// int8 queries: codes [B, Hq, D] and one fp32 scale per (token, head) row.
struct QueryInt8 {
  const int8_t* codes;
  const float* scale;
};

// Allocation-free decode: the partition states live in a static device array
// of kStaticScratchBytes per GPU; static_scratch() returns the current
// device's copy (looked up once per device), or nullptr if that fails.
constexpr size_t kStaticScratchBytes = MQA_NOALLOC_SCRATCH_BYTES;
void* static_scratch();

// Fixed tile-to-wave assignment for decode launches (bitwise repeatable
// results); returns the previous setting.
bool set_deterministic(bool on);

// q == nullptr with q8 set: the int8-query variant.
int launch_decode(const uint16_t* q, const mqa_kv_view& kv, const KVLayout& layout, const int32_t* seq_lens,
                  int32_t B, int32_t Hq, int32_t D, int32_t window, float softmax_scale, float* out,
                  void* workspace, const DecodePlan& plan, hipStream_t stream,
                  const AppendRows* append = nullptr, const QueryInt8* q8 = nullptr);

// Whole KV blocks of sequence b between device buffers and host pool slots.
int launch_kv_block_copy(bool to_device, const mqa_kv_view* bufs, int32_t n_bufs, int32_t b, int64_t first_block,
                         int64_t n_blocks, int32_t block_size, int32_t D, const int64_t* slots, void* pool,
                         hipStream_t stream);

size_t prefill_workspace_bytes(int32_t B, int32_t C, int32_t D, int32_t max_prefix_len);

int launch_prefill(const uint16_t* q, const mqa_kv_view& kv, const KVLayout& layout,
                   const int32_t* prefix_lens, int32_t max_prefix_len, int32_t B, int32_t C, int32_t Hq,
                   int32_t D, int32_t window, float softmax_scale, float* out, void* workspace,
                   hipStream_t stream);

}  // namespace mqa
