// C ABI of libmqa_int8: argument validation and dispatch.
//
// Validation runs before any HIP call, so invalid arguments are reported on a
// machine without a GPU. The library keeps no state except the cached
// compute-unit count of each device it has seen.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "../../include/mqa_int8.h"
#include "launch.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return 256;
  }
  int cached = g_cu_count[dev].load(std::memory_order_relaxed);
  if (cached > 0) return cached;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
    (void)hipGetLastError();
    cus = 256;
  }
  g_cu_count[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool supported_d(int32_t D) { return D == 64 || D == 128; }
bool supported_hq(int32_t Hq) { return Hq >= 1 && Hq <= 64; }

int check_kv(const mqa_kv_view* kv, int32_t D) {
  if (!kv || !kv->k || !kv->v || !kv->k_scale || !kv->v_scale) return MQA_ERR_NULL;
  if (kv->L_cap <= 0) return MQA_ERR_SHAPE;
  if (!aligned16(kv->k) || !aligned16(kv->v)) return MQA_ERR_ALIGN;
  if (((uintptr_t)kv->k_scale & 3u) || ((uintptr_t)kv->v_scale & 3u)) return MQA_ERR_ALIGN;
  // the kernels address one sequence's K or V rows with 32-bit byte offsets
  if ((int64_t)kv->L_cap * D > (int64_t)0xffffffff) return MQA_ERR_SHAPE;
  return MQA_OK;
}

// Validation of mqa_decode's arguments (shared with the workspace query).
int check_decode_shape(int32_t B, int32_t Hq, int32_t D, int32_t max_seq_len) {
  if (B <= 0 || Hq <= 0 || D <= 0 || max_seq_len < 0) return MQA_ERR_SHAPE;
  if (!supported_d(D) || !supported_hq(Hq)) return MQA_ERR_UNSUPPORTED;
  if ((int64_t)B > 65535) return MQA_ERR_SHAPE;  // grid.y limit
  return MQA_OK;
}

// Validation of a paged buffer; fills the internal layout on success.
int check_paged(const mqa_kv_paged* kv, mqa::KVLayout* layout) {
  if (!kv || !kv->k || !kv->v || !kv->k_scale || !kv->v_scale || !kv->block_table) return MQA_ERR_NULL;
  const int32_t bs = kv->block_size;
  if (bs < 32 || bs > 4096 || (bs & (bs - 1)) != 0) return MQA_ERR_SHAPE;
  if (kv->table_len <= 0 || kv->num_blocks <= 0) return MQA_ERR_SHAPE;
  if ((int64_t)kv->num_blocks * bs > ((int64_t)1 << 40)) return MQA_ERR_SHAPE;
  if (!aligned16(kv->k) || !aligned16(kv->v) || !aligned16(kv->k_scale) || !aligned16(kv->v_scale))
    return MQA_ERR_ALIGN;
  if (((uintptr_t)kv->block_table & 3u) != 0) return MQA_ERR_ALIGN;
  int lb = 0;
  while ((1 << lb) < bs) ++lb;
  layout->table = kv->block_table;
  layout->table_len = kv->table_len;
  layout->log2_bs = lb;
  layout->num_blocks = kv->num_blocks;
  layout->L_cap = mqa::kPagedPositionLimit;
  return MQA_OK;
}

// Keys a windowed layer reads are resident when the table wraps: position t
// and t + table_len * block_size share a pool row, so the buffer holds
// exactly the last table_len * block_size positions written, and the `span`
// positions ending at the newest must fit in them.
bool resident(const mqa_kv_paged* kv, int64_t max_pos_end, int32_t window, int64_t span) {
  const int64_t cap = (int64_t)kv->table_len * kv->block_size;
  if (max_pos_end <= cap) return true;
  if (window <= 0) return false;
  return span <= cap;
}

int check_decode_common(const uint16_t* q, const int32_t* seq_lens, const float* out, int32_t B, int32_t Hq,
                        int32_t D, int32_t max_seq_len) {
  if (!q || !seq_lens || !out) return MQA_ERR_NULL;
  int st = check_decode_shape(B, Hq, D, max_seq_len);
  if (st != MQA_OK) return st;
  if (!aligned16(q) || !aligned16(out)) return MQA_ERR_ALIGN;
  return MQA_OK;
}

}  // namespace

extern "C" {

int mqa_set_deterministic(int enable) { return mqa::set_deterministic(enable != 0) ? 1 : 0; }

const char* mqa_status_string(int status) {
  switch (status) {
    case MQA_OK: return "ok";
    case MQA_ERR_NULL: return "a required pointer is NULL";
    case MQA_ERR_SHAPE: return "a size argument is out of range or inconsistent";
    case MQA_ERR_UNSUPPORTED: return "unsupported shape (head_dim must be 64 or 128, 1 <= Hq <= 64)";
    case MQA_ERR_ALIGN:
      return "a pointer is not suitably aligned (16 bytes for tensors, 4 for scales), or a decode call's cache "
             "capacity L_cap is not a multiple of 32";
    case MQA_ERR_WORKSPACE: return "workspace is missing or smaller than the size the matching *_workspace_bytes() returns";
    case MQA_ERR_HIP: return "a HIP runtime call or kernel launch failed";
    default: return "unknown status";
  }
}

int kv_quantize_int8(const float* src, int8_t* dst, float* dst_scale, const int32_t* start_pos,
                     int32_t B, int32_t T, int32_t D, int32_t L_cap, void* stream) {
  if (!src || !dst || !dst_scale || !start_pos) return MQA_ERR_NULL;
  if (B <= 0 || T <= 0 || D <= 0 || L_cap <= 0 || L_cap < T) return MQA_ERR_SHAPE;
  if (!supported_d(D)) return MQA_ERR_UNSUPPORTED;
  if (!aligned16(src) || !aligned16(dst) || ((uintptr_t)dst_scale & 3u)) return MQA_ERR_ALIGN;
  return mqa::launch_quantize(src, dst, dst_scale, start_pos, B, T, D, L_cap,
                              static_cast<hipStream_t>(stream));
}

size_t mqa_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t D, int32_t max_seq_len,
                                  int32_t window) {
  if (check_decode_shape(B, Hq, D, max_seq_len) != MQA_OK) return 0;
  return mqa::plan_decode(B, Hq, D, max_seq_len, window, device_cu_count()).ws_bytes;
}

int mqa_decode(const uint16_t* q, const mqa_kv_view* kv, const int32_t* seq_lens,
               int32_t max_seq_len, int32_t B, int32_t Hq, int32_t D, int32_t window,
               float softmax_scale, float* out, void* workspace, size_t workspace_bytes,
               void* stream) {
  if (!q || !kv || !seq_lens || !out) return MQA_ERR_NULL;
  int st = check_decode_shape(B, Hq, D, max_seq_len);
  if (st != MQA_OK) return st;
  st = check_kv(kv, D);
  if (st != MQA_OK) return st;
  if (max_seq_len > kv->L_cap) return MQA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(out)) return MQA_ERR_ALIGN;
  // whole 32-key tiles per sequence; scales read four keys at a time
  if ((kv->L_cap & 31) || !aligned16(kv->k_scale) || !aligned16(kv->v_scale)) return MQA_ERR_ALIGN;
  const mqa::DecodePlan plan = mqa::plan_decode(B, Hq, D, max_seq_len, window, device_cu_count());
  if (plan.ws_bytes > 0) {
    if (!workspace || workspace_bytes < plan.ws_bytes) return MQA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MQA_ERR_ALIGN;
  }
  return mqa::launch_decode(q, *kv, mqa::KVLayout{}, seq_lens, B, Hq, D, window, softmax_scale, out, workspace,
                            plan, static_cast<hipStream_t>(stream));
}

int mqa_decode_noalloc(const uint16_t* q, const mqa_kv_view* kv, const int32_t* seq_lens, int32_t max_seq_len,
                       int32_t B, int32_t Hq, int32_t D, int32_t window, float softmax_scale, float* out,
                       void* stream) {
  if (!q || !kv || !seq_lens || !out) return MQA_ERR_NULL;
  int st = check_decode_shape(B, Hq, D, max_seq_len);
  if (st != MQA_OK) return st;
  st = check_kv(kv, D);
  if (st != MQA_OK) return st;
  if (max_seq_len > kv->L_cap) return MQA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(out)) return MQA_ERR_ALIGN;
  if ((kv->L_cap & 31) || !aligned16(kv->k_scale) || !aligned16(kv->v_scale)) return MQA_ERR_ALIGN;
  const mqa::DecodePlan plan = mqa::plan_decode(B, Hq, D, max_seq_len, window, device_cu_count());
  void* ws = nullptr;
  if (plan.ws_bytes > 0) {
    if (plan.ws_bytes > mqa::kStaticScratchBytes) return MQA_ERR_WORKSPACE;
    ws = mqa::static_scratch();
    if (ws == nullptr) return MQA_ERR_HIP;
  }
  return mqa::launch_decode(q, *kv, mqa::KVLayout{}, seq_lens, B, Hq, D, window, softmax_scale, out, ws, plan,
                            static_cast<hipStream_t>(stream));
}

int mqa_decode_append(const uint16_t* q, const mqa_kv_cache* kv, const float* k_new, const float* v_new,
                      const int32_t* seq_lens, int32_t max_seq_len, int32_t B, int32_t Hq, int32_t D,
                      int32_t window, float softmax_scale, float* out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (!kv || !k_new || !v_new) return MQA_ERR_NULL;
  if (((uintptr_t)k_new & 3u) || ((uintptr_t)v_new & 3u)) return MQA_ERR_ALIGN;
  const mqa_kv_view view{kv->k, kv->v, kv->k_scale, kv->v_scale, kv->L_cap};
  if (!q || !seq_lens || !out) return MQA_ERR_NULL;
  int st = check_decode_shape(B, Hq, D, max_seq_len);
  if (st != MQA_OK) return st;
  st = check_kv(&view, D);
  if (st != MQA_OK) return st;
  if (max_seq_len > kv->L_cap) return MQA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(out)) return MQA_ERR_ALIGN;
  if ((kv->L_cap & 31) || !aligned16(kv->k_scale) || !aligned16(kv->v_scale)) return MQA_ERR_ALIGN;
  const mqa::DecodePlan plan = mqa::plan_decode(B, Hq, D, max_seq_len, window, device_cu_count());
  if (plan.ws_bytes > 0) {
    if (!workspace || workspace_bytes < plan.ws_bytes) return MQA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MQA_ERR_ALIGN;
  }
  const mqa::AppendRows rows{k_new, v_new, kv->k, kv->v, kv->k_scale, kv->v_scale};
  return mqa::launch_decode(q, view, mqa::KVLayout{}, seq_lens, B, Hq, D, window, softmax_scale, out, workspace,
                            plan, static_cast<hipStream_t>(stream), &rows);
}

namespace {
// The balanced planner counts tiles and sequence-start costs in 32-bit
// integers.
bool ragged_tiles_fit(int32_t B, int32_t max_seq_len) {
  return (int64_t)B * (((int64_t)max_seq_len + 31) / 32 + 1 + mqa::kRaggedSegmentCost) < ((int64_t)1 << 31);
}

int decode_ragged_impl(const uint16_t* q, const mqa_kv_view& view, const mqa_kv_cache* cache, const float* k_new,
                       const float* v_new, const int32_t* seq_lens, int32_t max_seq_len, int32_t B, int32_t Hq,
                       int32_t D, int32_t window, float softmax_scale, float* out, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (!q || !seq_lens || !out) return MQA_ERR_NULL;
  int st = check_decode_shape(B, Hq, D, max_seq_len);
  if (st != MQA_OK) return st;
  st = check_kv(&view, D);
  if (st != MQA_OK) return st;
  if (max_seq_len > view.L_cap || !ragged_tiles_fit(B, max_seq_len)) return MQA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(out)) return MQA_ERR_ALIGN;
  if ((view.L_cap & 31) || !aligned16(view.k_scale) || !aligned16(view.v_scale)) return MQA_ERR_ALIGN;
  if (cache) {
    if (!k_new || !v_new) return MQA_ERR_NULL;
    if (((uintptr_t)k_new & 3u) || ((uintptr_t)v_new & 3u)) return MQA_ERR_ALIGN;
  }
  const mqa::DecodePlan plan = mqa::plan_decode_ragged(B, Hq, D, max_seq_len, window, device_cu_count());
  if (plan.ws_bytes > 0) {
    if (!workspace || workspace_bytes < plan.ws_bytes) return MQA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MQA_ERR_ALIGN;
  }
  if (cache) {
    const mqa::AppendRows rows{k_new, v_new, cache->k, cache->v, cache->k_scale, cache->v_scale};
    return mqa::launch_decode(q, view, mqa::KVLayout{}, seq_lens, B, Hq, D, window, softmax_scale, out, workspace,
                              plan, static_cast<hipStream_t>(stream), &rows);
  }
  return mqa::launch_decode(q, view, mqa::KVLayout{}, seq_lens, B, Hq, D, window, softmax_scale, out, workspace,
                            plan, static_cast<hipStream_t>(stream));
}
}  // namespace

size_t mqa_decode_ragged_workspace_bytes(int32_t B, int32_t Hq, int32_t D, int32_t max_seq_len, int32_t window) {
  if (check_decode_shape(B, Hq, D, max_seq_len) != MQA_OK || !ragged_tiles_fit(B, max_seq_len)) return 0;
  return mqa::plan_decode_ragged(B, Hq, D, max_seq_len, window, device_cu_count()).ws_bytes;
}

int mqa_decode_ragged(const uint16_t* q, const mqa_kv_view* kv, const int32_t* seq_lens, int32_t max_seq_len,
                      int32_t B, int32_t Hq, int32_t D, int32_t window, float softmax_scale, float* out,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (!kv) return MQA_ERR_NULL;
  return decode_ragged_impl(q, *kv, nullptr, nullptr, nullptr, seq_lens, max_seq_len, B, Hq, D, window,
                            softmax_scale, out, workspace, workspace_bytes, stream);
}

int mqa_decode_append_ragged(const uint16_t* q, const mqa_kv_cache* kv, const float* k_new, const float* v_new,
                             const int32_t* seq_lens, int32_t max_seq_len, int32_t B, int32_t Hq, int32_t D,
                             int32_t window, float softmax_scale, float* out, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (!kv) return MQA_ERR_NULL;
  const mqa_kv_view view{kv->k, kv->v, kv->k_scale, kv->v_scale, kv->L_cap};
  return decode_ragged_impl(q, view, kv, k_new, v_new, seq_lens, max_seq_len, B, Hq, D, window, softmax_scale,
                            out, workspace, workspace_bytes, stream);
}

size_t mqa_prefill_workspace_bytes(int32_t B, int32_t C, int32_t D, int32_t max_prefix_len) {
  if (B <= 0 || C <= 0 || max_prefix_len < 0 || !supported_d(D)) return 0;
  return mqa::prefill_workspace_bytes(B, C, D, max_prefix_len);
}

int mqa_prefill_chunk(const uint16_t* q, const mqa_kv_view* kv, const int32_t* prefix_lens,
                      int32_t max_prefix_len, int32_t B, int32_t C, int32_t Hq, int32_t D,
                      int32_t window, float softmax_scale, float* out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (!q || !kv || !prefix_lens || !out) return MQA_ERR_NULL;
  if (B <= 0 || C <= 0 || Hq <= 0 || D <= 0 || max_prefix_len < 0) return MQA_ERR_SHAPE;
  if (!supported_d(D) || !supported_hq(Hq)) return MQA_ERR_UNSUPPORTED;
  int st = check_kv(kv, D);
  if (st != MQA_OK) return st;
  if ((int64_t)max_prefix_len + C > kv->L_cap) return MQA_ERR_SHAPE;
  if ((int64_t)B > 65535) return MQA_ERR_SHAPE;  // grid.y of the staging pass
  if (!aligned16(q) || !aligned16(out)) return MQA_ERR_ALIGN;
  if (!workspace || workspace_bytes < mqa::prefill_workspace_bytes(B, C, D, max_prefix_len))
    return MQA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MQA_ERR_ALIGN;
  return mqa::launch_prefill(q, *kv, mqa::KVLayout{}, prefix_lens, max_prefix_len, B, C, Hq, D, window,
                             softmax_scale, out, workspace, static_cast<hipStream_t>(stream));
}

int kv_quantize_int8_paged(const float* k_src, const float* v_src, const mqa_kv_paged* kv,
                           const int32_t* start_pos, int32_t B, int32_t T, int32_t D, void* stream) {
  if (!k_src || !v_src || !start_pos) return MQA_ERR_NULL;
  mqa::KVLayout layout;
  int st = check_paged(kv, &layout);
  if (st != MQA_OK) return st;
  if (B <= 0 || T <= 0 || D <= 0) return MQA_ERR_SHAPE;
  if ((int64_t)T > (int64_t)kv->table_len * kv->block_size) return MQA_ERR_SHAPE;
  if (!supported_d(D)) return MQA_ERR_UNSUPPORTED;
  if (!aligned16(k_src) || !aligned16(v_src)) return MQA_ERR_ALIGN;
  return mqa::launch_quantize_paged(k_src, v_src, kv->k, kv->v, kv->k_scale, kv->v_scale, layout, start_pos, B,
                                    T, D, static_cast<hipStream_t>(stream));
}

size_t mqa_decode_paged_workspace_bytes(int32_t B, int32_t Hq, int32_t D, int32_t max_seq_len, int32_t window,
                                        int32_t block_size) {
  if (check_decode_shape(B, Hq, D, max_seq_len) != MQA_OK) return 0;
  if (block_size < 32 || block_size > 4096 || (block_size & (block_size - 1)) != 0) return 0;
  return mqa::plan_decode(B, Hq, D, max_seq_len, window, device_cu_count(), block_size).ws_bytes;
}

namespace {
int decode_paged_impl(const uint16_t* q, const mqa_kv_paged* kv, const float* k_new, const float* v_new,
                      bool append, const int32_t* seq_lens, int32_t max_seq_len, int32_t B, int32_t Hq,
                      int32_t D, int32_t window, float softmax_scale, float* out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  int st = check_decode_common(q, seq_lens, out, B, Hq, D, max_seq_len);
  if (st != MQA_OK) return st;
  mqa::KVLayout layout;
  st = check_paged(kv, &layout);
  if (st != MQA_OK) return st;
  if (append) {
    if (!k_new || !v_new) return MQA_ERR_NULL;
    if (((uintptr_t)k_new & 3u) || ((uintptr_t)v_new & 3u)) return MQA_ERR_ALIGN;
  }
  if (max_seq_len >= mqa::kPagedPositionLimit) return MQA_ERR_SHAPE;
  if (!resident(kv, max_seq_len, window, window)) return MQA_ERR_SHAPE;
  const mqa::DecodePlan plan =
      mqa::plan_decode(B, Hq, D, max_seq_len, window, device_cu_count(), kv->block_size);
  if (plan.ws_bytes > 0) {
    if (!workspace || workspace_bytes < plan.ws_bytes) return MQA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MQA_ERR_ALIGN;
  }
  const mqa_kv_view view{kv->k, kv->v, kv->k_scale, kv->v_scale, 0};
  if (append) {
    const mqa::AppendRows rows{k_new, v_new, kv->k, kv->v, kv->k_scale, kv->v_scale};
    return mqa::launch_decode(q, view, layout, seq_lens, B, Hq, D, window, softmax_scale, out, workspace, plan,
                              static_cast<hipStream_t>(stream), &rows);
  }
  return mqa::launch_decode(q, view, layout, seq_lens, B, Hq, D, window, softmax_scale, out, workspace, plan,
                            static_cast<hipStream_t>(stream));
}
}  // namespace

int mqa_decode_paged(const uint16_t* q, const mqa_kv_paged* kv, const int32_t* seq_lens, int32_t max_seq_len,
                     int32_t B, int32_t Hq, int32_t D, int32_t window, float softmax_scale, float* out,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return decode_paged_impl(q, kv, nullptr, nullptr, false, seq_lens, max_seq_len, B, Hq, D, window,
                           softmax_scale, out, workspace, workspace_bytes, stream);
}

int mqa_decode_append_paged(const uint16_t* q, const mqa_kv_paged* kv, const float* k_new, const float* v_new,
                            const int32_t* seq_lens, int32_t max_seq_len, int32_t B, int32_t Hq, int32_t D,
                            int32_t window, float softmax_scale, float* out, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return decode_paged_impl(q, kv, k_new, v_new, true, seq_lens, max_seq_len, B, Hq, D, window, softmax_scale,
                           out, workspace, workspace_bytes, stream);
}

namespace {
int decode_q8_impl(const int8_t* q8, const float* q_scale, const mqa_kv_view& view, const mqa_kv_cache* cache,
                   const float* k_new, const float* v_new, const int32_t* seq_lens, int32_t max_seq_len, int32_t B,
                   int32_t Hq, int32_t D, int32_t window, float softmax_scale, float* out, void* workspace,
                   size_t workspace_bytes, void* stream) {
  if (!q8 || !q_scale || !seq_lens || !out) return MQA_ERR_NULL;
  int st = check_decode_shape(B, Hq, D, max_seq_len);
  if (st != MQA_OK) return st;
  st = check_kv(&view, D);
  if (st != MQA_OK) return st;
  if (max_seq_len > view.L_cap) return MQA_ERR_SHAPE;
  if (!aligned16(q8) || ((uintptr_t)q_scale & 3u) || !aligned16(out)) return MQA_ERR_ALIGN;
  if ((view.L_cap & 31) || !aligned16(view.k_scale) || !aligned16(view.v_scale)) return MQA_ERR_ALIGN;
  if (cache) {
    if (!k_new || !v_new) return MQA_ERR_NULL;
    if (((uintptr_t)k_new & 3u) || ((uintptr_t)v_new & 3u)) return MQA_ERR_ALIGN;
  }
  const mqa::DecodePlan plan = mqa::plan_decode(B, Hq, D, max_seq_len, window, device_cu_count());
  if (plan.ws_bytes > 0) {
    if (!workspace || workspace_bytes < plan.ws_bytes) return MQA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MQA_ERR_ALIGN;
  }
  const mqa::QueryInt8 qi{q8, q_scale};
  if (cache) {
    const mqa::AppendRows rows{k_new, v_new, cache->k, cache->v, cache->k_scale, cache->v_scale};
    return mqa::launch_decode(nullptr, view, mqa::KVLayout{}, seq_lens, B, Hq, D, window, softmax_scale, out,
                              workspace, plan, static_cast<hipStream_t>(stream), &rows, &qi);
  }
  return mqa::launch_decode(nullptr, view, mqa::KVLayout{}, seq_lens, B, Hq, D, window, softmax_scale, out,
                            workspace, plan, static_cast<hipStream_t>(stream), nullptr, &qi);
}
}  // namespace

int mqa_decode_q8(const int8_t* q8, const float* q_scale, const mqa_kv_view* kv, const int32_t* seq_lens,
                  int32_t max_seq_len, int32_t B, int32_t Hq, int32_t D, int32_t window, float softmax_scale,
                  float* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!kv) return MQA_ERR_NULL;
  return decode_q8_impl(q8, q_scale, *kv, nullptr, nullptr, nullptr, seq_lens, max_seq_len, B, Hq, D, window,
                        softmax_scale, out, workspace, workspace_bytes, stream);
}

int mqa_decode_append_q8(const int8_t* q8, const float* q_scale, const mqa_kv_cache* kv, const float* k_new,
                         const float* v_new, const int32_t* seq_lens, int32_t max_seq_len, int32_t B, int32_t Hq,
                         int32_t D, int32_t window, float softmax_scale, float* out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (!kv) return MQA_ERR_NULL;
  const mqa_kv_view view{kv->k, kv->v, kv->k_scale, kv->v_scale, kv->L_cap};
  return decode_q8_impl(q8, q_scale, view, kv, k_new, v_new, seq_lens, max_seq_len, B, Hq, D, window,
                        softmax_scale, out, workspace, workspace_bytes, stream);
}

namespace {
int check_transfer(const mqa_kv_view* bufs, int32_t n_bufs, int32_t B, int32_t b, int64_t first_block,
                   int64_t n_blocks, int32_t block_size, int32_t D, const int64_t* slots, const void* pool,
                   int64_t pool_slots) {
  if (!bufs || !pool || (n_blocks > 0 && !slots)) return MQA_ERR_NULL;
  if (n_bufs < 1 || n_bufs > 8 || B <= 0 || b < 0 || b >= B || first_block < 0 || n_blocks < 0 || pool_slots <= 0)
    return MQA_ERR_SHAPE;
  if (block_size <= 0 || block_size % 16 != 0) return MQA_ERR_SHAPE;
  if (!supported_d(D)) return MQA_ERR_UNSUPPORTED;
  if (!aligned16(pool)) return MQA_ERR_ALIGN;
  for (int32_t i = 0; i < n_bufs; ++i) {
    const mqa_kv_view& v = bufs[i];
    if (!v.k || !v.v || !v.k_scale || !v.v_scale) return MQA_ERR_NULL;
    if (v.L_cap <= 0 || (first_block + n_blocks) * (int64_t)block_size > v.L_cap) return MQA_ERR_SHAPE;
    if (!aligned16(v.k) || !aligned16(v.v) || ((uintptr_t)v.k_scale & 3u) || ((uintptr_t)v.v_scale & 3u))
      return MQA_ERR_ALIGN;
  }
  for (int64_t i = 0; i < n_blocks; ++i)
    if (slots[i] < 0 || slots[i] >= pool_slots) return MQA_ERR_SHAPE;
  return MQA_OK;
}
}  // namespace

int mqa_kv_blocks_to_host(const mqa_kv_view* bufs, int32_t n_bufs, int32_t B, int32_t b, int64_t first_block,
                          int64_t n_blocks, int32_t block_size, int32_t D, const int64_t* slots, void* host_pool,
                          int64_t pool_slots, void* stream) {
  const int st =
      check_transfer(bufs, n_bufs, B, b, first_block, n_blocks, block_size, D, slots, host_pool, pool_slots);
  if (st != MQA_OK || n_blocks == 0) return st;
  return mqa::launch_kv_block_copy(false, bufs, n_bufs, b, first_block, n_blocks, block_size, D, slots, host_pool,
                                   static_cast<hipStream_t>(stream));
}

int mqa_kv_blocks_to_device(const mqa_kv_cache* bufs, int32_t n_bufs, int32_t B, int32_t b, int64_t first_block,
                            int64_t n_blocks, int32_t block_size, int32_t D, const int64_t* slots,
                            const void* host_pool, int64_t pool_slots, void* stream) {
  if (!bufs) return MQA_ERR_NULL;
  if (n_bufs < 1 || n_bufs > 8) return MQA_ERR_SHAPE;
  mqa_kv_view views[8];
  for (int32_t i = 0; i < n_bufs; ++i)
    views[i] = mqa_kv_view{bufs[i].k, bufs[i].v, bufs[i].k_scale, bufs[i].v_scale, bufs[i].L_cap};
  const int st =
      check_transfer(views, n_bufs, B, b, first_block, n_blocks, block_size, D, slots, host_pool, pool_slots);
  if (st != MQA_OK || n_blocks == 0) return st;
  return mqa::launch_kv_block_copy(true, views, n_bufs, b, first_block, n_blocks, block_size, D, slots,
                                   const_cast<void*>(host_pool), static_cast<hipStream_t>(stream));
}

int mqa_prefill_chunk_paged(const uint16_t* q, const mqa_kv_paged* kv, const int32_t* prefix_lens,
                            int32_t max_prefix_len, int32_t B, int32_t C, int32_t Hq, int32_t D, int32_t window,
                            float softmax_scale, float* out, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (!q || !prefix_lens || !out) return MQA_ERR_NULL;
  mqa::KVLayout layout;
  int st = check_paged(kv, &layout);
  if (st != MQA_OK) return st;
  if (B <= 0 || C <= 0 || Hq <= 0 || D <= 0 || max_prefix_len < 0) return MQA_ERR_SHAPE;
  if (!supported_d(D) || !supported_hq(Hq)) return MQA_ERR_UNSUPPORTED;
  if ((int64_t)max_prefix_len + C >= mqa::kPagedPositionLimit) return MQA_ERR_SHAPE;
  if (!resident(kv, (int64_t)max_prefix_len + C, window, (int64_t)window + C - 1)) return MQA_ERR_SHAPE;
  if ((int64_t)B > 65535) return MQA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(out)) return MQA_ERR_ALIGN;
  if (!workspace || workspace_bytes < mqa::prefill_workspace_bytes(B, C, D, max_prefix_len))
    return MQA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MQA_ERR_ALIGN;
  const mqa_kv_view view{kv->k, kv->v, kv->k_scale, kv->v_scale, 0};
  return mqa::launch_prefill(q, view, layout, prefix_lens, max_prefix_len, B, C, Hq, D, window, softmax_scale,
                             out, workspace, static_cast<hipStream_t>(stream));
}

}  // extern "C"
