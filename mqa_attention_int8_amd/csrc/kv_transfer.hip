// Copies of whole KV blocks between a sequence's rows in device KV buffers
// and slots of a host pool (the data plane of the host-memory prefix cache:
// 9c1h.cn news page, section 秘訣2, and explinks.com "Character.AI 的最佳实践",
// section 有状态缓存: KV kept in host memory between conversation turns and
// brought back for the matching prefix).
//
// Host slot layout: for each of the n_bufs buffers in order, the block's K
// rows [bs, D] int8, V rows [bs, D] int8, K scales [bs] fp32, V scales [bs]
// fp32. The pool is pinned host memory that the device reads and writes
// directly (one launch moves up to kMaxBlocks blocks of every buffer; no
// per-block runtime copies).
#include "common.h"
#include "launch.h"

namespace mqa {

namespace {

constexpr int kMaxBlocks = 64;
constexpr int kMaxBufs = 8;

struct TransferArgs {
  int8_t* k[kMaxBufs];
  int8_t* v[kMaxBufs];
  float* ks[kMaxBufs];
  float* vs[kMaxBufs];
  int64_t row0[kMaxBufs];  // device row of block 0's first position in each buffer
  int64_t slot[kMaxBlocks];
  char* pool;
  int32_t bs, D, n_bufs;
};

// grid (blocks, n_bufs, 4 tensors); TO_DEVICE: pool -> device, else device -> pool.
template <bool TO_DEVICE>
__global__ __launch_bounds__(256) void kv_block_copy_kernel(TransferArgs a) {
  const int blk = blockIdx.x, buf = blockIdx.y, part = blockIdx.z;
  const int bs = a.bs, D = a.D;
  const int64_t per_buf = (int64_t)bs * (2 * D + 8);
  char* slot = a.pool + a.slot[blk] * per_buf * a.n_bufs + per_buf * buf;
  const int64_t row = a.row0[buf] + (int64_t)blk * bs;
  if (part < 2) {
    int8_t* dev = (part == 0 ? a.k[buf] : a.v[buf]) + row * D;
    char* host = slot + (int64_t)part * bs * D;
    const int n16 = bs * D / 16;
    for (int i = threadIdx.x; i < n16; i += 256) {
      if (TO_DEVICE)
        reinterpret_cast<u32x4*>(dev)[i] = reinterpret_cast<const u32x4*>(host)[i];
      else
        reinterpret_cast<u32x4*>(host)[i] = reinterpret_cast<const u32x4*>(dev)[i];
    }
  } else {
    float* dev = (part == 2 ? a.ks[buf] : a.vs[buf]) + row;
    float* host = reinterpret_cast<float*>(slot + 2 * (int64_t)bs * D) + (part - 2) * bs;
    for (int i = threadIdx.x; i < bs; i += 256) {
      if (TO_DEVICE)
        dev[i] = host[i];
      else
        host[i] = dev[i];
    }
  }
}

}  // namespace

int launch_kv_block_copy(bool to_device, const mqa_kv_view* bufs, int32_t n_bufs, int32_t b, int64_t first_block,
                         int64_t n_blocks, int32_t block_size, int32_t D, const int64_t* slots, void* pool,
                         hipStream_t stream) {
  TransferArgs a;
  for (int i = 0; i < n_bufs; ++i) {
    a.k[i] = const_cast<int8_t*>(bufs[i].k);
    a.v[i] = const_cast<int8_t*>(bufs[i].v);
    a.ks[i] = const_cast<float*>(bufs[i].k_scale);
    a.vs[i] = const_cast<float*>(bufs[i].v_scale);
  }
  // The device address of the pinned pool; memory the runtime did not pin
  // and map (pageable memory) is refused here instead of faulting a kernel.
  void* dpool = nullptr;
  if (hipHostGetDevicePointer(&dpool, pool, 0) != hipSuccess || dpool == nullptr) {
    (void)hipGetLastError();
    return MQA_ERR_HIP;
  }
  a.pool = static_cast<char*>(dpool);
  a.bs = block_size;
  a.D = D;
  a.n_bufs = n_bufs;
  for (int64_t done = 0; done < n_blocks; done += kMaxBlocks) {
    const int64_t n = n_blocks - done < kMaxBlocks ? n_blocks - done : kMaxBlocks;
    for (int i = 0; i < n_bufs; ++i) a.row0[i] = (int64_t)b * bufs[i].L_cap + (first_block + done) * block_size;
    for (int64_t i = 0; i < n; ++i) a.slot[i] = slots[done + i];
    const dim3 grid((unsigned)n, (unsigned)n_bufs, 4);
    if (to_device)
      hipLaunchKernelGGL(kv_block_copy_kernel<true>, grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(kv_block_copy_kernel<false>, grid, dim3(256), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return MQA_ERR_HIP;
  }
  return MQA_OK;
}

}  // namespace mqa
