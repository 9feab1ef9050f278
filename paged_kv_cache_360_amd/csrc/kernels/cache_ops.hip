// Cache writes on gfx950: the slot scatter of new tokens' K/V rows, the
// copy-on-write block copy and the block copy between two pools (swapping
// between the device pool and a page-locked host pool).  Both are byte copies in 16-byte vectors; a token row
// (num_kv_heads * head_dim elements) and a block (16 rows) are contiguous in the
// [num_blocks, 16, num_kv_heads, head_dim] layout, so each workgroup streams one
// contiguous span with fully coalesced dwordx4 loads and stores.

#include <hip/hip_runtime.h>

#include "../pkv_internal.hpp"
#include "device_common.hpp"

namespace pkv {

namespace {

constexpr int kCopyThreads = 256;

// One workgroup per token: copy its K row and V row into slot slots[t].
__global__ __launch_bounds__(kCopyThreads) void kv_write_kernel(
    char* __restrict__ kc, char* __restrict__ vc, const char* __restrict__ k,
    const char* __restrict__ v, const int32_t* __restrict__ slots, int64_t num_slots,
    int32_t row_bytes) {
  const int64_t t = blockIdx.x;
  const int32_t slot = slots[t];
  if (slot < 0 || (int64_t)slot >= num_slots) return;  // padding token or out of the pool
  const int64_t dst = (int64_t)slot * row_bytes;
  const int64_t src = t * row_bytes;
  for (int32_t off = threadIdx.x * 16; off < row_bytes; off += kCopyThreads * 16) {
    const uint4 a = load16(k + src + off);
    const uint4 b = load16(v + src + off);
    *reinterpret_cast<uint4*>(kc + dst + off) = a;
    *reinterpret_cast<uint4*>(vc + dst + off) = b;
  }
}

// One workgroup per (pair, cache): block dst := block src.
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    char* __restrict__ kc, char* __restrict__ vc, const int32_t* __restrict__ pairs,
    int32_t num_blocks, int64_t block_bytes) {
  const int32_t src = pairs[2 * blockIdx.x];
  const int32_t dst = pairs[2 * blockIdx.x + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  char* base = blockIdx.y == 0 ? kc : vc;
  const char* s = base + (int64_t)src * block_bytes;
  char* d = base + (int64_t)dst * block_bytes;
  for (int64_t off = threadIdx.x * 16; off < block_bytes; off += kCopyThreads * 16) {
    *reinterpret_cast<uint4*>(d + off) = load16(s + off);
  }
}

// Loads in flight per thread in the pool-to-pool copy: a read across the host
// link takes microseconds, so each thread issues a whole batch before storing.
constexpr int kSwapBatch = 8;

// One workgroup per (pair, cache): block dst of the destination pool := block
// src of the source pool.  Either pool may be page-locked host memory reached
// through its device mapping.
__global__ __launch_bounds__(kCopyThreads) void swap_blocks_kernel(
    char* __restrict__ dk, char* __restrict__ dv, const char* __restrict__ sk,
    const char* __restrict__ sv, const int32_t* __restrict__ pairs, int32_t src_blocks,
    int32_t dst_blocks, int64_t block_bytes) {
  const int32_t src = pairs[2 * blockIdx.x];
  const int32_t dst = pairs[2 * blockIdx.x + 1];
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
  const char* s = (blockIdx.y == 0 ? sk : sv) + (int64_t)src * block_bytes;
  char* d = (blockIdx.y == 0 ? dk : dv) + (int64_t)dst * block_bytes;
  constexpr int64_t kStride = (int64_t)kCopyThreads * 16;
  for (int64_t base = threadIdx.x * 16; base < block_bytes; base += kStride * kSwapBatch) {
    uint4 r[kSwapBatch];
#pragma unroll
    for (int u = 0; u < kSwapBatch; ++u) {
      const int64_t off = base + u * kStride;
      if (off < block_bytes) r[u] = load16(s + off);
    }
#pragma unroll
    for (int u = 0; u < kSwapBatch; ++u) {
      const int64_t off = base + u * kStride;
      if (off < block_bytes) *reinterpret_cast<uint4*>(d + off) = r[u];
    }
  }
}

}  // namespace

int launch_kv_write(void* kc, void* vc, const void* k, const void* v, const int32_t* slots,
                    int32_t num_tokens, int64_t num_slots, int32_t row_bytes, void* stream) {
  hipLaunchKernelGGL(kv_write_kernel, dim3(num_tokens), dim3(kCopyThreads), 0,
                     (hipStream_t)stream, (char*)kc, (char*)vc, (const char*)k, (const char*)v,
                     slots, num_slots, row_bytes);
  return (int)hipGetLastError();
}

int launch_copy_blocks(void* kc, void* vc, const int32_t* pairs, int32_t num_pairs,
                       int32_t num_blocks, int64_t block_bytes, void* stream) {
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs, 2), dim3(kCopyThreads), 0,
                     (hipStream_t)stream, (char*)kc, (char*)vc, pairs, num_blocks, block_bytes);
  return (int)hipGetLastError();
}

int launch_swap_blocks(void* dk, void* dv, const void* sk, const void* sv, const int32_t* pairs,
                       int32_t num_pairs, int32_t src_blocks, int32_t dst_blocks, int64_t block_bytes,
                       void* stream) {
  hipLaunchKernelGGL(swap_blocks_kernel, dim3(num_pairs, 2), dim3(kCopyThreads), 0,
                     (hipStream_t)stream, (char*)dk, (char*)dv, (const char*)sk, (const char*)sv, pairs,
                     src_blocks, dst_blocks, block_bytes);
  return (int)hipGetLastError();
}

}  // namespace pkv
