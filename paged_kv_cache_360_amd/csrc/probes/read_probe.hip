// Read-bandwidth probes: plain read kernels over the same K/V bytes a decode
// launch reads, the ceiling its achieved rate is compared with.
//
// Measurement code (libpkvprobe.so), not part of the attention library: the
// bench loads it to report the partition kernel's KV-read rate against what a
// kernel that only reads the same bytes, in the same block order, reaches on
// the same device.  Two access patterns:
//
//  * blocks: each work item is one whole block of the pool (16 token rows of
//    all KV heads, contiguous) of K and of V;
//  * slices: each work item is one (block, KV head) slice, 16 rows of
//    head_dim * 2 bytes at the token stride, of K and of V -- the pattern of
//    the partition kernel, which serves one KV head per work item.
//
// Items are taken in list order by a grid-stride loop; each thread keeps eight
// 16-byte loads in flight and folds what it read into one word, stored per
// workgroup so that no load can be dropped.  The loads carry the nontemporal
// hint, as the partition kernel's block loads do (the faster form of a plain
// read here: 6.8 against 6.1 TB/s for blocks in random order).

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 8;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t fold(uint4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

// Whole blocks: item i reads block ids[i] of K and of V (block_bytes each).
__global__ __launch_bounds__(kThreads) void probe_read_blocks_kernel(const char* __restrict__ kc,
                                                                     const char* __restrict__ vc,
                                                                     const int32_t* __restrict__ ids,
                                                                     int32_t n_items, int32_t block_bytes,
                                                                     uint32_t* __restrict__ sink) {
  const int per = block_bytes / 16;  // 16-byte pieces per block and cache
  uint32_t acc = 0;
  for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
    const int64_t base = (int64_t)ids[it] * block_bytes;
    const uint4* k = reinterpret_cast<const uint4*>(kc + base);
    const uint4* v = reinterpret_cast<const uint4*>(vc + base);
    for (int p0 = threadIdx.x; p0 < per; p0 += kThreads * kInFlight / 2) {
      uint4 r[kInFlight];
#pragma unroll
      for (int u = 0; u < kInFlight / 2; ++u) {
        const int p = p0 + u * kThreads;
        r[2 * u] = p < per ? ld(k + p) : uint4{0, 0, 0, 0};
        r[2 * u + 1] = p < per ? ld(v + p) : uint4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < kInFlight; ++u) acc ^= fold(r[u]);
    }
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;  // never taken in practice; keeps the loads
}

// Per-head slices: item i reads KV head i % hkv of block ids[i / hkv], 16 rows
// of row_bytes (head_dim * 2) at a stride of tok_bytes, of K and of V.  A
// workgroup handles four items at once, one per wave.
__global__ __launch_bounds__(kThreads) void probe_read_slices_kernel(const char* __restrict__ kc,
                                                                     const char* __restrict__ vc,
                                                                     const int32_t* __restrict__ ids,
                                                                     int32_t n_items, int32_t hkv, int32_t row_bytes,
                                                                     int32_t tok_bytes, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int per_row = row_bytes / 16;     // 16-byte pieces per row (16 at head_dim 128)
  const int pieces = 16 * per_row;        // per slice and cache
  uint32_t acc = 0;
  for (int it0 = blockIdx.x * 4; it0 < n_items; it0 += gridDim.x * 4) {
    const int it = it0 + wave;
    if (it < n_items) {
      const int64_t base = (int64_t)ids[it / hkv] * 16 * tok_bytes + (int64_t)(it % hkv) * row_bytes;
      for (int p0 = lane; p0 < pieces; p0 += 64 * kInFlight / 2) {
        uint4 r[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight / 2; ++u) {
          const int p = p0 + u * 64;
          const int64_t off = base + (int64_t)(p / per_row) * tok_bytes + (p % per_row) * 16;
          r[2 * u] = p < pieces ? ld(kc + off) : uint4{0, 0, 0, 0};
          r[2 * u + 1] = p < pieces ? ld(vc + off) : uint4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) acc ^= fold(r[u]);
      }
    }
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" {

// Reads K and V of the n_items blocks listed in ids (device int32; every id in
// [0, pool blocks)) from the pools kc, vc (device, blocks of block_bytes, a
// multiple of 16) on `stream`; sink: device uint32[grid].  Returns 0 or a HIP error.
int pkv_probe_read_blocks(const void* kc, const void* vc, const int32_t* ids, int32_t n_items,
                          int32_t block_bytes, int32_t grid, uint32_t* sink, void* stream) {
  if (n_items <= 0 || grid <= 0 || block_bytes <= 0 || block_bytes % 16) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(probe_read_blocks_kernel, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                     static_cast<const char*>(kc), static_cast<const char*>(vc), ids, n_items, block_bytes, sink);
  return (int)hipGetLastError();
}

// Reads, for each listed block and each KV head, that head's 16-row slice of K
// and of V (n_items = blocks * hkv work items).  Rows are row_bytes long (a
// multiple of 16) at a stride of tok_bytes = hkv * row_bytes.
int pkv_probe_read_slices(const void* kc, const void* vc, const int32_t* ids, int32_t n_blocks, int32_t hkv,
                          int32_t row_bytes, int32_t grid, uint32_t* sink, void* stream) {
  if (n_blocks <= 0 || hkv <= 0 || grid <= 0 || row_bytes <= 0 || row_bytes % 16) return (int)hipErrorInvalidValue;
  const int64_t items = (int64_t)n_blocks * hkv;
  if (items > INT32_MAX) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(probe_read_slices_kernel, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                     static_cast<const char*>(kc), static_cast<const char*>(vc), ids, (int32_t)items, hkv, row_bytes,
                     hkv * row_bytes, sink);
  return (int)hipGetLastError();
}

}  // extern "C"
