// Shared between the two decode partition kernels (fp32 on the vector ALUs, bf16
// on the matrix cores) and the log-sum-exp merge: the kernel parameter block and
// the output store.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"

namespace pkv {

constexpr int kDecodeThreads = 256;                 // 4 wavefronts per workgroup
constexpr int kDecodeWaves = kDecodeThreads / kWave;

struct DecodeParams {
  void* out;
  const void* q;
  const char* kc;
  const char* vc;
  const int32_t* tables;
  const int32_t* ctx;
  float scale_log2;
  int32_t Hkv;
  int32_t MB;
  int32_t NB;
  int32_t max_parts;
  float* part_m;
  float* part_l;
  float* part_o;
};

template <bool BF16>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float v) {
  if constexpr (BF16) {
    reinterpret_cast<uint16_t*>(out)[idx] = f32_to_bf16(v);
  } else {
    reinterpret_cast<float*>(out)[idx] = v;
  }
}

// Context length of sequence s, clamped to what the table width and the
// workspace can hold (a larger value is never faulted on).
__device__ __forceinline__ int clamped_ctx(const DecodeParams& p, int s) {
  const int c = p.ctx[s];
  return max(0, min(c, min(p.MB * kBlockTokens, p.max_parts * kPartTokens)));
}

}  // namespace pkv

namespace pkv {
struct DecodeArgs;
// bf16 partition kernel on the matrix cores (decode_mfma.hip).
int launch_decode_partitions_bf16(const DecodeParams& p, const DecodeArgs& a, void* stream);
}  // namespace pkv
