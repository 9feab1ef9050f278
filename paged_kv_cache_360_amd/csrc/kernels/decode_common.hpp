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
constexpr int kPlanThreads = 1024;                  // work-list builder: one workgroup
// A decode work item covers up to PKV_ITEM_PARTS consecutive 512-token
// partitions of one (sequence, KV head): the waves keep one state per partition
// and meet once per item, while each partition still yields its own partial for
// the merge.
#ifndef PKV_ITEM_PARTS
#define PKV_ITEM_PARTS 2
#endif
constexpr int kItemParts = PKV_ITEM_PARTS;
constexpr int kItemBlocks = kItemParts * kPartBlocks;

struct DecodeParams {
  void* out;
  const void* q;
  const char* kc;
  const char* vc;
  const int32_t* tables;
  const int32_t* ctx;
  const int32_t* qsl;    // [S+1] or null (row s is sequence s)
  float scale_log2;
  int32_t num_seqs;
  int32_t num_tokens;    // query rows T
  int32_t Hkv;
  int32_t MB;
  int32_t NB;
  int32_t max_parts;
  int32_t ctx_cap;       // min(MB * 16, max_parts * 512): larger lengths are clamped
  int32_t* sched;        // [0] decode tickets taken from the counter, [1] decode tickets; [2], [3] prefill
  const int4* dec_recs;  // decode records {sequence, partition, context, query row}
  const int4* pre_recs;  // prefill records, two int4 each (see plan.hip)
  const int32_t* row_slots;
  int32_t dec_cap, pre_cap;
  float* part_m;
  float* part_l;
  float* part_o;
  const char* knew;      // append form: the new tokens' K [S, Hkv, D] (else null)
  const char* vnew;      // and V
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
  return max(0, min(p.ctx[s], p.ctx_cap));
}

}  // namespace pkv

namespace pkv {
struct DecodeArgs;
DecodeParams make_params(const DecodeArgs& a);
// bf16 partition kernel on the matrix cores (decode_mfma.hip).
int launch_decode_partitions_bf16(const DecodeParams& p, const DecodeArgs& a, void* stream);
}  // namespace pkv
