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
// A decode work item covers up to kItemParts consecutive 512-token partitions
// of one (sequence, KV head), or kLongItemParts for a sequence of at least
// kLongItemFrom partitions (fewer item boundaries where a sequence has many
// items); on the matrix cores its waves keep one softmax state for the whole
// item, meet once at its end and write one partial result.
constexpr int kItemParts = 2;
constexpr int kLongItemParts = 4;
constexpr int kLongItemFrom = 9;
__host__ __device__ inline int item_parts(int nparts) {
  return nparts >= kLongItemFrom ? kLongItemParts : kItemParts;
}
// Flags in a decode record's partition field (partition numbers stay below
// 2^16): the item covers that one partition only; the sequence's context
// length was not clamped, so its new token (position ctx - 1) is the one the
// append form stores; the item is the sequence's only one.
constexpr int kOnePartition = 1 << 16;
constexpr int kAppendable = 1 << 17;
// (and, for the matrix-core kernel, which writes one partial per item: the
// item is the sequence's only one, so its result is the output)
constexpr int kWholeSequence = 1 << 18;
constexpr int kPartitionMask = kOnePartition - 1;
// Slot of the plan's ticket header (sched) that is nonzero when some decode
// sequence's first block is also another decode sequence's first block (a
// shared prefix, a fork): the partition launch then keeps the default cache
// policy for its block loads instead of the streaming hint.
constexpr int kSchedShared = 4;

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
// The merge of one output row (query row x q head) by one wave (lane = its lane).  PER_TOKEN: the slot count is
// that of the row's query token (counts = the plan's row_slots; rows with one
// slot were already written by the partition or prefill kernels and are
// skipped); otherwise num_parts[row].
// Latency is one round trip per kMergeUnroll partitions: the first group's
// partial outputs are loaded before the maxima are reduced, and the maxima and
// sums are read lane-parallel (64 partitions per load).
constexpr int kMergeUnroll = 8;

template <bool BF16, int D, bool PER_TOKEN>
__device__ __forceinline__ void merge_row(
    int64_t row, int lane, void* __restrict__ out, const float* __restrict__ pm, const float* __restrict__ pl,
    const float* __restrict__ po, const int32_t* __restrict__ counts, int32_t Hq, int32_t max_parts) {
  constexpr int PER = D / kWave;
  constexpr int U = kMergeUnroll;
  int n;
  if constexpr (PER_TOKEN) {
    n = min(counts[row / Hq], max_parts);
    if (n <= 1) return;
  } else {
    n = max(0, min(counts[row], max_parts));
  }
  const float* rm = pm + row * max_parts;
  const float* rl = pl + row * max_parts;
  const float* ro = po + row * max_parts * D;

  float ov[U][PER];  // first group of partial outputs, in flight during the reductions
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int k = 0; k < PER; ++k) ov[u][k] = u < n ? ro[(int64_t)u * D + lane + k * kWave] : 0.f;
  }

  // live partial: l > 0 and a finite max; the rest weigh 0
  float M = -INFINITY;
  for (int base = 0; base < n; base += kWave) {
    const int i = base + lane;
    if (i < n && rl[i] > 0.f) M = fmaxf(M, rm[i]);
  }
  M = xor_max<1, kWave>(M);
  float o[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) o[k] = 0.f;
  float L = 0.f;
  if (M != -INFINITY) {
    // a dead partial is skipped, not weighted by 0: its output may hold NaN
    auto add = [&](int i, const float (&v)[PER]) {
      const float mi = rm[i], li = rl[i];
      if (li > 0.f && mi != -INFINITY) {
        const float w = li * exp2_fast(mi - M);
        L += w;
#pragma unroll
        for (int k = 0; k < PER; ++k) o[k] = fmaf(w, v[k], o[k]);
      }
    };
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u < n) add(u, ov[u]);
    }
    for (int base = U; base < n; base += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int k = 0; k < PER; ++k)
          ov[u][k] = base + u < n ? ro[(int64_t)(base + u) * D + lane + k * kWave] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (base + u < n) add(base + u, ov[u]);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    store_out<BF16>(out, row * D + lane + k * kWave, L > 0.f ? o[k] / L : 0.f);
  }
}


}  // namespace pkv
