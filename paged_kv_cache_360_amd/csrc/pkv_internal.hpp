// Internal interface between the C ABI (api.cpp), the allocator and the HIP
// kernel launchers.  Not installed; no HIP types appear here so that host-only
// translation units can include it.
#pragma once

#include <cstddef>
#include <cstdint>

namespace pkv {

// Per-thread last-error message (pkv_last_error()).
void set_error(const char* msg);
inline int fail(int code, const char* msg) {
  set_error(msg);
  return code;
}

// Launchers return 0 on success or the HIP error code of the failed launch.
// All pointers are device pointers already validated by api.cpp.

int launch_kv_write(void* kc, void* vc, const void* k, const void* v, const int32_t* slots,
                    int32_t num_tokens, int64_t num_slots, int32_t row_bytes, void* stream);

int launch_copy_blocks(void* kc, void* vc, const int32_t* pairs, int32_t num_pairs,
                       int32_t num_blocks, int64_t block_bytes, void* stream);

struct DecodeArgs {
  void* out;
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* tables;
  const int32_t* ctx;
  float scale_log2;      // softmax scale times log2(e)
  int32_t num_seqs, num_q_heads, num_kv_heads, head_dim;
  int32_t max_blocks;    // table row width
  int32_t num_blocks;    // pool size (ids outside [0, num_blocks) are not read)
  int32_t max_parts;     // partitions per sequence the workspace holds
  bool bf16;
  int32_t num_cus;       // compute units of the current device
  int32_t* sched;        // workspace header: ticket counter and ticket count
  int32_t* recs;         // workspace: work list, [S * max_parts, 4] int32 records
  float* part_m;         // [S*Hq, max_parts]
  float* part_l;         // [S*Hq, max_parts]
  float* part_o;         // [S*Hq, max_parts, D]
};

// Split-context decode partitions: writes the output of single-partition
// sequences and the partials of the others.
int launch_decode_partitions(const DecodeArgs& a, void* stream);
// Log-sum-exp merge of the partials of multi-partition sequences.
int launch_decode_merge(const DecodeArgs& a, void* stream);

int launch_lse_merge(void* out, const float* part_m, const float* part_l, const float* part_o,
                     const int32_t* num_parts, int32_t rows, int32_t max_parts, int32_t head_dim,
                     bool bf16, void* stream);

}  // namespace pkv
