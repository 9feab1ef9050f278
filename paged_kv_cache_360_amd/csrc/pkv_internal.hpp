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

// Pool-to-pool block copy; the pool pointers are device addresses (a host pool's
// device mapping).
int launch_swap_blocks(void* dk, void* dv, const void* sk, const void* sv, const int32_t* pairs,
                       int32_t num_pairs, int32_t src_blocks, int32_t dst_blocks, int64_t block_bytes,
                       void* stream);

struct DecodeArgs {
  void* out;             // [T, Hq, D]
  const void* q;         // [T, Hq, D]
  const void* kc;
  const void* vc;
  const int32_t* tables;
  const int32_t* ctx;
  const int32_t* qsl;    // [S+1] first query row of each sequence; null: row s is sequence s
  float scale_log2;      // softmax scale times log2(e)
  int32_t num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim;
  int32_t max_blocks;    // table row width
  int32_t num_blocks;    // pool size (ids outside [0, num_blocks) are not read)
  int32_t max_parts;     // partitions per query row the workspace holds
  int32_t max_query_len; // host bound on query rows per sequence (1 for decode)
  bool bf16;
  int32_t num_cus;       // compute units of the current device
  // workspace (see workspace_layout in api.cpp)
  int32_t* sched;        // [0], [1]: decode ticket counter, tickets; [2], [3]: prefill
  int32_t* dec_recs;     // decode work list, dec_cap records of 4 int32
  int32_t* pre_recs;     // prefill work list, pre_cap records of 8 int32
  int32_t* row_slots;    // [T] partial results each query row's merge combines (plan)
  int32_t dec_cap, pre_cap;
  float* part_m;         // [T*Hq, max_parts]
  float* part_l;         // [T*Hq, max_parts]
  float* part_o;         // [T*Hq, max_parts, D]
  // Append form of decode (bf16): each sequence's new token (position ctx - 1)
  // is read from these [S, Hkv, D] rows instead of the cache, and written to
  // the cache, by the partition launch.  Null otherwise.
  const void* knew;
  const void* vnew;
};

// Rows of one prefill work item (one workgroup of eight wavefronts, each with
// one 32-column MFMA tile of 32/G rows x G heads).
inline int32_t prefill_rows_per_item(int32_t G) { return 256 / G; }

// Work-list plan: decode records, prefill records and per-row merge slot counts.
int launch_plan(const DecodeArgs& a, void* stream);
// Plan (decode, or varlen when a.qsl is set: query_start_loc is read from the
// device) from a page-locked host copy of the context lengths (host_ctx,
// its device address), fused with a copy of `bytes` (a multiple of 16) from
// page-locked host memory src to device memory dst (device addresses), with
// the copy of the used entries of each row of the page-locked host_tables
// (device address; null: none) into a.tables, and, when prev is given, with the
// merge of the partials in prev's workspace into prev->out (a previous step of
// the same shapes, another workspace).
int launch_upload_plan(const DecodeArgs& a, const int32_t* host_ctx, const void* src, void* dst,
                       int64_t bytes, const int32_t* host_tables, const DecodeArgs* prev, void* stream);
// Chunked-prefill rows (sequences with more than one query row), bf16 only.
int launch_prefill(const DecodeArgs& a, void* stream);

// Split-context decode partitions of the one-row sequences: writes the output
// of single-partition rows and the partials of the others.  Expects the plan.
int launch_decode_partitions(const DecodeArgs& a, void* stream);
// Log-sum-exp merge of the partials of multi-partition rows (any query length).
int launch_decode_merge(const DecodeArgs& a, void* stream);

// The decode workspace in a library-owned device array (static_workspace.hip):
// its size, and its address on the current device, taken once per device
// (returns 0, or the HIP error of that lookup).
size_t static_workspace_capacity();
int static_workspace(void** out);

int launch_lse_merge(void* out, const float* part_m, const float* part_l, const float* part_o,
                     const int32_t* num_parts, int32_t rows, int32_t max_parts, int32_t head_dim,
                     bool bf16, void* stream);

}  // namespace pkv
