// C ABI: argument validation, workspace layout and launch dispatch.
//
// Every entry point validates its arguments on the host before any HIP call, so
// an error launches nothing and touches no buffer.  Launch failures reported by
// the runtime map to PKV_ELAUNCH.

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/pagedkv.h"
#include "pkv_internal.hpp"

namespace pkv {

namespace {
thread_local char g_last_error[256] = "";

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline int64_t elem_size(pkv_dtype dt) { return dt == PKV_BF16 ? 2 : 4; }
inline bool dtype_ok(pkv_dtype dt) { return dt == PKV_F32 || dt == PKV_BF16; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
int64_t parts_for(int64_t max_ctx) { return (max_ctx + PKV_PARTITION_TOKENS - 1) / PKV_PARTITION_TOKENS; }

constexpr size_t kSchedBytes = 256;  // decode workspace header: ticket counters and counts
constexpr size_t kDecRecBytes = 4 * sizeof(int32_t);  // {sequence, partition, context, query row}
constexpr size_t kPreRecBytes = 8 * sizeof(int32_t);  // two int4 (see plan.hip)

// Workspace of one attention call: header, the two work lists, per-row slot
// counts and (when a row can span several partitions) the partials.
struct WsLayout {
  size_t dec, pre, slots, pm, pl, po, total;
  int64_t P, dec_cap, pre_cap;
};
WsLayout workspace_layout(int64_t S, int64_t T, int64_t Hq, int64_t G, int64_t D, int64_t max_qlen,
                          int64_t max_ctx) {
  WsLayout w{};
  w.P = std::max<int64_t>(1, parts_for(max_ctx));
  w.dec_cap = S * w.P;
  const int64_t rpi = prefill_rows_per_item((int32_t)G);
  w.pre_cap = max_qlen > 1 ? ((T + rpi - 1) / rpi + S) * w.P : 0;
  size_t off = kSchedBytes;
  w.dec = off; off += align256((size_t)w.dec_cap * kDecRecBytes);
  w.pre = off; off += align256((size_t)w.pre_cap * kPreRecBytes);
  w.slots = off; off += align256((size_t)T * sizeof(int32_t));
  if (w.P > 1) {
    const size_t rows = (size_t)T * Hq;
    w.pm = off; off += align256(rows * w.P * sizeof(float));
    w.pl = off; off += align256(rows * w.P * sizeof(float));
    w.po = off; off += align256(rows * w.P * D * sizeof(float));
  }
  w.total = off;
  return w;
}

// Compute units of the current device, queried once per device.
int32_t device_cus() {
  static int32_t cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64 && cache[dev] > 0) return cache[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < 64) cache[dev] = n;
  return n;
}


// Device address of a buffer of `bytes` bytes at p: device memory as is,
// page-locked host memory through its device mapping.  False for pageable or
// unknown memory, or when the first and last byte do not lie in one mapping.
bool device_span(const void* p, int64_t bytes, void** dev_out) {
  if (!p || bytes <= 0) return false;
  hipPointerAttribute_t a0{}, a1{};
  const char* last = static_cast<const char*>(p) + (bytes - 1);
  if (hipPointerGetAttributes(&a0, p) != hipSuccess) { (void)hipGetLastError(); return false; }
  if (hipPointerGetAttributes(&a1, last) != hipSuccess) { (void)hipGetLastError(); return false; }
  if (a0.type != a1.type || !a0.devicePointer || !a1.devicePointer) return false;
  if (a0.type != hipMemoryTypeDevice && a0.type != hipMemoryTypeHost) return false;
  const char* d0 = static_cast<const char*>(a0.devicePointer);
  const char* d1 = static_cast<const char*>(a1.devicePointer);
  if (d1 - d0 != bytes - 1) return false;
  *dev_out = a0.devicePointer;
  return true;
}

// Page-locked host memory mapped for the device: its device address.
bool host_mapped(const void* p, int64_t bytes, void** dev_out) {
  if (!device_span(p, bytes, dev_out)) return false;
  hipPointerAttribute_t a{};
  return hipPointerGetAttributes(&a, p) == hipSuccess && a.type == hipMemoryTypeHost;
}

// A small table the kernel reads (pairs): device memory only.
bool device_readable(const void* p, int64_t bytes) {
  void* d = nullptr;
  if (!device_span(p, bytes, &d)) return false;
  hipPointerAttribute_t a{};
  return hipPointerGetAttributes(&a, p) == hipSuccess && a.type == hipMemoryTypeDevice && d == p;
}

int launched(int hip_status, const char* who) {
  if (hip_status == 0) return PKV_OK;
  char buf[256];
  std::snprintf(buf, sizeof(buf), "%s: launch failed: %s", who,
                hipGetErrorString((hipError_t)hip_status));
  set_error(buf);
  return PKV_ELAUNCH;
}
}  // namespace

void set_error(const char* msg) {
  std::strncpy(g_last_error, msg, sizeof(g_last_error) - 1);
  g_last_error[sizeof(g_last_error) - 1] = '\0';
}

}  // namespace pkv

using pkv::fail;

extern "C" {

const char* pkv_last_error(void) { return pkv::g_last_error; }

const char* pkv_strerror(int code) {
  switch (code) {
    case PKV_OK: return "PKV_OK";
    case PKV_EINVAL: return "PKV_EINVAL";
    case PKV_EUNSUPPORTED: return "PKV_EUNSUPPORTED";
    case PKV_ENOMEM: return "PKV_ENOMEM";
    case PKV_ELAUNCH: return "PKV_ELAUNCH";
    case PKV_ENOSEQ: return "PKV_ENOSEQ";
    case PKV_EWORKSPACE: return "PKV_EWORKSPACE";
    case PKV_ESWAPPED: return "PKV_ESWAPPED";
    default: return "PKV_UNKNOWN";
  }
}

int pkv_write(void* key_cache, void* value_cache, const void* k, const void* v,
              const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
              int32_t block_size, int32_t num_kv_heads, int32_t head_dim, pkv_dtype dt,
              void* stream) {
  if (!pkv::dtype_ok(dt)) return fail(PKV_EUNSUPPORTED, "pkv_write: unsupported dtype");
  if (block_size != PKV_BLOCK_SIZE) return fail(PKV_EUNSUPPORTED, "pkv_write: block_size must be 16");
  if (num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0 || head_dim <= 0)
    return fail(PKV_EINVAL, "pkv_write: bad sizes");
  const int64_t row_bytes = (int64_t)num_kv_heads * head_dim * pkv::elem_size(dt);
  if (row_bytes % 16 != 0 || row_bytes > INT32_MAX)
    return fail(PKV_EUNSUPPORTED, "pkv_write: row bytes must be a multiple of 16");
  if (num_tokens == 0) return PKV_OK;
  if (!key_cache || !value_cache || !k || !v || !slot_mapping)
    return fail(PKV_EINVAL, "pkv_write: null pointer");
  if (!pkv::aligned16(key_cache) || !pkv::aligned16(value_cache) || !pkv::aligned16(k) ||
      !pkv::aligned16(v))
    return fail(PKV_EINVAL, "pkv_write: pointers must be 16-byte aligned");
  return pkv::launched(pkv::launch_kv_write(key_cache, value_cache, k, v, slot_mapping, num_tokens,
                                            (int64_t)num_blocks * block_size, (int32_t)row_bytes,
                                            stream),
                       "pkv_write");
}

size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                  int32_t max_context_len) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 0) return 0;
  return pkv::workspace_layout(num_seqs, num_seqs, num_q_heads, 1, head_dim, 1, max_context_len).total;
}

size_t pkv_varlen_workspace_bytes(int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t max_query_len,
                                  int32_t max_context_len) {
  if (num_seqs <= 0 || num_tokens < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads != 0 || head_dim <= 0 || max_query_len < 1 || max_context_len < 0)
    return 0;
  const int32_t G = num_q_heads / num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return 0;
  return pkv::workspace_layout(num_seqs, num_tokens, num_q_heads, G, head_dim, max_query_len,
                               max_context_len).total;
}

}  // extern "C"

namespace {

// Shared validation of the decode arguments; fills `a` on success.
// qsl == nullptr: decode (query row s is sequence s, num_tokens == num_seqs).
int prepare_attention(const char* who, pkv::DecodeArgs& a, void* out, const void* q,
                      const void* key_cache, const void* value_cache, const int32_t* block_tables,
                      const int32_t* context_lens, const int32_t* qsl, int32_t num_tokens,
                      int32_t max_query_len, float scale, int32_t block_size, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t num_seqs,
                      int32_t max_blocks_per_seq, int32_t num_blocks, int32_t max_context_len,
                      pkv_dtype dt, void* workspace, size_t workspace_bytes) {
  char msg[160];
  auto bad = [&](int code, const char* what) {
    std::snprintf(msg, sizeof(msg), "%s: %s", who, what);
    return fail(code, msg);
  };
  if (!pkv::dtype_ok(dt)) return bad(PKV_EUNSUPPORTED, "unsupported dtype");
  if (block_size != PKV_BLOCK_SIZE) return bad(PKV_EUNSUPPORTED, "block_size must be 16");
  if (head_dim != 64 && head_dim != 128) return bad(PKV_EUNSUPPORTED, "head_dim must be 64 or 128");
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return bad(PKV_EINVAL, "num_q_heads must be a positive multiple of num_kv_heads");
  const int32_t G = num_q_heads / num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return bad(PKV_EUNSUPPORTED, "q heads per KV head must be 1, 2, 4 or 8");
  if (num_seqs < 0 || num_seqs > 65535 || max_blocks_per_seq <= 0 || num_blocks <= 0 ||
      max_context_len < 0 || num_kv_heads > 65535)
    return bad(PKV_EINVAL, "bad sizes");
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * PKV_BLOCK_SIZE)
    return bad(PKV_EINVAL, "max_context_len exceeds the table width");
  // The kernels take the row max of raw scores and mask with -inf before the
  // scale is applied, which is right only for a positive scale.
  if (!std::isfinite(scale) || !(scale > 0.f)) return bad(PKV_EINVAL, "scale must be finite and positive");
  if (num_tokens < 0 || max_query_len < 1) return bad(PKV_EINVAL, "bad query sizes");
  if (num_seqs == 0 || num_tokens == 0) return PKV_OK;
  if (!out || !q || !key_cache || !value_cache || !block_tables || !context_lens)
    return bad(PKV_EINVAL, "null pointer");
  if (!pkv::aligned16(out) || !pkv::aligned16(q) || !pkv::aligned16(key_cache) ||
      !pkv::aligned16(value_cache))
    return bad(PKV_EINVAL, "pointers must be 16-byte aligned");
  const int64_t P = std::max<int64_t>(1, pkv::parts_for(max_context_len));
  if (P > 65535) return bad(PKV_EUNSUPPORTED, "context too long");
  const pkv::WsLayout w = pkv::workspace_layout(num_seqs, num_tokens, num_q_heads, G, head_dim,
                                                max_query_len, max_context_len);
  if ((int64_t)num_tokens * num_q_heads * w.P > INT32_MAX || w.dec_cap * num_kv_heads > INT32_MAX ||
      w.pre_cap * num_kv_heads > INT32_MAX)
    return bad(PKV_EUNSUPPORTED, "batch too large");
  if (!workspace || workspace_bytes < w.total || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return bad(PKV_EWORKSPACE, "workspace missing, too small or not 256-byte aligned");

  a.out = out;
  a.q = q;
  a.kc = key_cache;
  a.vc = value_cache;
  a.tables = block_tables;
  a.ctx = context_lens;
  a.qsl = qsl;
  a.scale_log2 = scale * 1.4426950408889634f;  // log2(e)
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.max_query_len = max_query_len;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.max_parts = (int32_t)P;
  a.bf16 = dt == PKV_BF16;
  a.num_cus = pkv::device_cus();
  char* ws = static_cast<char*>(workspace);
  a.sched = reinterpret_cast<int32_t*>(ws);
  a.dec_recs = reinterpret_cast<int32_t*>(ws + w.dec);
  a.pre_recs = reinterpret_cast<int32_t*>(ws + w.pre);
  a.row_slots = reinterpret_cast<int32_t*>(ws + w.slots);
  a.dec_cap = (int32_t)w.dec_cap;
  a.pre_cap = (int32_t)w.pre_cap;
  if (w.P > 1) {
    a.part_m = reinterpret_cast<float*>(ws + w.pm);
    a.part_l = reinterpret_cast<float*>(ws + w.pl);
    a.part_o = reinterpret_cast<float*>(ws + w.po);
  }
  return PKV_OK;
}

// The page-locked host buffers and device targets of a fused upload + plan
// launch, checked with the HIP runtime; their device addresses on success.
struct UploadPtrs {
  const int32_t* hctx = nullptr;
  const void* src = nullptr;
  void* dst = nullptr;
  const int32_t* htab = nullptr;
};
int check_upload(const char* who, int32_t num_seqs, int32_t max_blocks_per_seq, const int32_t* block_tables,
                 const int32_t* host_context_lens, const void* upload_src, void* upload_dst, size_t upload_bytes,
                 const int32_t* host_block_tables, UploadPtrs& up) {
  char msg[200];
  auto bad = [&](const char* what) {
    std::snprintf(msg, sizeof(msg), "%s: %s", who, what);
    return fail(PKV_EINVAL, msg);
  };
  void* hctx = nullptr;
  if (!pkv::host_mapped(host_context_lens, (int64_t)num_seqs * 4, &hctx))
    return bad("host_context_lens must be page-locked host memory");
  void* src = nullptr;
  if (upload_bytes > 0) {
    if (!pkv::host_mapped(upload_src, (int64_t)upload_bytes, &src))
      return bad("upload_src must be page-locked host memory");
    if (!pkv::device_readable(upload_dst, (int64_t)upload_bytes)) return bad("upload_dst must be device memory");
    if (!pkv::aligned16(src) || !pkv::aligned16(upload_dst)) return bad("upload buffers must be 16-byte aligned");
    up.dst = upload_dst;
  }
  void* htab = nullptr;
  if (host_block_tables != nullptr) {
    const int64_t tab_bytes = (int64_t)num_seqs * max_blocks_per_seq * 4;
    if (!pkv::host_mapped(host_block_tables, tab_bytes, &htab))
      return bad("host_block_tables must be page-locked host memory");
    if (!pkv::device_readable(block_tables, tab_bytes)) return bad("block_tables must be device memory");
  }
  up.hctx = static_cast<const int32_t*>(hctx);
  up.src = src;
  up.htab = static_cast<const int32_t*>(htab);
  return PKV_OK;
}

}  // namespace

#define PKV_DECODE_ARGS                                                                        \
  void *out, const void *q, const void *key_cache, const void *value_cache,                    \
      const int32_t *block_tables, const int32_t *context_lens, float scale, int32_t block_size, \
      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t num_seqs,           \
      int32_t max_blocks_per_seq, int32_t num_blocks, int32_t max_context_len, pkv_dtype dt,   \
      void *workspace, size_t workspace_bytes, void *stream
#define PKV_DECODE_FWD                                                                          \
  out, q, key_cache, value_cache, block_tables, context_lens, nullptr, num_seqs, 1, scale,     \
      block_size, num_q_heads, num_kv_heads, head_dim, num_seqs, max_blocks_per_seq, num_blocks, \
      max_context_len, dt, workspace, workspace_bytes

extern "C" {

int pkv_attention_decode_plan(PKV_DECODE_ARGS) {
  pkv::DecodeArgs a{};
  const char* who = "pkv_attention_decode_plan";
  int rc = prepare_attention(who, a, PKV_DECODE_FWD);
  if (rc != PKV_OK || num_seqs == 0) return rc;
  return pkv::launched(pkv::launch_plan(a, stream), who);
}

int pkv_attention_decode_plan_upload(void* out, const void* q, const void* key_cache, const void* value_cache,
                                     const int32_t* block_tables, const int32_t* context_lens, float scale,
                                     int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t num_seqs, int32_t max_blocks_per_seq,
                                     int32_t num_blocks, int32_t max_context_len, pkv_dtype dt, void* workspace,
                                     size_t workspace_bytes, const int32_t* host_context_lens,
                                     const void* upload_src, void* upload_dst, size_t upload_bytes,
                                     const int32_t* host_block_tables, void* merge_out,
                                     const void* merge_workspace, void* stream) {
  pkv::DecodeArgs a{};
  const char* who = "pkv_attention_decode_plan_upload";
  if (num_seqs <= 0) return fail(PKV_EINVAL, "pkv_attention_decode_plan_upload: num_seqs must be > 0");
  if (upload_bytes % 16 != 0 || upload_bytes > (size_t)INT64_MAX)
    return fail(PKV_EINVAL, "pkv_attention_decode_plan_upload: upload_bytes must be a multiple of 16");
  int rc = prepare_attention(who, a, PKV_DECODE_FWD);
  if (rc != PKV_OK) return rc;
  UploadPtrs up{};
  rc = check_upload(who, num_seqs, max_blocks_per_seq, block_tables, host_context_lens, upload_src, upload_dst,
                    upload_bytes, host_block_tables, up);
  if (rc != PKV_OK) return rc;
  pkv::DecodeArgs prev{};
  const pkv::DecodeArgs* prev_p = nullptr;
  if (merge_out != nullptr || merge_workspace != nullptr) {
    if (merge_workspace == workspace)
      return fail(PKV_EINVAL, "pkv_attention_decode_plan_upload: merge_workspace must differ from workspace");
    // the previous step: same shapes and bound, its own output and workspace
    rc = prepare_attention(who, prev, merge_out, q, key_cache, value_cache, block_tables, context_lens, nullptr,
                           num_seqs, 1, scale, block_size, num_q_heads, num_kv_heads, head_dim, num_seqs,
                           max_blocks_per_seq, num_blocks, max_context_len, dt, const_cast<void*>(merge_workspace),
                           workspace_bytes);
    if (rc != PKV_OK) return rc;
    prev_p = &prev;
  }
  return pkv::launched(pkv::launch_upload_plan(a, up.hctx, up.src, up.dst, (int64_t)upload_bytes, up.htab, prev_p,
                                               stream),
                       who);
}

int pkv_attention_decode_partitions(PKV_DECODE_ARGS) {
  pkv::DecodeArgs a{};
  const char* who = "pkv_attention_decode_partitions";
  int rc = prepare_attention(who, a, PKV_DECODE_FWD);
  if (rc != PKV_OK || num_seqs == 0) return rc;
  return pkv::launched(pkv::launch_decode_partitions(a, stream), who);
}

int pkv_attention_decode_merge(PKV_DECODE_ARGS) {
  pkv::DecodeArgs a{};
  const char* who = "pkv_attention_decode_merge";
  int rc = prepare_attention(who, a, PKV_DECODE_FWD);
  if (rc != PKV_OK || num_seqs == 0) return rc;
  return pkv::launched(pkv::launch_decode_merge(a, stream), who);
}

int pkv_attention_decode(PKV_DECODE_ARGS) {
  pkv::DecodeArgs a{};
  const char* who = "pkv_attention_decode";
  int rc = prepare_attention(who, a, PKV_DECODE_FWD);
  if (rc != PKV_OK || num_seqs == 0) return rc;
  rc = pkv::launched(pkv::launch_plan(a, stream), who);
  if (rc != PKV_OK) return rc;
  rc = pkv::launched(pkv::launch_decode_partitions(a, stream), who);
  if (rc != PKV_OK) return rc;
  return pkv::launched(pkv::launch_decode_merge(a, stream), who);
}

int pkv_attention_decode_noalloc(void* out, const void* q, const void* key_cache, const void* value_cache,
                                 const int32_t* block_tables, const int32_t* context_lens, float scale,
                                 int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks,
                                 int32_t max_context_len, pkv_dtype dt, void* stream) {
  const char* who = "pkv_attention_decode_noalloc";
  const size_t cap = pkv::static_workspace_capacity();
  // Every check before any HIP call: the size against the array, then the
  // decode checks with a stand-in workspace of the array's size (never read).
  const size_t need = pkv_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len);
  if (need > cap) {
    char msg[192];
    std::snprintf(msg, sizeof(msg), "%s: this batch needs a %zu-byte workspace; the static one holds %zu", who,
                  need, cap);
    return fail(PKV_EWORKSPACE, msg);
  }
  {
    pkv::DecodeArgs a{};
    int rc = prepare_attention(who, a, out, q, key_cache, value_cache, block_tables, context_lens, nullptr,
                               num_seqs, 1, scale, block_size, num_q_heads, num_kv_heads, head_dim, num_seqs,
                               max_blocks_per_seq, num_blocks, max_context_len, dt,
                               reinterpret_cast<void*>(uintptr_t(256)), cap);
    if (rc != PKV_OK || num_seqs == 0) return rc;
  }
  void* ws = nullptr;
  const int e = pkv::static_workspace(&ws);
  if (e != 0) return pkv::launched(e, who);
  // the plan launch clears the ticket counters itself: nothing to reset here
  return pkv_attention_decode(out, q, key_cache, value_cache, block_tables, context_lens, scale, block_size,
                              num_q_heads, num_kv_heads, head_dim, num_seqs, max_blocks_per_seq, num_blocks,
                              max_context_len, dt, ws, cap, stream);
}

#define PKV_APPEND_ARGS                                                                         \
  void *out, const void *q, const void *k_new, const void *v_new, void *key_cache,               \
      void *value_cache, const int32_t *block_tables, const int32_t *context_lens, float scale,   \
      int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,           \
      int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks, int32_t max_context_len, \
      pkv_dtype dt, void *workspace, size_t workspace_bytes, void *stream

namespace {
// Validation shared by the append entries: the decode checks plus the new rows.
int prepare_append(const char* who, pkv::DecodeArgs& a, PKV_APPEND_ARGS) {
  (void)stream;
  char msg[160];
  if (dt != PKV_BF16) {
    std::snprintf(msg, sizeof(msg), "%s: bf16 only", who);
    return fail(PKV_EUNSUPPORTED, msg);
  }
  int rc = prepare_attention(who, a, PKV_DECODE_FWD);
  if (rc != PKV_OK || num_seqs == 0) return rc;
  if (!k_new || !v_new) {
    std::snprintf(msg, sizeof(msg), "%s: null k_new / v_new", who);
    return fail(PKV_EINVAL, msg);
  }
  if (!pkv::aligned16(k_new) || !pkv::aligned16(v_new)) {
    std::snprintf(msg, sizeof(msg), "%s: k_new / v_new must be 16-byte aligned", who);
    return fail(PKV_EINVAL, msg);
  }
  a.knew = k_new;
  a.vnew = v_new;
  return PKV_OK;
}
}  // namespace

int pkv_attention_decode_partitions_append(PKV_APPEND_ARGS) {
  pkv::DecodeArgs a{};
  const char* who = "pkv_attention_decode_partitions_append";
  int rc = prepare_append(who, a, out, q, k_new, v_new, key_cache, value_cache, block_tables,
                          context_lens, scale, block_size, num_q_heads, num_kv_heads, head_dim,
                          num_seqs, max_blocks_per_seq, num_blocks, max_context_len, dt, workspace,
                          workspace_bytes, stream);
  if (rc != PKV_OK || num_seqs == 0) return rc;
  return pkv::launched(pkv::launch_decode_partitions(a, stream), who);
}

int pkv_attention_decode_append(PKV_APPEND_ARGS) {
  pkv::DecodeArgs a{};
  const char* who = "pkv_attention_decode_append";
  int rc = prepare_append(who, a, out, q, k_new, v_new, key_cache, value_cache, block_tables,
                          context_lens, scale, block_size, num_q_heads, num_kv_heads, head_dim,
                          num_seqs, max_blocks_per_seq, num_blocks, max_context_len, dt, workspace,
                          workspace_bytes, stream);
  if (rc != PKV_OK || num_seqs == 0) return rc;
  rc = pkv::launched(pkv::launch_plan(a, stream), who);
  if (rc != PKV_OK) return rc;
  rc = pkv::launched(pkv::launch_decode_partitions(a, stream), who);
  if (rc != PKV_OK) return rc;
  return pkv::launched(pkv::launch_decode_merge(a, stream), who);
}

int pkv_attention_varlen(void* out, const void* q, const void* key_cache, const void* value_cache,
                         const int32_t* block_tables, const int32_t* context_lens,
                         const int32_t* query_start_loc, int32_t num_tokens, int32_t max_query_len,
                         float scale, int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t num_seqs, int32_t max_blocks_per_seq,
                         int32_t num_blocks, int32_t max_context_len, pkv_dtype dt, void* workspace,
                         size_t workspace_bytes, void* stream) {
  pkv::DecodeArgs a{};
  const char* who = "pkv_attention_varlen";
  if (dt != PKV_BF16) return fail(PKV_EUNSUPPORTED, "pkv_attention_varlen: bf16 only");
  if (num_tokens > 0 && num_seqs > 0 && !query_start_loc)
    return fail(PKV_EINVAL, "pkv_attention_varlen: null query_start_loc");
  int rc = prepare_attention(who, a, out, q, key_cache, value_cache, block_tables, context_lens,
                             query_start_loc, num_tokens, max_query_len, scale, block_size, num_q_heads,
                             num_kv_heads, head_dim, num_seqs, max_blocks_per_seq, num_blocks,
                             max_context_len, dt, workspace, workspace_bytes);
  if (rc != PKV_OK || num_seqs == 0 || num_tokens == 0) return rc;
  rc = pkv::launched(pkv::launch_plan(a, stream), who);
  if (rc != PKV_OK) return rc;
  rc = pkv::launched(pkv::launch_decode_partitions(a, stream), who);
  if (rc != PKV_OK) return rc;
  rc = pkv::launched(pkv::launch_prefill(a, stream), who);
  if (rc != PKV_OK) return rc;
  return pkv::launched(pkv::launch_decode_merge(a, stream), who);
}

#define PKV_VARLEN_ARGS                                                                            \
  void *out, const void *q, const void *key_cache, const void *value_cache,                        \
      const int32_t *block_tables, const int32_t *context_lens, const int32_t *query_start_loc,     \
      int32_t num_tokens, int32_t max_query_len, float scale, int32_t block_size, int32_t num_q_heads, \
      int32_t num_kv_heads, int32_t head_dim, int32_t num_seqs, int32_t max_blocks_per_seq,         \
      int32_t num_blocks, int32_t max_context_len, pkv_dtype dt, void *workspace, size_t workspace_bytes
#define PKV_VARLEN_FWD                                                                             \
  out, q, key_cache, value_cache, block_tables, context_lens, query_start_loc, num_tokens, max_query_len, \
      scale, block_size, num_q_heads, num_kv_heads, head_dim, num_seqs, max_blocks_per_seq, num_blocks, \
      max_context_len, dt, workspace, workspace_bytes

namespace {
static int prepare_varlen(const char* who, pkv::DecodeArgs& a, PKV_VARLEN_ARGS) {
  char msg[160];
  if (dt != PKV_BF16) {
    std::snprintf(msg, sizeof(msg), "%s: bf16 only", who);
    return fail(PKV_EUNSUPPORTED, msg);
  }
  if (num_tokens > 0 && num_seqs > 0 && !query_start_loc) {
    std::snprintf(msg, sizeof(msg), "%s: null query_start_loc", who);
    return fail(PKV_EINVAL, msg);
  }
  return prepare_attention(who, a, out, q, key_cache, value_cache, block_tables, context_lens, query_start_loc,
                           num_tokens, max_query_len, scale, block_size, num_q_heads, num_kv_heads, head_dim,
                           num_seqs, max_blocks_per_seq, num_blocks, max_context_len, dt, workspace,
                           workspace_bytes);
}
}  // namespace

int pkv_attention_varlen_plan_upload(PKV_VARLEN_ARGS, const int32_t* host_context_lens, const void* upload_src,
                                     void* upload_dst, size_t upload_bytes, const int32_t* host_block_tables,
                                     void* stream) {
  pkv::DecodeArgs a{};
  const char* who = "pkv_attention_varlen_plan_upload";
  if (num_seqs <= 0 || num_tokens <= 0)
    return fail(PKV_EINVAL, "pkv_attention_varlen_plan_upload: num_seqs and num_tokens must be > 0");
  if (upload_bytes % 16 != 0 || upload_bytes > (size_t)INT64_MAX)
    return fail(PKV_EINVAL, "pkv_attention_varlen_plan_upload: upload_bytes must be a multiple of 16");
  int rc = prepare_varlen(who, a, PKV_VARLEN_FWD);
  if (rc != PKV_OK) return rc;
  UploadPtrs up{};
  rc = check_upload(who, num_seqs, max_blocks_per_seq, block_tables, host_context_lens, upload_src, upload_dst,
                    upload_bytes, host_block_tables, up);
  if (rc != PKV_OK) return rc;
  return pkv::launched(pkv::launch_upload_plan(a, up.hctx, up.src, up.dst, (int64_t)upload_bytes, up.htab, nullptr,
                                               stream),
                       who);
}

int pkv_attention_varlen_partitions(PKV_VARLEN_ARGS, void* stream) {
  pkv::DecodeArgs a{};
  const char* who = "pkv_attention_varlen_partitions";
  int rc = prepare_varlen(who, a, PKV_VARLEN_FWD);
  if (rc != PKV_OK || num_seqs == 0 || num_tokens == 0) return rc;
  rc = pkv::launched(pkv::launch_decode_partitions(a, stream), who);
  if (rc != PKV_OK) return rc;
  rc = pkv::launched(pkv::launch_prefill(a, stream), who);
  if (rc != PKV_OK) return rc;
  return pkv::launched(pkv::launch_decode_merge(a, stream), who);
}

// The launches of pkv_attention_varlen one by one (plan, decode partitions,
// prefill tiles, merge), in that order on one workspace.
int pkv_attention_varlen_plan(PKV_VARLEN_ARGS, void* stream) {
  pkv::DecodeArgs a{};
  const char* who = "pkv_attention_varlen_plan";
  int rc = prepare_varlen(who, a, PKV_VARLEN_FWD);
  if (rc != PKV_OK || num_seqs == 0 || num_tokens == 0) return rc;
  return pkv::launched(pkv::launch_plan(a, stream), who);
}

int pkv_attention_varlen_decode_partitions(PKV_VARLEN_ARGS, void* stream) {
  pkv::DecodeArgs a{};
  const char* who = "pkv_attention_varlen_decode_partitions";
  int rc = prepare_varlen(who, a, PKV_VARLEN_FWD);
  if (rc != PKV_OK || num_seqs == 0 || num_tokens == 0) return rc;
  return pkv::launched(pkv::launch_decode_partitions(a, stream), who);
}

int pkv_attention_varlen_prefill_tiles(PKV_VARLEN_ARGS, void* stream) {
  pkv::DecodeArgs a{};
  const char* who = "pkv_attention_varlen_prefill_tiles";
  int rc = prepare_varlen(who, a, PKV_VARLEN_FWD);
  if (rc != PKV_OK || num_seqs == 0 || num_tokens == 0) return rc;
  return pkv::launched(pkv::launch_prefill(a, stream), who);
}

int pkv_attention_varlen_merge(PKV_VARLEN_ARGS, void* stream) {
  pkv::DecodeArgs a{};
  const char* who = "pkv_attention_varlen_merge";
  int rc = prepare_varlen(who, a, PKV_VARLEN_FWD);
  if (rc != PKV_OK || num_seqs == 0 || num_tokens == 0) return rc;
  return pkv::launched(pkv::launch_decode_merge(a, stream), who);
}

int pkv_lse_merge(void* out, const float* part_m, const float* part_l, const float* part_o,
                  const int32_t* num_parts, int32_t rows, int32_t max_parts, int32_t head_dim,
                  pkv_dtype out_dt, void* stream) {
  if (!pkv::dtype_ok(out_dt)) return fail(PKV_EUNSUPPORTED, "pkv_lse_merge: unsupported dtype");
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_EUNSUPPORTED, "pkv_lse_merge: head_dim must be 64 or 128");
  if (rows < 0 || max_parts <= 0) return fail(PKV_EINVAL, "pkv_lse_merge: bad sizes");
  if (rows == 0) return PKV_OK;
  if (!out || !part_m || !part_l || !part_o || !num_parts)
    return fail(PKV_EINVAL, "pkv_lse_merge: null pointer");
  return pkv::launched(pkv::launch_lse_merge(out, part_m, part_l, part_o, num_parts, rows, max_parts,
                                             head_dim, out_dt == PKV_BF16, stream),
                       "pkv_lse_merge");
}

int pkv_copy_blocks(void* key_cache, void* value_cache, const int32_t* pairs,
                    int32_t num_pairs, int32_t num_blocks, int32_t block_size,
                    int32_t num_kv_heads, int32_t head_dim, pkv_dtype dt, void* stream) {
  if (!pkv::dtype_ok(dt)) return fail(PKV_EUNSUPPORTED, "pkv_copy_blocks: unsupported dtype");
  if (block_size != PKV_BLOCK_SIZE)
    return fail(PKV_EUNSUPPORTED, "pkv_copy_blocks: block_size must be 16");
  if (num_pairs < 0 || num_blocks <= 0 || num_kv_heads <= 0 || head_dim <= 0)
    return fail(PKV_EINVAL, "pkv_copy_blocks: bad sizes");
  const int64_t block_bytes = (int64_t)block_size * num_kv_heads * head_dim * pkv::elem_size(dt);
  if (block_bytes % 16 != 0)
    return fail(PKV_EUNSUPPORTED, "pkv_copy_blocks: block bytes must be a multiple of 16");
  if (num_pairs == 0) return PKV_OK;
  if (!key_cache || !value_cache || !pairs) return fail(PKV_EINVAL, "pkv_copy_blocks: null pointer");
  if (!pkv::aligned16(key_cache) || !pkv::aligned16(value_cache))
    return fail(PKV_EINVAL, "pkv_copy_blocks: caches must be 16-byte aligned");
  if (num_pairs > 2147483647 / 2) return fail(PKV_EINVAL, "pkv_copy_blocks: too many pairs");
  return pkv::launched(pkv::launch_copy_blocks(key_cache, value_cache, pairs, num_pairs, num_blocks,
                                               block_bytes, stream),
                       "pkv_copy_blocks");
}

int pkv_swap_blocks(void* dst_key_cache, void* dst_value_cache, const void* src_key_cache,
                    const void* src_value_cache, const int32_t* pairs, int32_t num_pairs,
                    int32_t src_num_blocks, int32_t dst_num_blocks, int32_t block_size,
                    int32_t num_kv_heads, int32_t head_dim, pkv_dtype dt, void* stream) {
  if (!pkv::dtype_ok(dt)) return fail(PKV_EUNSUPPORTED, "pkv_swap_blocks: unsupported dtype");
  if (block_size != PKV_BLOCK_SIZE)
    return fail(PKV_EUNSUPPORTED, "pkv_swap_blocks: block_size must be 16");
  if (num_pairs < 0 || src_num_blocks <= 0 || dst_num_blocks <= 0 || num_kv_heads <= 0 || head_dim <= 0)
    return fail(PKV_EINVAL, "pkv_swap_blocks: bad sizes");
  const int64_t block_bytes = (int64_t)block_size * num_kv_heads * head_dim * pkv::elem_size(dt);
  if (block_bytes % 16 != 0)
    return fail(PKV_EUNSUPPORTED, "pkv_swap_blocks: block bytes must be a multiple of 16");
  if (num_pairs == 0) return PKV_OK;
  if (!dst_key_cache || !dst_value_cache || !src_key_cache || !src_value_cache || !pairs)
    return fail(PKV_EINVAL, "pkv_swap_blocks: null pointer");
  if (num_pairs > 2147483647 / 2 || num_pairs > 65535 * 1024)
    return fail(PKV_EINVAL, "pkv_swap_blocks: too many pairs");
  void* dk = nullptr; void* dv = nullptr; void* sk = nullptr; void* sv = nullptr;
  const int64_t dst_bytes = (int64_t)dst_num_blocks * block_bytes;
  const int64_t src_bytes = (int64_t)src_num_blocks * block_bytes;
  if (!pkv::device_span(dst_key_cache, dst_bytes, &dk) || !pkv::device_span(dst_value_cache, dst_bytes, &dv) ||
      !pkv::device_span(src_key_cache, src_bytes, &sk) || !pkv::device_span(src_value_cache, src_bytes, &sv))
    return fail(PKV_EINVAL,
                "pkv_swap_blocks: each pool must be device memory or page-locked host memory mapped for "
                "the device, covering num_blocks blocks");
  if (!pkv::device_readable(pairs, (int64_t)num_pairs * 2 * sizeof(int32_t)))
    return fail(PKV_EINVAL, "pkv_swap_blocks: pairs must be device memory");
  if (!pkv::aligned16(dk) || !pkv::aligned16(dv) || !pkv::aligned16(sk) || !pkv::aligned16(sv))
    return fail(PKV_EINVAL, "pkv_swap_blocks: pools must be 16-byte aligned");
  return pkv::launched(pkv::launch_swap_blocks(dk, dv, sk, sv, pairs, num_pairs, src_num_blocks,
                                               dst_num_blocks, block_bytes, stream),
                       "pkv_swap_blocks");
}

int pkv_check_pool(const void* pool, size_t bytes) {
  void* d = nullptr;
  if (!pool || bytes == 0 || bytes > (size_t)INT64_MAX) return fail(PKV_EINVAL, "pkv_check_pool: bad arguments");
  if (!pkv::device_span(pool, (int64_t)bytes, &d))
    return fail(PKV_EINVAL, "pkv_check_pool: not device memory or mapped page-locked host memory of that size");
  return PKV_OK;
}

int pkv_check_tables(const int32_t* host_block_tables, const int32_t* host_context_lens,
                     int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks) {
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || num_blocks <= 0)
    return fail(PKV_EINVAL, "pkv_check_tables: bad sizes");
  if (num_seqs > 0 && (!host_block_tables || !host_context_lens))
    return fail(PKV_EINVAL, "pkv_check_tables: null pointer");
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t n = host_context_lens[s];
    if (n < 0 || n > (int64_t)max_blocks_per_seq * PKV_BLOCK_SIZE)
      return fail(PKV_EINVAL, "pkv_check_tables: context length out of range");
    const int64_t nb = (n + PKV_BLOCK_SIZE - 1) / PKV_BLOCK_SIZE;
    const int32_t* row = host_block_tables + (int64_t)s * max_blocks_per_seq;
    for (int64_t b = 0; b < nb; ++b) {
      if (row[b] < 0 || row[b] >= num_blocks) return fail(PKV_EINVAL, "pkv_check_tables: block id out of range");
    }
  }
  return PKV_OK;
}

int pkv_check_slots(const int32_t* host_slot_mapping, int32_t num_tokens, int32_t num_blocks,
                    int32_t block_size) {
  if (num_tokens < 0 || num_blocks <= 0 || block_size != PKV_BLOCK_SIZE)
    return fail(PKV_EINVAL, "pkv_check_slots: bad sizes");
  if (num_tokens > 0 && !host_slot_mapping) return fail(PKV_EINVAL, "pkv_check_slots: null pointer");
  const int64_t nslots = (int64_t)num_blocks * block_size;
  std::vector<uint8_t> seen((size_t)nslots, 0);
  for (int32_t i = 0; i < num_tokens; ++i) {
    const int32_t s = host_slot_mapping[i];
    if (s < 0) continue;
    if (s >= nslots) return fail(PKV_EINVAL, "pkv_check_slots: slot beyond the pool");
    if (seen[(size_t)s]) return fail(PKV_EINVAL, "pkv_check_slots: duplicate slot (write race)");
    seen[(size_t)s] = 1;
  }
  return PKV_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// One decode step captured into a HIP graph: the launches of pkv_write +
// pkv_attention_decode (or of pkv_attention_decode_append) recorded once on a
// private stream and replayed with one hipGraphLaunch.

struct pkv_graph {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};

extern "C" {

int pkv_decode_graph_create(pkv_graph** graph_out, void* out, const void* q, const void* k_new,
                            const void* v_new, const int32_t* slot_mapping, int32_t num_new_tokens,
                            void* key_cache, void* value_cache, const int32_t* block_tables,
                            const int32_t* context_lens, float scale, int32_t block_size,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t num_seqs,
                            int32_t max_blocks_per_seq, int32_t num_blocks, int32_t max_context_len,
                            pkv_dtype dt, void* workspace, size_t workspace_bytes) {
  const char* who = "pkv_decode_graph_create";
  if (!graph_out) return fail(PKV_EINVAL, "pkv_decode_graph_create: null graph_out");
  *graph_out = nullptr;
  if (num_seqs <= 0) return fail(PKV_EINVAL, "pkv_decode_graph_create: num_seqs must be > 0");
  const bool append_form = slot_mapping == nullptr;
  if (append_form && dt != PKV_BF16)
    return fail(PKV_EUNSUPPORTED, "pkv_decode_graph_create: the append form (no slot_mapping) is bf16 only");
  if (!append_form && num_new_tokens < 0) return fail(PKV_EINVAL, "pkv_decode_graph_create: bad num_new_tokens");
  // Validate everything with a dry run of the same checks the launches make.
  {
    pkv::DecodeArgs a{};
    const int rc = prepare_attention(who, a, out, q, key_cache, value_cache, block_tables, context_lens,
                                     nullptr, num_seqs, 1, scale, block_size, num_q_heads, num_kv_heads,
                                     head_dim, num_seqs, max_blocks_per_seq, num_blocks, max_context_len, dt,
                                     workspace, workspace_bytes);
    if (rc != PKV_OK) return rc;
    if (append_form && (!k_new || !v_new || !pkv::aligned16(k_new) || !pkv::aligned16(v_new)))
      return fail(PKV_EINVAL, "pkv_decode_graph_create: k_new / v_new null or misaligned");
  }
  pkv_graph* g = new (std::nothrow) pkv_graph();
  if (!g) return fail(PKV_ENOMEM, "pkv_decode_graph_create: out of host memory");
  hipStream_t s = nullptr;
  if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) {
    delete g;
    return fail(PKV_ELAUNCH, "pkv_decode_graph_create: hipStreamCreateWithFlags failed");
  }
  int rc = PKV_OK;
  if (hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal) != hipSuccess) {
    rc = fail(PKV_ELAUNCH, "pkv_decode_graph_create: hipStreamBeginCapture failed");
  } else {
    if (append_form) {
      rc = pkv_attention_decode_append(out, q, k_new, v_new, key_cache, value_cache, block_tables, context_lens,
                                       scale, block_size, num_q_heads, num_kv_heads, head_dim, num_seqs,
                                       max_blocks_per_seq, num_blocks, max_context_len, dt, workspace,
                                       workspace_bytes, s);
    } else {
      if (num_new_tokens > 0)
        rc = pkv_write(key_cache, value_cache, k_new, v_new, slot_mapping, num_new_tokens, num_blocks,
                       block_size, num_kv_heads, head_dim, dt, s);
      if (rc == PKV_OK)
        rc = pkv_attention_decode(out, q, key_cache, value_cache, block_tables, context_lens, scale, block_size,
                                  num_q_heads, num_kv_heads, head_dim, num_seqs, max_blocks_per_seq, num_blocks,
                                  max_context_len, dt, workspace, workspace_bytes, s);
    }
    const hipError_t end = hipStreamEndCapture(s, &g->graph);
    if (rc == PKV_OK && end != hipSuccess)
      rc = fail(PKV_ELAUNCH, "pkv_decode_graph_create: hipStreamEndCapture failed");
  }
  if (rc == PKV_OK && hipGraphInstantiateWithFlags(&g->exec, g->graph, 0) != hipSuccess)
    rc = fail(PKV_ELAUNCH, "pkv_decode_graph_create: hipGraphInstantiate failed");
  (void)hipStreamDestroy(s);
  if (rc != PKV_OK) {
    pkv_decode_graph_destroy(g);
    return rc;
  }
  *graph_out = g;
  return PKV_OK;
}

int pkv_decode_graph_launch(pkv_graph* g, void* stream) {
  if (!g || !g->exec) return fail(PKV_EINVAL, "pkv_decode_graph_launch: null graph");
  const hipError_t e = hipGraphLaunch(g->exec, (hipStream_t)stream);
  if (e != hipSuccess) return pkv::launched((int)e, "pkv_decode_graph_launch");
  return PKV_OK;
}

void pkv_decode_graph_destroy(pkv_graph* g) {
  if (!g) return;
  if (g->exec) (void)hipGraphExecDestroy(g->exec);
  if (g->graph) (void)hipGraphDestroy(g->graph);
  delete g;
}

}  // extern "C"
