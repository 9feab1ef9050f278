// Work-list plan for the persistent attention kernels, built on the device from
// context_lens (and query_start_loc for variable-length batches), so the host
// never waits for the device.
//
// A sequence with one query row is a decode sequence; one with more rows is a
// chunked-prefill sequence whose rows sit at the end of its context: with q
// rows and ctx keys (the chunk's own tokens included), row r sees keys
// 0 .. ctx - q + r ("How vLLM Works?", section 04 on chunked prefill; the usual
// causal mask).  Keys are split into 512-token partitions merged by
// log-sum-exp.
//
// Outputs (all in the caller's workspace):
//  * decode records {sequence, first partition, context, query row}, one per
//    item_parts(n) consecutive partitions of a sequence of n partitions (four
//    when n >= kLongItemFrom, else two).  In front: every item but a sequence's
//    last, the four-partition ones first (items roughly in decreasing size),
//    and the only item of a sequence with one item when it has more than
//    kTailBlocks blocks.  Then the tail, in
//    decreasing block count (a counting sort over the kTailBlocks + 1 possible
//    counts): the other last items, where the last item of a sequence with
//    several items is split into one-partition records (first partition field
//    | kOnePartition) when it covers more than one partition, so that the
//    persistent run ends on items of at most one partition, the shortest last.
//    The field also carries kAppendable when the context length was not
//    clamped, and kWholeSequence on a sequence's only record;
//  * prefill records, two int4 each: {sequence, first partition, context, first
//    query row} and {rows, ctx - q + r0 + 1, span, 0} (row i of the group sees
//    max(0, that + i) keys; negative when the chunk is longer than the context);
//    one per (group of rows_per_item consecutive rows, run of `span` partitions
//    up to the one the group's last row reaches).  The span is 2 when halving
//    the item count still leaves every compute unit the same number of rounds
//    of items (then each row writes half the partial results), else 1;
//  * row_slots[T]: the partial results each query row's merge combines: for a
//    decode row, its record count when the partition kernel writes one partial
//    per record (bf16, on the matrix cores), else its partition count (fp32);
//    its item count (partitions / span, rounded up) for a prefill row; 1 for a
//    row written directly (or with no keys), 0 for rows no sequence owns;
//  * sched: both ticket counters reset, each list's ticket count (records
//    times KV heads: ticket t is record t / Hkv, KV head t % Hkv), and
//    sched[kSchedShared]: whether some decode sequence's first block is also
//    another decode sequence's first block (found through a hash table in LDS
//    over the first entry of each table row; a hint for the partition launch's
//    load cache policy only).
// One workgroup; per-thread counts are scanned with lane shuffles and one
// exchange of wave totals in LDS.

#include <hip/hip_runtime.h>

#include <algorithm>

#include "../pkv_internal.hpp"
#include "decode_common.hpp"

namespace pkv {

namespace {

// Open-addressing table of first block ids in LDS: a slot holds an id and how
// many decode sequences start with it.
constexpr int kShareSlots = 4096;
constexpr int kShareProbes = 16;
constexpr int32_t kShareEmpty = INT32_MIN;
__device__ __forceinline__ int share_hash(int32_t id) {
  return (int)(((uint32_t)id * 2654435761u) >> 20) & (kShareSlots - 1);
}

__device__ __forceinline__ void plan_body(
    const int32_t* __restrict__ ctx, const int32_t* __restrict__ qsl, int32_t S, int32_t T,
    int32_t ctx_cap, int32_t Hkv, int32_t rows_per_item, int32_t dec_cap, int32_t pre_cap,
    int32_t num_cus, int32_t* __restrict__ sched, int4* __restrict__ dec, int4* __restrict__ pre,
    int32_t* __restrict__ row_slots, bool record_slots, const int32_t* __restrict__ tab, int32_t MB) {
  constexpr int kTailBlocks = 2 * kPartBlocks;  // largest record sorted into the tail
  constexpr int NBK = kTailBlocks + 1;          // buckets: tail-record block count kTailBlocks .. 0
  __shared__ int32_t s_wsum[kPlanThreads / kWave][4];  // per wave: full items, prefill records at span 1, 2
  __shared__ int32_t s_wpre[kPlanThreads / kWave][4];  // the same summed over the waves before it
  __shared__ int32_t s_tot[3];                          // prefill records at span 1, 2 over all waves
  __shared__ int32_t s_bucket[NBK];
  __shared__ int32_t s_key[kShareSlots];
  __shared__ int32_t s_cnt[kShareSlots];
  __shared__ int32_t s_shared_any;
  const int t = threadIdx.x;
  const int per = (S + kPlanThreads - 1) / kPlanThreads;
  const int s0 = min(S, t * per);
  const int s1 = min(S, s0 + per);

  auto clamp_ctx = [&](int raw) { return max(0, min(raw, ctx_cap)); };
  auto row0_from = [&](int s, int qs) { return qsl ? min(max(qs, 0), T) : s; };
  auto rows_from = [&](int row0, int qe) { return qsl ? max(0, min(qe, T) - row0) : 1; };
  auto ctx_of = [&](int s) { return clamp_ctx(ctx[s]); };
  auto parts_of = [&](int keys) { return max(1, (keys + kPartTokens - 1) / kPartTokens); };
  auto first_row = [&](int s) { return row0_from(s, qsl ? qsl[s] : 0); };
  auto rows_of = [&](int s) { return rows_from(first_row(s), qsl ? qsl[s + 1] : 0); };
  auto items_of = [&](int n) { return (n + item_parts(n) - 1) / item_parts(n); };
  auto last_blocks = [&](int c, int n) {  // blocks of the last item: a full item's when full, 0 when empty
    return (c + kBlockTokens - 1) / kBlockTokens - (items_of(n) - 1) * item_parts(n) * kPartBlocks;
  };
  auto bucket_of = [&](int blocks) { return kTailBlocks - blocks; };
  // prefill: the keys seen by row r of a sequence with q rows and c keys
  auto row_keys_of = [&](int c, int q, int r) { return max(0, c - q + r + 1); };

  if (t < NBK) s_bucket[t] = 0;
  for (int r = t; r < T; r += kPlanThreads) row_slots[r] = 0;  // rows no sequence owns: nothing to merge
  for (int k = t; k < kShareSlots; k += kPlanThreads) {
    s_key[k] = kShareEmpty;
    s_cnt[k] = 0;
  }
  if (t == 0) s_shared_any = 0;
  __syncthreads();
  // first block id of a decode sequence with keys (a hint only: any value is
  // safe, it is never dereferenced here)
  auto first_block = [&](int s) { return (tab && MB > 0) ? tab[(int64_t)s * MB] : kShareEmpty; };
  auto share_insert = [&](int32_t id) {
    if (id == kShareEmpty) return;
    int h = share_hash(id);
    for (int k = 0; k < kShareProbes; ++k, h = (h + 1) & (kShareSlots - 1)) {
      const int32_t prev = atomicCAS(&s_key[h], kShareEmpty, id);
      if (prev == kShareEmpty || prev == id) {
        atomicAdd(&s_cnt[h], 1);
        return;
      }
    }
  };
  // after the inserts: does another decode sequence start with this id?  (A
  // probe run that found no slot counts as shared: the cached policy is the
  // safe default.)
  auto share_count = [&](int32_t id) {
    if (id == kShareEmpty) return 1;
    int h = share_hash(id);
    for (int k = 0; k < kShareProbes; ++k, h = (h + 1) & (kShareSlots - 1)) {
      const int32_t key = s_key[h];
      if (key == id) return s_cnt[h];
      if (key == kShareEmpty) return 1;
    }
    return 2;
  };
  // front records: two-partition items (and only items above kTailBlocks),
  // four-partition items; prefill records at span 1 and 2
  int full = 0, npre = 0, npre2 = 0, flong = 0;
  int own_c = 0, own_q = 0, own_row0 = 0, own_raw = 0;  // this thread's (last) sequence, for the write loop
  int32_t own_b0 = kShareEmpty;
  for (int s = s0; s < s1; ++s) {
    // the sequence's length, query rows and first table entry read at once,
    // each exactly once: from host memory, every read that waited on another
    // would add a round trip over the link
    // (an absent array's read goes to the length instead, so that all four
    // loads issue unconditionally, back to back)
    const bool has_tab = tab != nullptr && MB > 0;
    const int32_t* p_b0 = has_tab ? tab + (int64_t)s * MB : ctx + s;
    const int32_t* p_qs = qsl ? qsl + s : ctx + s;
    const int32_t* p_qe = qsl ? qsl + s + 1 : ctx + s;
    const int32_t v_b0 = *p_b0, raw = ctx[s], v_qs = *p_qs, v_qe = *p_qe;
    const int32_t b0 = has_tab ? v_b0 : kShareEmpty;
    const int qs = qsl ? v_qs : 0;
    const int qe = qsl ? v_qe : 0;
    const int c = clamp_ctx(raw);
    const int row0 = row0_from(s, qs);
    const int q = rows_from(row0, qe);
    own_raw = raw;
    own_c = c;
    own_q = q;
    own_row0 = row0;
    own_b0 = (q == 1 && c > 0) ? b0 : kShareEmpty;
    share_insert(own_b0);
    if (q == 1) {
      const int n = parts_of(c);
      const int ni = items_of(n);
      const int lb = last_blocks(c, n);
      if (ni == 1) {                 // the sequence's only record
        if (lb > kTailBlocks) ++full; else atomicAdd(&s_bucket[bucket_of(lb)], 1);
      } else {
        if (item_parts(n) == kLongItemParts) flong += ni - 1; else full += ni - 1;
        if (lb > kPartBlocks) {      // the last item in one-partition pieces
          for (int b = lb; b > 0; b -= kPartBlocks) atomicAdd(&s_bucket[bucket_of(min(b, kPartBlocks))], 1);
        } else {
          atomicAdd(&s_bucket[bucket_of(lb)], 1);
        }
      }
    } else if (q > 1) {
      for (int r0 = 0; r0 < q; r0 += rows_per_item) {
        const int n = parts_of(row_keys_of(c, q, min(q, r0 + rows_per_item) - 1));
        npre += n;
        npre2 += (n + 1) / 2;
      }
    }
  }
  // Inclusive scans of (full, npre, npre2, flong) over the workgroup: within each
  // wave by lane shuffles, then across the waves' totals by wave 0 (through LDS).
  constexpr int NWV = kPlanThreads / kWave;
  const int lane = t & (kWave - 1);
  const int wv = t / kWave;
  int inc_f = full, inc_p = npre, inc_p2 = npre2, inc_l = flong;
  for (int off = 1; off < kWave; off <<= 1) {
    const int vf = __shfl_up(inc_f, off, kWave);
    const int vp = __shfl_up(inc_p, off, kWave);
    const int vp2 = __shfl_up(inc_p2, off, kWave);
    const int vl = __shfl_up(inc_l, off, kWave);
    if (lane >= off) {
      inc_f += vf;
      inc_p += vp;
      inc_p2 += vp2;
      inc_l += vl;
    }
  }
  if (lane == kWave - 1) {
    s_wsum[wv][0] = inc_f;
    s_wsum[wv][1] = inc_p;
    s_wsum[wv][2] = inc_p2;
    s_wsum[wv][3] = inc_l;
  }
  __syncthreads();  // (also orders the bucket counts and the first-block table of the loop above)
  // While wave 0 scans: does another decode sequence start with this thread's
  // sequence's first block?
  const bool own_shared = per == 1 && share_count(own_b0) > 1;
  if (own_shared) s_shared_any = 1;
  if (wv == 0) {
    // The waves' totals: an exclusive scan over lanes 0 .. NWV-1 (one lane per
    // wave); the last lane holds the grand totals.
    static_assert(NWV <= kWave, "one lane per wave");
    const int a0 = lane < NWV ? s_wsum[lane][0] : 0;
    const int a1 = lane < NWV ? s_wsum[lane][1] : 0;
    const int a2 = lane < NWV ? s_wsum[lane][2] : 0;
    const int a3 = lane < NWV ? s_wsum[lane][3] : 0;
    int i0 = a0, i1 = a1, i2 = a2, i3 = a3;
    for (int off = 1; off < kWave; off <<= 1) {
      const int v0 = __shfl_up(i0, off, kWave);
      const int v1 = __shfl_up(i1, off, kWave);
      const int v2 = __shfl_up(i2, off, kWave);
      const int v3 = __shfl_up(i3, off, kWave);
      if (lane >= off) {
        i0 += v0;
        i1 += v1;
        i2 += v2;
        i3 += v3;
      }
    }
    if (lane < NWV) {
      s_wpre[lane][0] = i0 - a0;
      s_wpre[lane][1] = i1 - a1;
      s_wpre[lane][2] = i2 - a2;
      s_wpre[lane][3] = i3 - a3;
    }
    const int full_total = __shfl(i0, kWave - 1, kWave) + __shfl(i3, kWave - 1, kWave);
    if (lane == kWave - 1) {
      s_tot[0] = i1;
      s_tot[1] = i2;
      s_tot[2] = i3;
    }
    // bucket start offsets in the decode tail region: a lane-parallel scan
    static_assert(NBK == kWave + 1, "one bucket per lane plus the empty-item bucket");
    const int c = s_bucket[lane];
    int inc = c;
    for (int off = 1; off < kWave; off <<= 1) {
      const int v = __shfl_up(inc, off, kWave);
      if (lane >= off) inc += v;
    }
    s_bucket[lane] = full_total + inc - c;
    if (lane == kWave - 1) s_bucket[kWave] = full_total + inc;
  }
  __syncthreads();
  inc_f += s_wpre[wv][0];
  inc_p += s_wpre[wv][1];
  inc_p2 += s_wpre[wv][2];
  inc_l += s_wpre[wv][3];
  const int tot_p = s_tot[0], tot_p2 = s_tot[1], tot_l = s_tot[2];
  // Prefill span: rounds of items per compute unit (one workgroup each) at
  // span 1 and 2; span 2 when its rounds, each twice as long, take no longer.
  const int64_t cus = max(1, num_cus);
  const int64_t rounds1 = ((int64_t)tot_p * Hkv + cus - 1) / cus;
  const int64_t rounds2 = ((int64_t)tot_p2 * Hkv + cus - 1) / cus;
  const int span = (rounds1 > 1 && 2 * rounds2 <= rounds1) ? 2 : 1;
  const int num_pre = span == 2 ? tot_p2 : tot_p;

  // Writes.  Decode sequences (at most a few records each): every thread writes
  // its own.  Prefill sequences (hundreds of rows and records each): the wave
  // takes them one at a time, in each owner's order, and all 64 lanes write.
  int od = tot_l + inc_f - full;   // the two-partition front records after all four-partition ones
  int odl = inc_l - flong;
  for (int s = s0; s < s1; ++s) {
    const int c = per == 1 ? own_c : ctx_of(s);
    const int q = per == 1 ? own_q : rows_of(s);
    if (q != 1) continue;
    const int row0 = per == 1 ? own_row0 : first_row(s);
    const int app = (per == 1 ? own_raw : ctx[s]) == c ? kAppendable : 0;
    if (per > 1 && share_count(c > 0 ? first_block(s) : kShareEmpty) > 1) s_shared_any = 1;
    const int n = parts_of(c);
    const int ni = items_of(n);
    const bool lng = item_parts(n) == kLongItemParts;
    for (int k = 0; k < ni - 1; ++k) {
      const int at = lng ? odl++ : od++;
      if (at < dec_cap) dec[at] = make_int4(s, (k * item_parts(n)) | app, c, row0);
    }
    const int lb = last_blocks(c, n);
    const int p0 = (ni - 1) * item_parts(n);
    int recs = ni;
    if (ni == 1) {
      const int4 rec = make_int4(s, p0 | app | kWholeSequence, c, row0);
      if (lb > kTailBlocks) {
        if (od < dec_cap) dec[od] = rec;
        ++od;
      } else {
        const int at = atomicAdd(&s_bucket[bucket_of(lb)], 1);
        if (at < dec_cap) dec[at] = rec;
      }
    } else if (lb > kPartBlocks) {
      int j = 0;
      for (int b = lb; b > 0; b -= kPartBlocks, ++j) {
        const int at = atomicAdd(&s_bucket[bucket_of(min(b, kPartBlocks))], 1);
        if (at < dec_cap) dec[at] = make_int4(s, (p0 + j) | kOnePartition | app, c, row0);
      }
      recs = ni - 1 + j;
    } else {
      const int at = atomicAdd(&s_bucket[bucket_of(lb)], 1);
      if (at < dec_cap) dec[at] = make_int4(s, p0 | app, c, row0);
    }
    row_slots[row0] = record_slots ? recs : n;
  }
  auto next_prefill = [&](int from) {
    for (int s = from; s < s1; ++s)
      if ((per == 1 ? own_q : rows_of(s)) > 1) return s;
    return s1;
  };
  int op = span == 2 ? inc_p2 - npre2 : inc_p - npre;
  int ps = next_prefill(s0);
  for (;;) {
    const unsigned long long pending = __ballot(ps < s1);
    if (pending == 0) break;
    const int src = __ffsll(pending) - 1;
    const int s = __shfl(ps, src, kWave);
    int cop = __shfl(op, src, kWave);
    // with one sequence per thread, the owner lane's values from the first
    // loop (no second read of host memory)
    const int c = per == 1 ? __shfl(own_c, src, kWave) : ctx_of(s);
    const int q = per == 1 ? __shfl(own_q, src, kWave) : rows_of(s);
    const int row0 = per == 1 ? __shfl(own_row0, src, kWave) : first_row(s);
    for (int r0 = 0; r0 < q; r0 += rows_per_item) {
      const int nr = min(q, r0 + rows_per_item) - r0;
      const int n = (parts_of(row_keys_of(c, q, r0 + nr - 1)) + span - 1) / span;
      for (int k = lane; k < n; k += kWave) {
        if (cop + k < pre_cap) {
          pre[2 * (cop + k)] = make_int4(s, k * span, c, row0 + r0);
          // unclamped: row i of the group sees max(0, this + i) keys
          pre[2 * (cop + k) + 1] = make_int4(nr, c - q + r0 + 1, span, 0);
        }
      }
      cop += n;
    }
    for (int r = lane; r < q; r += kWave) row_slots[row0 + r] = (parts_of(row_keys_of(c, q, r)) + span - 1) / span;
    if (lane == src) {
      op = cop;
      ps = next_prefill(ps + 1);
    }
  }
  __syncthreads();
  if (t == 0) {
    // every bucket cursor has advanced past its records: the last one ends the list
    const int num_dec_recs = s_bucket[NBK - 1];
    sched[0] = 0;
    sched[1] = min(num_dec_recs, dec_cap) * Hkv;
    sched[2] = 0;
    sched[3] = min(num_pre, pre_cap) * Hkv;
    sched[kSchedShared] = s_shared_any;
  }
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(
    const int32_t* __restrict__ ctx, const int32_t* __restrict__ qsl, int32_t S, int32_t T,
    int32_t ctx_cap, int32_t Hkv, int32_t rows_per_item, int32_t dec_cap, int32_t pre_cap,
    int32_t num_cus, int32_t* __restrict__ sched, int4* __restrict__ dec, int4* __restrict__ pre,
    int32_t* __restrict__ row_slots, bool record_slots, const int32_t* __restrict__ tab, int32_t MB) {
  plan_body(ctx, qsl, S, T, ctx_cap, Hkv, rows_per_item, dec_cap, pre_cap, num_cus, sched, dec, pre, row_slots,
            record_slots, tab, MB);
}

// Loads in flight per thread in the staging copy (reads cross the host link).
constexpr int kUploadBatch = 4;
constexpr int kMergeRowsPerBlock = kPlanThreads / kWave;

// The plan of a step whose metadata is still in page-locked host memory, fused
// with the copy of that metadata to the device and, optionally, with the
// log-sum-exp merge of the previous step's partials.  Workgroup 0 builds the
// work list from the host copy of the context lengths (read through its device
// mapping); workgroups 1 .. n_up copy n16 16-byte words from src (host) to dst
// (device); the next ones copy, one table row per wave, the entries of each
// sequence's block-table row that its (clamped) context uses, from a host table
// to the device one (entries past them are never read, so they are not sent);
// the rest merge one row per wave.  One launch on the compute stream
// replaces a copy-engine transfer, a cross-stream wait and the merge launch:
// the three parts are latency-bound and overlap.  The previous step's partials
// and row counts live in another workspace than the one planned here.
template <bool BF16, int D>
__global__ __launch_bounds__(kPlanThreads) void upload_plan_kernel(
    const int32_t* __restrict__ host_ctx, const int32_t* __restrict__ qsl, int32_t S, int32_t T,
    int32_t ctx_cap, int32_t Hkv, int32_t rows_per_item, int32_t dec_cap, int32_t pre_cap, int32_t num_cus,
    int32_t* __restrict__ sched, int4* __restrict__ dec, int4* __restrict__ pre, int32_t* __restrict__ row_slots,
    const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t n16, int32_t n_up,
    const int32_t* __restrict__ host_tables, int32_t* __restrict__ tables, int32_t MB, int32_t n_tab,
    void* __restrict__ m_out, const float* __restrict__ m_pm, const float* __restrict__ m_pl,
    const float* __restrict__ m_po, const int32_t* __restrict__ m_counts, int32_t Hq, int32_t m_max_parts,
    int64_t m_rows) {
  if (blockIdx.x == 0) {
    // first entries of the table rows: from the host copy when this launch
    // uploads the tables, else from the device tables as they are
    plan_body(host_ctx, qsl, S, T, ctx_cap, Hkv, rows_per_item, dec_cap, pre_cap, num_cus, sched, dec, pre,
              row_slots, BF16, host_tables ? host_tables : tables, MB);
    return;
  }
  if ((int)blockIdx.x <= n_up) {
    const int64_t stride = (int64_t)n_up * kPlanThreads;
    for (int64_t base = (int64_t)(blockIdx.x - 1) * kPlanThreads + threadIdx.x; base < n16;
         base += stride * kUploadBatch) {
      uint4 r[kUploadBatch];
#pragma unroll
      for (int u = 0; u < kUploadBatch; ++u)
        if (base + u * stride < n16) r[u] = src[base + u * stride];
#pragma unroll
      for (int u = 0; u < kUploadBatch; ++u)
        if (base + u * stride < n16) dst[base + u * stride] = r[u];
    }
    return;
  }
  if ((int)blockIdx.x <= n_up + n_tab) {
    const int s = ((int)blockIdx.x - 1 - n_up) * kMergeRowsPerBlock + (int)threadIdx.x / kWave;
    if (s >= S) return;
    const int lane = threadIdx.x & (kWave - 1);
    const int c = max(0, min(host_ctx[s], ctx_cap));
    const int n = min((c + kBlockTokens - 1) / kBlockTokens, MB);
    const int32_t* from = host_tables + (int64_t)s * MB;
    int32_t* to = tables + (int64_t)s * MB;
    for (int base = lane; base < n; base += kWave * kUploadBatch) {
      int32_t r[kUploadBatch];
#pragma unroll
      for (int u = 0; u < kUploadBatch; ++u)
        if (base + u * kWave < n) r[u] = from[base + u * kWave];
#pragma unroll
      for (int u = 0; u < kUploadBatch; ++u)
        if (base + u * kWave < n) to[base + u * kWave] = r[u];
    }
    return;
  }
  const int64_t row = (int64_t)(blockIdx.x - 1 - n_up - n_tab) * kMergeRowsPerBlock + threadIdx.x / kWave;
  if (row < m_rows)
    merge_row<BF16, D, true>(row, threadIdx.x & (kWave - 1), m_out, m_pm, m_pl, m_po, m_counts, Hq, m_max_parts);
}

}  // namespace

int launch_plan(const DecodeArgs& a, void* stream) {
  // The fp32 decode kernel runs on a grid of (KV head, partition, sequence) and
  // reads no work list; the plan's only other output, the per-row partial
  // counts, feeds the merge, which has nothing to do when every row fits one
  // partition.
  if (!a.bf16 && a.qsl == nullptr && a.max_parts <= 1) return 0;
  const DecodeParams p = make_params(a);
  const int32_t G = a.num_q_heads / a.num_kv_heads;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, (hipStream_t)stream, a.ctx, a.qsl,
                     a.num_seqs, a.num_tokens, p.ctx_cap, a.num_kv_heads, prefill_rows_per_item(G),
                     a.dec_cap, a.pre_cap, a.num_cus, a.sched, reinterpret_cast<int4*>(a.dec_recs),
                     reinterpret_cast<int4*>(a.pre_recs), a.row_slots, a.bf16, a.tables, a.max_blocks);
  return (int)hipGetLastError();
}

int launch_upload_plan(const DecodeArgs& a, const int32_t* host_ctx, const void* src, void* dst,
                       int64_t bytes, const int32_t* host_tables, const DecodeArgs* prev, void* stream) {
  const DecodeParams p = make_params(a);
  const int64_t n16 = bytes / 16;
  // copy workgroups: enough 16-byte loads in flight to cover the host link's latency
  const int64_t per_wg = (int64_t)kPlanThreads * kUploadBatch;
  const int n_up = n16 > 0 ? (int)std::min<int64_t>((n16 + per_wg - 1) / per_wg, 256) : 0;
  // merge of the previous step: only rows spanning several partitions need it
  const bool merge = prev != nullptr && prev->max_parts > 1;
  const int64_t m_rows = merge ? (int64_t)prev->num_tokens * prev->num_q_heads : 0;
  const int64_t n_mg = (m_rows + kMergeRowsPerBlock - 1) / kMergeRowsPerBlock;
  const DecodeArgs& m = merge ? *prev : a;
  // table rows, one per wave
  const int n_tab = host_tables ? (a.num_seqs + kMergeRowsPerBlock - 1) / kMergeRowsPerBlock : 0;
  const dim3 grid((unsigned)(1 + n_up + n_tab + n_mg));
  const bool bf16 = merge ? prev->bf16 : a.bf16;
  const int D = merge ? prev->head_dim : a.head_dim;
#define PKV_UPLOAD_PLAN_LAUNCH(B, DD)                                                                   \
  hipLaunchKernelGGL((upload_plan_kernel<B, DD>), grid, dim3(kPlanThreads), 0, (hipStream_t)stream, host_ctx, \
                     a.qsl, a.num_seqs, a.num_tokens, p.ctx_cap, a.num_kv_heads,                          \
                     prefill_rows_per_item(a.num_q_heads / a.num_kv_heads), a.dec_cap, a.pre_cap, a.num_cus, \
                     a.sched, reinterpret_cast<int4*>(a.dec_recs), reinterpret_cast<int4*>(a.pre_recs),    \
                     a.row_slots, reinterpret_cast<const uint4*>(src),                                    \
                     reinterpret_cast<uint4*>(dst), n16, n_up, host_tables, const_cast<int32_t*>(a.tables), \
                     a.max_blocks, n_tab, m.out, m.part_m, m.part_l, m.part_o,                            \
                     m.row_slots, m.num_q_heads, m.max_parts, m_rows)
  if (bf16) {
    if (D == 64) PKV_UPLOAD_PLAN_LAUNCH(true, 64); else PKV_UPLOAD_PLAN_LAUNCH(true, 128);
  } else {
    if (D == 64) PKV_UPLOAD_PLAN_LAUNCH(false, 64); else PKV_UPLOAD_PLAN_LAUNCH(false, 128);
  }
#undef PKV_UPLOAD_PLAN_LAUNCH
  return (int)hipGetLastError();
}

}  // namespace pkv
