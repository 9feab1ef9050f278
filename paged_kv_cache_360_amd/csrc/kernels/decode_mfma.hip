// bf16 split-context paged decode attention on the gfx950 matrix cores.
//
// What is computed is the same as the fp32 kernel (decode.hip): attention for one
// new token per sequence over K/V reached block by block through the block table,
// each block's contribution accumulated into a running softmax ("vLLM and
// PagedAttention", §2 "Reworking the Attention Computation"; cache layout
// [num_blocks, 16, num_kv_heads, head_dim] from the kernel sketch there).
//
// Why matrix cores for decode: one workgroup serves the G = Hq / Hkv query heads
// that share a KV head, so a 16-token block is a real 16 x G x head_dim product
// twice over (scores and weighted values).  On the vector ALUs the bf16 -> fp32
// widening, the 4·G·head_dim flops per token and the cross-lane dot-product
// reductions cost more issue slots than the HBM stream leaves; as MFMA operands
// bf16 is consumed as stored and no cross-lane reduction remains.
//
// Work decomposition: one persistent 4-wave workgroup per compute unit takes
// work items from the plan's list (ticket t = record t / Hkv, KV head t % Hkv);
// an item is one (sequence, KV head) over one or two consecutive 512-token
// partitions (partition p is tokens [512p, 512p + 512)).  Wave w takes the
// item's blocks w, w + 4, ... and keeps one online-softmax state for the whole
// item; the four waves' states merge through LDS into one partial result per
// item (the output itself when the item is the sequence's only one).
//
// Per 16-token block, one wave (lane = 16 j + h, h = lane & 15, j = lane >> 4):
//  scores  S[t][n] = sum_d K[t][d] q[n][d]  (v_mfma_f32_16x16x32_bf16, D/32 of
//          them).  A = K: lane (h, j) holds token h, dims 32c + 8j .. +7 -- one
//          16-byte load per chunk c, 64 contiguous bytes per token row per load.
//          B = q: lane (h, j) holds q head h at the same dims (zero for h >= G).
//          C: lane (h, j) holds tokens 4j .. 4j + 3 of head h.
//  softmax in base 2 per head h: block max over the lane's 4 tokens and the 4
//          lane groups; the running sum l is lane-local until the end.
//  values  O^T[d][n] += sum_t V[t][d] P[n][t]  (v_mfma_f32_16x16x16bf16_1k, D/8
//          of them).  B = P^T is exactly the score layout above, rounded to bf16.
//          A = V^T: lane (h, j) needs 4 tokens of one dim.  It loads tokens 4j+i
//          (i = 0..3) at dims EPL*h .. EPL*h + EPL-1 (EPL = D/16; one coalesced
//          row of 16 lanes per token) and regroups 16-bit halves of those four
//          rows with byte permutes, so tile e has row slot m <-> dim EPL*m + e.
//          C: lane (h, j), tile e, element i <-> head h, dim EPL*(4j + i) + e.
//
// Masking: tokens past the context in the last block get score -inf AND their V
// rows are zeroed before the product (0 * NaN would otherwise poison the
// accumulator), so NaN/Inf in unused slots never reaches the output.  Block ids
// outside [0, num_blocks) are not dereferenced; such a block counts as masked.
//
// Memory-level parallelism: each wave double-buffers two blocks (its KV head's
// K and V slices, 8 KiB at head_dim 128) in registers, issuing block i+1's
// loads before computing i.
// Loads go through per-block buffer resources (base = the block, range = its
// size): the lane offsets are 32-bit, and a block that must not be read gets a
// zero range, so the prefetch needs no branch.  Block loads carry the
// nontemporal hint, as each (block, KV head) slice is read once per launch,
// unless the plan finds sequences sharing their first block (a shared prefix):
// their blocks are read by several items, and the hint would evict them
// between those reads.

#include <hip/hip_runtime.h>

#include <algorithm>

#include "../pkv_internal.hpp"
#include "decode_common.hpp"

namespace pkv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Blocks each wave keeps in flight, and the occupancy the register budget is
// sized for (waves per SIMD).
constexpr int kMfmaPipelineDepth = 2;
constexpr int kMfmaWavesPerSimd = 2;
// Persistent workgroups per compute unit (capped by what fits).  Fewer, deeper
// pipelined workgroups keep the same bytes in flight and finish each item
// sooner, which shortens the end-of-run tail of the ticket schedule.
constexpr int kMfmaWgPerCu = 1;
// Threads per workgroup: the waves of a workgroup split each item's blocks.
constexpr int kMfmaThreads = 256;

// One lane's share of a V row load: head_dim / 16 bf16 values.
template <int D> struct VPiece;
template <> struct VPiece<128> { using T = uint4; };
template <> struct VPiece<64> { using T = uint2; };

// 16-bit halves of two words: (low(a), low(b)) and (high(a), high(b)).
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) {
  return (a & 0xFFFFu) | (b << 16);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xFFFF0000u);
}

// Per-lane choice between two register pieces.
__device__ __forceinline__ uint4 pick(bool t, uint4 a, uint4 b) {
  return make_uint4(t ? a.x : b.x, t ? a.y : b.y, t ? a.z : b.z, t ? a.w : b.w);
}
__device__ __forceinline__ uint2 pick(bool t, uint2 a, uint2 b) {
  return make_uint2(t ? a.x : b.x, t ? a.y : b.y);
}

// Two fp32 values to a packed bf16 pair (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Persistent partition kernel: each workgroup takes tickets from the counter
// until none are left.  After the last block of an item each wave already holds
// the next item's record (its ticket was passed through LDS at the previous
// item's barrier and its record loaded right after), so it issues that item's
// first blocks before the barrier.  The cross-wave merge of an item runs inside
// the next item's block loop, where its LDS reads and output stores overlap
// with loads in flight.  LDS state is double-buffered by item parity: item
// i+1's state is written while item i's is still being merged.
//
// Nothing at an item boundary waits for the block loads in flight: records
// come in on the scalar path, the block ids and the ticket land in registers
// that only loads and the atomic write, and the ticket is consumed while only
// the zero-sized tail loads are outstanding (vector memory operations complete
// in order, so any earlier wait would drain the prefetch).
//
// kPolicy is the cache policy of the block loads (the kernel below picks it
// per launch).
template <int D, int G, int kPolicy>
__device__ __forceinline__ void decode_partition_body(const DecodeParams& p) {
  constexpr int EPL = D / 16;            // dims per lane in one V row load
  constexpr int WPL = EPL / 2;           // 32-bit words per V row load
  constexpr int NKC = D / 32;            // 16x16x32 MFMAs per block for the scores
  constexpr int NWAVE = kMfmaThreads / kWave;
  constexpr int NBUF = kMfmaPipelineDepth;
  using VT = typename VPiece<D>::T;
  static_assert(G >= 1 && G <= 16, "the q heads of one KV head fill at most 16 MFMA columns");
  static_assert(kPartBlocks % NWAVE == 0 && kLongItemParts * kPartBlocks / NWAVE <= kWave,
                "each wave holds its block ids of an item in one register");

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int h = lane & 15;
  const int j = lane >> 4;
  const int Hq = p.Hkv * G;
  const int64_t tok_bytes = (int64_t)p.Hkv * D * 2;
  const int64_t blk_bytes = tok_bytes * kBlockTokens;
  // tickets of this launch, bounded by the work-list capacity
  const int total = min(p.sched[1], p.dec_cap * p.Hkv);

  // One work item as this wave sees it.
  struct Item {
    int s, part, g, ctx, b_begin, nmine;  // part: first of the item's partitions
    bool whole;                            // the sequence's only item: its result is the output
    int slot;                              // else the item's partial: its slot in the row
    int64_t row0;       // first q head (row of q / out) of the KV head group
    int my_id;          // lane k < nmine: id of the wave's k-th block
    int k_lane, v_lane; // this lane's byte offsets inside a block
    // Append form: the wave's block k_new holds the sequence's new token (row
    // new_row); k_new < 0: not this wave's, or no append.
    int k_new, new_row;
  };
  // This lane's pieces of the new token's K and V rows in the block-load layout
  // (append form), for the current item and the next one.
  uint4 kn_cur[NKC], kn_nxt[NKC];
  VT vn_cur, vn_nxt;
  // Record of ticket tk.  The records are written by the plan launch and only
  // read here, so they are read through the constant address space: with tk
  // wave-uniform that is a scalar load, and waiting for it does not wait for
  // the vector loads in flight (vector loads complete in order, so a record
  // fetched with one would drain the block prefetch at every item).
  auto load_rec = [&](int tk) {
    const __attribute__((address_space(4))) int* r =
        (const __attribute__((address_space(4))) int*)(const void*)p.dec_recs + 4 * (tk / p.Hkv);
    return make_int4(r[0], r[1], r[2], r[3]);
  };
  auto make_item = [&](int tk, int4 r, Item& it) {
    it.g = tk % p.Hkv;
    it.s = r.x;
    it.part = r.y & kPartitionMask;
    it.ctx = r.z;
    it.whole = (r.y & kWholeSequence) != 0;
    {
      // slots: the full items in order, then the pieces of the last item
      const int nparts = max(1, (it.ctx + kPartTokens - 1) / kPartTokens);
      const int ip = item_parts(nparts);
      const int full_end = (nparts + ip - 1) / ip * ip - ip;
      it.slot = it.part < full_end ? it.part / ip : full_end / ip + (it.part - full_end);
    }
    const int nblk = (it.ctx + kBlockTokens - 1) / kBlockTokens;
    it.b_begin = it.part * kPartBlocks;
    const int in_item = min((r.y & kOnePartition) ? kPartBlocks : item_parts((it.ctx + kPartTokens - 1) / kPartTokens) * kPartBlocks,
                            nblk - it.b_begin);
    it.nmine = max(0, (in_item - wave + NWAVE - 1) / NWAVE);
    it.row0 = (int64_t)r.w * Hq + (int64_t)it.g * G;  // r.w: the sequence's query row
    it.k_lane = (int)(h * tok_bytes + (it.g * D + 8 * j) * 2);
    it.v_lane = (int)(4 * j * tok_bytes + (it.g * D + EPL * h) * 2);
    it.k_new = -1;
    it.new_row = 0;
    if (p.knew != nullptr && it.ctx >= 1 && (r.y & kAppendable)) {
      // (a context clamped to the workspace bound has no new token to append;
      // the plan leaves kAppendable out of its records)
      const int bn = (it.ctx - 1) / kBlockTokens - it.b_begin;  // item-relative block
      if (bn >= 0 && bn < in_item && bn % NWAVE == wave) {
        it.k_new = bn / NWAVE;
        it.new_row = (it.ctx - 1) % kBlockTokens;
      }
    }
  };
  // ids of the wave's blocks b_begin + wave + NWAVE*k, one per lane (a vector
  // load through a resource over the sequence's table row; lanes past the row
  // read 0).  Only lanes k < nmine are ever used, so the load needs no branch,
  // and its register is written by loads alone, which complete in order: a
  // conditional default value would make the compiler wait for every load in
  // flight before overwriting it.
  auto load_ids = [&](Item& it) {
    const __amdgpu_buffer_rsrc_t tr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int32_t*>(p.tables + (int64_t)it.s * p.MB), (short)0, p.MB * 4, kRawBufferWord3);
    it.my_id = (int)__builtin_amdgcn_raw_buffer_load_b32(tr, (it.b_begin + wave + NWAVE * lane) * 4, 0, 0);
    // The new token's K/V pieces (append form), loaded with the ids through
    // resources that are empty unless this wave holds the token's block.
    const int nrec = it.k_new >= 0 ? D * 2 : 0;
    const int64_t nrow = nrec ? ((int64_t)it.s * p.Hkv + it.g) * D * 2 : 0;
    const __amdgpu_buffer_rsrc_t knr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p.knew + nrow), (short)0, nrec, kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t vnr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p.vnew + nrow), (short)0, nrec, kRawBufferWord3);
#pragma unroll
    for (int c = 0; c < NKC; ++c) kn_nxt[c] = buffer_load16(knr, 16 * j + 64 * c, 0);
    vn_nxt = buffer_load_piece<VT>(vnr, EPL * h * 2, 0);
  };

  // q as the B operand of the score MFMAs.  The resource covers the group's G
  // rows; lanes of columns h >= G point past it and read zeros (no branch).
  bf16x8 qf[NKC];
  auto load_q = [&](const Item& it) {
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(reinterpret_cast<const char*>(p.q) + it.row0 * D * 2), (short)0, G * D * 2,
        kRawBufferWord3);
    const int off = h < G ? (h * D + 8 * j) * 2 : G * D * 2;
#pragma unroll
    for (int c = 0; c < NKC; ++c) qf[c] = __builtin_bit_cast(bf16x8, buffer_load16(qr, off + 64 * c, 0));
  };

  struct Blk {
    uint4 k[NKC];
    VT v[4];
    int valid;
  };

  // Loads of the wave's k-th block of an item through buffer resources sized to
  // the block: k past the wave's share or an id outside the pool gets a
  // zero-sized resource, so its loads return zeros without touching memory and
  // the prefetch of later blocks needs no branch.
  auto issue = [&](const Item& it, int k, Blk& B) {
    const int pb = k < it.nmine ? __builtin_amdgcn_readlane(it.my_id, k) : -1;
    const bool ok = (unsigned)pb < (unsigned)p.NB;
    const int b = it.b_begin + wave + NWAVE * k;
    B.valid = ok ? min(kBlockTokens, it.ctx - b * kBlockTokens) : 0;
    const int64_t base = (int64_t)(ok ? pb : 0) * blk_bytes;
    const int nrec = ok ? (int)blk_bytes : 0;
    const __amdgpu_buffer_rsrc_t kr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p.kc + base), (short)0, nrec, kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p.vc + base), (short)0, nrec, kRawBufferWord3);
#pragma unroll
    for (int c = 0; c < NKC; ++c) B.k[c] = buffer_load16<kPolicy>(kr, it.k_lane + 64 * c, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) B.v[i] = buffer_load_piece<VT, kPolicy>(vr, it.v_lane, i * tok_bytes);
  };

  float m, l;            // reference max of head h (log2 domain, uniform over j); this lane's sum
  f32x4 acc[EPL];

  // Append form, the wave's k-th block of the current item holding the new
  // token: that token's cache row is not written yet, so its K and V come from
  // the inputs (the lanes of its row in the block-load layout), and those lanes
  // write the row to the cache.  No other work item reads this (token, KV head)
  // row.
  auto append = [&](Blk& B, const Item& it, int k) {
    const int pb = __builtin_amdgcn_readlane(it.my_id, k);
    if ((unsigned)pb >= (unsigned)p.NB) return;  // block id outside the pool: nothing read or written
    const int64_t base = (int64_t)pb * blk_bytes;
    const int row = it.new_row;
    const bool krow = h == row;
    // V: lane (h, j) holds tokens 4j .. 4j+3; the new token is its piece i = row & 3
    // when j == row / 4.  Per-lane selects keep the block in registers.
    const int vsel = j == (row >> 2) ? (row & 3) : -1;
#pragma unroll
    for (int c = 0; c < NKC; ++c) B.k[c] = pick(krow, kn_cur[c], B.k[c]);
#pragma unroll
    for (int i = 0; i < 4; ++i) B.v[i] = pick(i == vsel, vn_cur, B.v[i]);
    if (krow) {
#pragma unroll
      for (int c = 0; c < NKC; ++c)
        *reinterpret_cast<uint4*>(const_cast<char*>(p.kc) + base + it.k_lane + 64 * c) = kn_cur[c];
    }
    if (vsel >= 0)
      *reinterpret_cast<VT*>(const_cast<char*>(p.vc) + base + it.v_lane + vsel * tok_bytes) = vn_cur;
  };

  auto compute = [&](Blk& B) {
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NKC; ++c)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, B.k[c]), qf[c], sc, 0, 0, 0);
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = sc[i] * p.scale_log2;
    if (B.valid < kBlockTokens) {  // last block of the context, or a skipped id
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (4 * j + i >= B.valid) {
          x[i] = -INFINITY;
          B.v[i] = VT{};
        }
      }
    }
    const float mb = max_over_rows(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
    const bool up = mb > m + kRescaleLog2;  // lazy reference max (-inf + 8 = -inf)
    const float mn = up ? mb : m;
    const float ms = (mn == -INFINITY) ? 0.f : mn;
    if (__ballot(up)) {  // some head's reference moved: rescale what was accumulated
      const float alpha = exp2_fast(m - ms);
      l *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] *= alpha;
    }
    m = mn;
    const uint32_t p01 = pack_bf16x2(exp2_fast(x[0] - ms), exp2_fast(x[1] - ms));
    const uint32_t p23 = pack_bf16x2(exp2_fast(x[2] - ms), exp2_fast(x[3] - ms));
    // the sum uses the rounded weights, so the result is an exact convex combination
    l += (bf16_lo(p01) + bf16_hi(p01)) + (bf16_lo(p23) + bf16_hi(p23));
    const i16x4 pt = __builtin_bit_cast(i16x4, make_uint2(p01, p23));

    const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&B.v[0]);
    const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&B.v[1]);
    const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&B.v[2]);
    const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&B.v[3]);
#pragma unroll
    for (int w = 0; w < WPL; ++w) {
      const i16x4 ae = __builtin_bit_cast(i16x4, make_uint2(pair_lo(w0[w], w1[w]), pair_lo(w2[w], w3[w])));
      const i16x4 ao = __builtin_bit_cast(i16x4, make_uint2(pair_hi(w0[w], w1[w]), pair_hi(w2[w], w3[w])));
      acc[2 * w] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ae, pt, acc[2 * w], 0, 0, 0);
      acc[2 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ao, pt, acc[2 * w + 1], 0, 0, 0);
    }
  };

  // [item parity][wave]
  __shared__ float s_m[2][NWAVE][G];
  __shared__ float s_l[2][NWAVE][G];
  __shared__ float s_o[2][NWAVE][G][D];
  __shared__ int s_ticket[2];  // by item parity

  // Tickets run two items ahead: while item i is computed the wave already
  // holds item i+1's record and block ids, and thread 0 is fetching ticket i+2.
  // Each workgroup's first two tickets are static (blockIdx.x and blockIdx.x +
  // gridDim.x); the counter hands out the rest, from 2 * gridDim.x on, so the
  // launch does not start with every workgroup queueing on one atomic.
  // The first record is loaded with the ticket count, not after it: its
  // index blockIdx.x / Hkv is below the list's capacity (the grid is at most
  // capacity x Hkv), and a workgroup past the count returns before using it.
  const int tk0 = blockIdx.x;
  const int4 rec0 = load_rec(tk0);
  if (tk0 >= total) return;
  int tk1 = blockIdx.x + gridDim.x;
  bool have1 = tk1 < total;

  // NBUF-deep software pipeline over an item's blocks: blocks k+1 .. k+NBUF-1
  // are in flight while block k is computed.  The trip count is rounded up to
  // whole rounds; the extra blocks have zero-sized resources and are fully
  // masked, so they leave the running state unchanged.
  Blk buf[NBUF];
  Item cur, nxt;
  make_item(tk0, rec0, cur);
  load_ids(cur);
#pragma unroll
  for (int c = 0; c < NKC; ++c) kn_cur[c] = kn_nxt[c];
  vn_cur = vn_nxt;
  load_q(cur);
#pragma unroll
  for (int u = 0; u < NBUF - 1; ++u) issue(cur, u, buf[u]);
  int4 rec1 = have1 ? load_rec(tk1) : make_int4(0, 0, 0, 0);

  // Cross-wave merge of a finished item whose wave states are in LDS half
  // `par`: per (head, dim), the four waves' states combined by log-sum-exp;
  // written to out (the sequence's only item) or to the item's partial: one
  // partial per item, whatever the number of partitions it covers (slot k for
  // the k-th full item, then one per piece of the last item).
  // Each thread takes G * D / 256 elements.
  auto merge = [&](const Item& it, int par) {
    for (int idx = threadIdx.x; idx < G * D; idx += kMfmaThreads) {
      const int hh = idx / D;
      const int d = idx % D;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NWAVE; ++w) M = fmaxf(M, s_m[par][w][hh]);
      float L = 0.f, O = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < NWAVE; ++w) {
          const float f = exp2_fast(s_m[par][w][hh] - M);
          L = fmaf(s_l[par][w][hh], f, L);
          O = fmaf(s_o[par][w][hh][d], f, O);
        }
      }
      const float r = L > 0.f ? O / L : 0.f;
      if (it.whole) {
        store_out<true>(p.out, (it.row0 + hh) * D + d, r);
      } else {
        const int64_t pr = (it.row0 + hh) * p.max_parts + it.slot;
        p.part_o[pr * D + d] = r;
        if (d == 0) {
          p.part_m[pr] = M;
          p.part_l[pr] = L;
        }
      }
    }
  };

  // The merge of item i runs inside item i+1's block loop, right after the
  // wave's first block: there its LDS reads and output stores overlap with the
  // loads in flight instead of holding the whole workgroup after the barrier.
  // Item i+1's closing barrier orders it before item i+2 reuses LDS half i%2.
  Item prev;
  bool pending = false;
  int parity = 0;
  for (;; parity ^= 1) {
    // The next item's record (loaded after the last barrier) is read after
    // this item's first block, not here: waiting for it here would leave only
    // the pre-issued first block of each wave in flight.
    bool nxt_ready = !have1;
    auto take_next = [&]() {
      if (!nxt_ready) {
        make_item(tk1, rec1, nxt);
        load_ids(nxt);
        nxt_ready = true;
      }
    };
    // (left unset in other lanes: like the ids, its register is written by the
    // atomic alone, so nothing waits for the loads in flight before it is issued)
    int fetched;
    if (threadIdx.x == 0) fetched = atomicAdd(&p.sched[0], 1);  // offset added where it is read

    // The wave's state over its blocks of the item goes to LDS at the end of
    // the item (the four waves' states meet at the barrier).
    auto reset = [&]() {
      m = -INFINITY;
      l = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
    };
    auto save = [&]() {
      const float lt = sum_over_rows(l);
      if (h < G) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int e = 0; e < EPL; ++e) s_o[parity][wave][h][EPL * (4 * j + i) + e] = acc[e][i];
        }
        if (j == 0) {
          s_m[parity][wave][h] = m;
          s_l[parity][wave][h] = lt;
        }
      }
    };
    reset();
    const int rounds = (cur.nmine + NBUF - 1) / NBUF;
    for (int r = 0; r < rounds; ++r) {
#pragma unroll
      for (int u = 0; u < NBUF; ++u) {
        const int k = r * NBUF + u;
        issue(cur, r * NBUF + u + NBUF - 1, buf[(u + NBUF - 1) % NBUF]);
        if (k == cur.k_new) append(buf[u], cur, k);  // uniform
        compute(buf[u]);
        if (u == 0 && r == 0) {
          take_next();
          if (pending) {
            merge(prev, parity ^ 1);
            pending = false;
          }
        }
      }
    }
    take_next();    // the wave had no block in this item
    if (pending) {
      merge(prev, parity ^ 1);
      pending = false;
    }
    // The ticket goes to LDS while only the zero-sized tail loads are in
    // flight: waiting for the atomic here waits for nothing else.
    if (threadIdx.x == 0) s_ticket[parity] = fetched;

    // The next item's q and first blocks go out before this item's merge.
    const Item done = cur;
    if (have1) {
      cur = nxt;
#pragma unroll
      for (int c = 0; c < NKC; ++c) kn_cur[c] = kn_nxt[c];
      vn_cur = vn_nxt;
      load_q(cur);
#pragma unroll
      for (int u = 0; u < NBUF - 1; ++u) issue(cur, u, buf[u]);
    }

    // the partition the wave ended in, and empty states for any it never reached
    save();
    __syncthreads();
    const int tk2 = 2 * (int)gridDim.x + __builtin_amdgcn_readfirstlane(s_ticket[parity]);
    const bool have2 = have1 && tk2 < total;
    const int4 rec2 = have2 ? load_rec(tk2) : make_int4(0, 0, 0, 0);

    prev = done;
    pending = true;
    if (!have1) break;
    tk1 = tk2;
    have1 = have2;
    rec1 = rec2;
  }
  merge(prev, parity);  // the last item (its closing barrier has passed)
}

// The block loads stream (nontemporal hint) unless the plan found decode
// sequences that share their first block (a shared prefix, a fork): then the
// launch keeps the default policy, so the shared blocks stay in the caches for
// their other readers.  (A per-item choice costs a branch at every block load,
// 5% on batches that share nothing.)
template <int D, int G>
__global__ __launch_bounds__(kMfmaThreads, kMfmaWavesPerSimd) void decode_partition_mfma_kernel(
    DecodeParams p) {
  if (p.sched[kSchedShared] != 0) {
    decode_partition_body<D, G, kCachedLoad>(p);
  } else {
    decode_partition_body<D, G, kStreamLoad>(p);
  }
}

template <int D, int G>
int launch_mfma_t(const DecodeParams& p, const DecodeArgs& a, hipStream_t st) {
  static int per_cu = 0;  // resident workgroups per CU for this instantiation (queried once)
  if (per_cu == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_partition_mfma_kernel<D, G>,
                                                     kMfmaThreads, 0) != hipSuccess || n < 1)
      n = 1;
    per_cu = n;
  }
  const int64_t items = (int64_t)a.dec_cap * a.num_kv_heads;  // upper bound
  const int64_t grid = std::min<int64_t>(items, (int64_t)a.num_cus * std::min(per_cu, kMfmaWgPerCu));
  hipLaunchKernelGGL((decode_partition_mfma_kernel<D, G>), dim3((unsigned)grid), dim3(kMfmaThreads),
                     0, st, p);
  return (int)hipGetLastError();
}

template <int D>
int launch_mfma_g(const DecodeParams& p, const DecodeArgs& a, hipStream_t st) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_mfma_t<D, 1>(p, a, st);
    case 2: return launch_mfma_t<D, 2>(p, a, st);
    case 4: return launch_mfma_t<D, 4>(p, a, st);
    case 8: return launch_mfma_t<D, 8>(p, a, st);
    default: return (int)hipErrorInvalidValue;
  }
}

}  // namespace

int launch_decode_partitions_bf16(const DecodeParams& p, const DecodeArgs& a, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  return a.head_dim == 64 ? launch_mfma_g<64>(p, a, st) : launch_mfma_g<128>(p, a, st);
}

}  // namespace pkv
