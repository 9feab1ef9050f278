// Chunked-prefill rows over the paged cache on the gfx950 matrix cores (bf16).
//
// A prefill chunk is a run of consecutive query rows at the end of a sequence's
// context, batched with decode rows ("How vLLM Works?", section 04 on chunked
// prefill; "vLLM and PagedAttention", key engineering optimizations); row r of
// a chunk of q rows over ctx keys sees keys 0 .. ctx - q + r (causal).  Keys
// are read block by block through the block table ("vLLM and PagedAttention",
// §2 "Reworking the Attention Computation"), split into 512-token partitions
// whose partial softmax results the log-sum-exp merge combines.
//
// Unlike a decode row, a chunk's rows make a real dense tile: one wavefront
// takes a work item of 64/G consecutive rows x the G q heads of one KV head =
// four 16-column MFMA tiles (column n of tile c = row c*16/G + n/G, head n%G),
// over one partition of keys.  Per 16-token block the K operand (A of
// v_mfma_f32_16x16x32_bf16, token = lane & 15) and the V^T operand (A of
// v_mfma_f32_16x16x16bf16_1k, regrouped from coalesced rows by 16-bit
// permutes) are loaded once and used by all four tiles; the score tile's lane
// layout is the P^T operand of the value product, as in the decode kernel.
// Each column keeps its own online softmax and causal mask (token < the keys
// its row sees), so the diagonal block needs no special case.
//
// The waves of a workgroup are independent: each takes tickets from the
// prefill counter (a ticket names a work record and a KV head), holds the next
// record while computing the current one, and issues the next item's q and
// first blocks before writing the current item's partials, so the memory
// pipeline does not drain between items.  A row whose keys fit one partition
// gets its output written directly; other rows' partials go to the workspace
// for the merge.

#include <hip/hip_runtime.h>

#include <algorithm>

#include "../pkv_internal.hpp"
#include "decode_common.hpp"

#ifndef PKV_PREFILL_NBUF
#define PKV_PREFILL_NBUF 2
#endif

namespace pkv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kPrefillNbuf = PKV_PREFILL_NBUF;  // blocks in flight per wave
constexpr int kTiles = 4;                        // 16-column MFMA tiles per work item

template <int D> struct VPiece;
template <> struct VPiece<128> { using T = uint4; };
template <> struct VPiece<64> { using T = uint2; };

__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

template <int D, int G>
__global__ __launch_bounds__(kDecodeThreads, 1) void prefill_mfma_kernel(DecodeParams p) {
  constexpr int EPL = D / 16;            // dims per lane in one V row load
  constexpr int WPL = EPL / 2;           // 32-bit words per V row load
  constexpr int NKC = D / 32;            // 16x16x32 MFMAs per tile per block for the scores
  constexpr int R = 16 / G;              // rows per tile
  constexpr int NBUF = kPrefillNbuf;
  using VT = typename VPiece<D>::T;
  static_assert(G >= 1 && G <= 16 && 16 % G == 0, "a tile holds whole rows of G heads");

  const int lane = threadIdx.x & (kWave - 1);
  const int n = lane & 15;               // MFMA column (row n / G, head n % G of a tile)
  const int j = lane >> 4;
  const int Hq = p.Hkv * G;
  const int64_t tok_bytes = (int64_t)p.Hkv * D * 2;
  const int64_t blk_bytes = tok_bytes * kBlockTokens;
  const int total = min(p.sched[3], p.pre_cap * p.Hkv);

  auto ticket = [&]() {  // one ticket per wave
    int t = 0;
    if (lane == 0) t = atomicAdd(&p.sched[2], 1);
    return __builtin_amdgcn_readfirstlane(t);
  };
  struct Rec {
    int4 a, b;  // {sequence, partition, context, first query row}, {rows, key0}: row i sees max(0, key0 + i)
  };
  auto load_rec = [&](int tk) {
    Rec r;
    r.a = p.pre_recs[2 * (tk / p.Hkv)];
    r.b = p.pre_recs[2 * (tk / p.Hkv) + 1];
    return r;
  };

  struct Item {
    int s, part, g, ctx, qrow0, nrows, key0, b_begin, nblk;
    int ids;             // lane k < nblk: physical id of the item's k-th block
    int k_lane, v_lane;
  };
  auto make_item = [&](int tk, const Rec& r, Item& it) {
    it.g = tk % p.Hkv;
    it.s = r.a.x;
    it.part = r.a.y;
    it.ctx = r.a.z;
    it.qrow0 = r.a.w;
    it.nrows = r.b.x;
    it.key0 = r.b.y;
    const int key_last = max(0, it.key0 + it.nrows - 1);  // keys the item's last row sees
    const int k_begin = it.part * kPartTokens;
    const int k_end = min(k_begin + kPartTokens, key_last);
    it.b_begin = it.part * kPartBlocks;
    it.nblk = max(0, (k_end - k_begin + kBlockTokens - 1) / kBlockTokens);
    it.ids = lane < it.nblk ? p.tables[(int64_t)it.s * p.MB + it.b_begin + lane] : -1;
    it.k_lane = (int)(n * tok_bytes + (it.g * D + 8 * j) * 2);
    it.v_lane = (int)(4 * j * tok_bytes + (it.g * D + EPL * n) * 2);
  };

  // q operands (B of the score MFMAs): tile c, column n = row c*R + n/G, head n%G
  bf16x8 qf[kTiles][NKC];
  auto load_q = [&](const Item& it) {
#pragma unroll
    for (int c = 0; c < kTiles; ++c) {
      const int r = c * R + n / G;
      const bool ok = r < it.nrows;
      const char* qrow = reinterpret_cast<const char*>(p.q) +
                         ((int64_t)(it.qrow0 + (ok ? r : 0)) * Hq + it.g * G + n % G) * D * 2;
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const uint4 v = ok ? load16(qrow + (32 * kc + 8 * j) * 2) : make_uint4(0, 0, 0, 0);
        qf[c][kc] = __builtin_bit_cast(bf16x8, v);
      }
    }
  };

  struct Blk {
    uint4 k[NKC];
    VT v[4];
    int valid;   // tokens of the block inside the context
    int t0;      // first token of the block
  };
  auto issue = [&](const Item& it, int k, Blk& B) {
    const int b = it.b_begin + k;
    const int pb = k < it.nblk ? __builtin_amdgcn_readlane(it.ids, k) : -1;
    const bool ok = (unsigned)pb < (unsigned)p.NB;
    B.t0 = b * kBlockTokens;
    B.valid = ok ? min(kBlockTokens, it.ctx - B.t0) : 0;
    const int64_t base = (int64_t)(ok ? pb : 0) * blk_bytes;
    const int nrec = ok ? (int)blk_bytes : 0;
    const __amdgpu_buffer_rsrc_t kr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p.kc + base), (short)0, nrec, kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p.vc + base), (short)0, nrec, kRawBufferWord3);
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) B.k[kc] = buffer_load16(kr, it.k_lane + 64 * kc, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) B.v[i] = buffer_load_piece<VT>(vr, it.v_lane, i * tok_bytes);
  };

  float m[kTiles], l[kTiles];
  f32x4 acc[kTiles][EPL];
  int col_keys[kTiles];  // keys the column's row sees (0 for a column past the item's rows)

  auto compute = [&](Blk& B) {
    if (B.valid < kBlockTokens) {  // tokens past the context: V rows to zero (0 * NaN)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * j + i >= B.valid) B.v[i] = VT{};
    }
    const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&B.v[0]);
    const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&B.v[1]);
    const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&B.v[2]);
    const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&B.v[3]);
    i16x4 av[EPL];  // V^T operand tiles, shared by the four column tiles
#pragma unroll
    for (int w = 0; w < WPL; ++w) {
      av[2 * w] = __builtin_bit_cast(i16x4, make_uint2(pair_lo(w0[w], w1[w]), pair_lo(w2[w], w3[w])));
      av[2 * w + 1] = __builtin_bit_cast(i16x4, make_uint2(pair_hi(w0[w], w1[w]), pair_hi(w2[w], w3[w])));
    }
#pragma unroll
    for (int c = 0; c < kTiles; ++c) {
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, B.k[kc]), qf[c][kc], sc,
                                                     0, 0, 0);
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = B.t0 + 4 * j + i;
        x[i] = t < col_keys[c] ? sc[i] * p.scale_log2 : -INFINITY;
      }
      float mb = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      mb = fmaxf(mb, __shfl_xor(mb, 16, kWave));
      mb = fmaxf(mb, __shfl_xor(mb, 32, kWave));
      const float mn = fmaxf(m[c], mb);
      const float ms = (mn == -INFINITY) ? 0.f : mn;
      if (__ballot(mn != m[c])) {
        const float alpha = exp2_fast(m[c] - ms);
        l[c] *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[c][e] *= alpha;
      }
      m[c] = mn;
      const uint32_t p01 = pack_bf16x2(exp2_fast(x[0] - ms), exp2_fast(x[1] - ms));
      const uint32_t p23 = pack_bf16x2(exp2_fast(x[2] - ms), exp2_fast(x[3] - ms));
      l[c] += (bf16_lo(p01) + bf16_hi(p01)) + (bf16_lo(p23) + bf16_hi(p23));
      const i16x4 pt = __builtin_bit_cast(i16x4, make_uint2(p01, p23));
#pragma unroll
      for (int e = 0; e < EPL; ++e)
        acc[c][e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av[e], pt, acc[c][e], 0, 0, 0);
    }
  };

  // per-wave ticket pipeline: the current and the next record are held
  int tk = ticket();
  int tk_next = ticket();
  if (tk >= total) return;
  Rec rec = load_rec(tk);
  Rec rec_next = tk_next < total ? load_rec(tk_next) : Rec{};

  Blk buf[NBUF];
  Item cur;
  make_item(tk, rec, cur);
  load_q(cur);
#pragma unroll
  for (int u = 0; u < NBUF - 1; ++u) issue(cur, u, buf[u]);

  for (;;) {
    const int tk_after = ticket();
#pragma unroll
    for (int c = 0; c < kTiles; ++c) {
      m[c] = -INFINITY;
      l[c] = 0.f;
      const int r = c * R + n / G;
      col_keys[c] = r < cur.nrows ? max(0, cur.key0 + r) : 0;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[c][e] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int rounds = (cur.nblk + NBUF - 1) / NBUF;
    for (int rr = 0; rr < rounds; ++rr) {
#pragma unroll
      for (int u = 0; u < NBUF; ++u) {
        issue(cur, rr * NBUF + u + NBUF - 1, buf[(u + NBUF - 1) % NBUF]);
        compute(buf[u]);
      }
    }

    // next item's q and first blocks before this item's writes
    const Item done = cur;
    const bool more = tk_next < total;
    if (more) {
      make_item(tk_next, rec_next, cur);
      load_q(cur);
#pragma unroll
      for (int u = 0; u < NBUF - 1; ++u) issue(cur, u, buf[u]);
    }

#pragma unroll
    for (int c = 0; c < kTiles; ++c) {
      float lt = l[c];
      lt += __shfl_xor(lt, 16, kWave);
      lt += __shfl_xor(lt, 32, kWave);
      const int r = c * R + n / G;
      const int keys = max(0, done.key0 + r);
      const int nparts = max(1, (keys + kPartTokens - 1) / kPartTokens);
      // a row that ends before this partition has nothing here (its own items
      // cover its partitions); only partition 0 of a one-partition row is output
      if (r < done.nrows && done.part < nparts) {
        const int64_t orow = (int64_t)(done.qrow0 + r) * Hq + done.g * G + n % G;
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        if (nparts == 1) {
          uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + orow * D;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[EPL * (4 * j + i) + e] = f32_to_bf16(acc[c][e][i] * inv);
          }
        } else {
          const int64_t pr = orow * p.max_parts + done.part;
          float* o = p.part_o + pr * D;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[EPL * (4 * j + i) + e] = acc[c][e][i] * inv;
          }
          if (j == 0) {
            p.part_m[pr] = m[c];
            p.part_l[pr] = lt;
          }
        }
      }
    }
    if (!more) break;
    tk_next = tk_after;
    rec_next = tk_next < total ? load_rec(tk_next) : Rec{};
  }
}

template <int D, int G>
int launch_prefill_t(const DecodeArgs& a, hipStream_t st) {
  const DecodeParams p = make_params(a);
  static int per_cu = 0;
  if (per_cu == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, prefill_mfma_kernel<D, G>, kDecodeThreads, 0) !=
            hipSuccess || nb < 1)
      nb = 1;
    per_cu = nb;
  }
  const int64_t waves = (int64_t)a.pre_cap * a.num_kv_heads;                    // upper bound on items
  const int64_t grid = std::min<int64_t>((waves + kDecodeWaves - 1) / kDecodeWaves,
                                         (int64_t)a.num_cus * per_cu);
  hipLaunchKernelGGL((prefill_mfma_kernel<D, G>), dim3((unsigned)std::max<int64_t>(grid, 1)),
                     dim3(kDecodeThreads), 0, st, p);
  return (int)hipGetLastError();
}

template <int D>
int launch_prefill_g(const DecodeArgs& a, hipStream_t st) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_prefill_t<D, 1>(a, st);
    case 2: return launch_prefill_t<D, 2>(a, st);
    case 4: return launch_prefill_t<D, 4>(a, st);
    case 8: return launch_prefill_t<D, 8>(a, st);
    default: return (int)hipErrorInvalidValue;
  }
}

}  // namespace

int launch_prefill(const DecodeArgs& a, void* stream) {
  if (a.pre_cap <= 0) return 0;  // no sequence has more than one query row
  hipStream_t st = (hipStream_t)stream;
  return a.head_dim == 64 ? launch_prefill_g<64>(a, st) : launch_prefill_g<128>(a, st);
}

}  // namespace pkv
