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
// Unlike a decode row, a chunk's rows make a real dense tile.  A workgroup takes
// a work item of 256/G consecutive rows x the G q heads of one KV head over one
// partition of keys; each of its four waves owns 64/G rows = four 16-column
// MFMA tiles (column n of tile c = row c*16/G + n/G, head n%G).  Each
// 16-token block of K and V is loaded once per workgroup (coalesced 16-byte
// pieces, a few blocks in flight in registers), staged through a double-buffered
// LDS slab with padded rows, and read by every wave as the K operand (A of
// v_mfma_f32_16x16x32_bf16, token = lane & 15) and the V^T operand (A of
// v_mfma_f32_16x16x16bf16_1k, regrouped by 16-bit permutes), each used by all
// four of the wave's tiles; the score tile's lane layout is the P^T operand of
// the value product, as in the decode kernel.  Each column keeps its own
// online softmax and causal mask (token < the keys its row sees), so the
// diagonal block needs no special case.
//
// Workgroups take tickets from the prefill counter (a ticket names a work
// record and a KV head).  A row whose keys fit one partition gets its output
// written directly; other rows' partials go to the workspace for the merge.

#include <hip/hip_runtime.h>

#include <algorithm>

#include "../pkv_internal.hpp"
#include "decode_common.hpp"

#ifndef PKV_PREFILL_NBUF
#define PKV_PREFILL_NBUF 4
#endif

namespace pkv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kPrefillNbuf = PKV_PREFILL_NBUF;  // blocks in flight per workgroup
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
  constexpr int EPL = D / 16;            // dims per lane in one V row piece
  constexpr int WPL = EPL / 2;           // 32-bit words per V row piece
  constexpr int NKC = D / 32;            // 16x16x32 MFMAs per tile per block for the scores
  constexpr int R = 16 / G;              // rows per tile
  constexpr int RPW = kTiles * R;        // rows per wave
  constexpr int NPF = kPrefillNbuf;      // blocks in flight (cooperative loads)
  constexpr int RS = D * 2 + 16;         // LDS row stride in bytes (16-byte pad: no bank conflicts)
  using VT = typename VPiece<D>::T;
  static_assert(G >= 1 && G <= 16 && 16 % G == 0, "a tile holds whole rows of G heads");
  static_assert(kDecodeThreads == kBlockTokens * 16, "16 threads per token row load a block");

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n = lane & 15;               // MFMA column (row n / G, head n % G of a tile)
  const int j = lane >> 4;
  const int Hq = p.Hkv * G;
  const int64_t tok_bytes = (int64_t)p.Hkv * D * 2;
  const int64_t blk_bytes = tok_bytes * kBlockTokens;
  const int total = min(p.sched[3], p.pre_cap * p.Hkv);

  // [buffer][K, V][16 rows x RS bytes]
  __shared__ __attribute__((aligned(16))) char s_kv[2][2][kBlockTokens * RS];
  __shared__ int s_ticket[2];

  struct Item {
    int s, part, g, ctx, qrow0, nrows, key0, b_begin, nblk, ids;
  };
  auto make_item = [&](int tk, Item& it) {
    const int4 ra = p.pre_recs[2 * (tk / p.Hkv)];
    const int4 rb = p.pre_recs[2 * (tk / p.Hkv) + 1];
    it.g = tk % p.Hkv;
    it.s = ra.x;
    it.part = ra.y;
    it.ctx = ra.z;
    it.qrow0 = ra.w;
    it.nrows = rb.x;
    it.key0 = rb.y;                                      // row i sees max(0, key0 + i) keys
    const int key_last = max(0, it.key0 + it.nrows - 1);  // keys the item's last row sees
    const int k_begin = it.part * kPartTokens;
    const int k_end = min(k_begin + kPartTokens, key_last);
    it.b_begin = it.part * kPartBlocks;
    it.nblk = max(0, (k_end - k_begin + kBlockTokens - 1) / kBlockTokens);
    it.ids = lane < it.nblk ? p.tables[(int64_t)it.s * p.MB + it.b_begin + lane] : -1;
  };

  // q operands (B of the score MFMAs) of this wave's rows: tile c, column n =
  // row wave*RPW + c*R + n/G of the item, head n%G
  bf16x8 qf[kTiles][NKC];
  auto load_q = [&](const Item& it) {
#pragma unroll
    for (int c = 0; c < kTiles; ++c) {
      const int r = wave * RPW + c * R + n / G;
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

  // cooperative block loads: thread t loads the same piece of K and of V, row
  // t / 16 of the block, bytes (t % 16) * PS .. + PS of KV head g's slice
  // (PS = D / 8: one coalesced 16-lane row per token), so every load uses one
  // resource and the pipeline needs no per-thread selection
  constexpr int PS = D / 8;
  const int st_row = tid / 16;
  const int st_col = (tid % 16) * PS;
  struct Stage {
    VT k, v;
  };
  auto issue = [&](const Item& it, int k, Stage& st) {
    const int pb = k < it.nblk ? __builtin_amdgcn_readlane(it.ids, k) : -1;
    const bool ok = (unsigned)pb < (unsigned)p.NB;
    const int64_t base = (int64_t)(ok ? pb : 0) * blk_bytes;
    const int nrec = ok ? (int)blk_bytes : 0;
    const __amdgpu_buffer_rsrc_t kr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p.kc + base), (short)0, nrec, kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p.vc + base), (short)0, nrec, kRawBufferWord3);
    const int off = (int)(st_row * tok_bytes + it.g * D * 2 + st_col);
    st.k = buffer_load_piece<VT>(kr, off, 0);
    st.v = buffer_load_piece<VT>(vr, off, 0);
  };
  auto stage_to_lds = [&](const Stage& st, int buf) {
    *reinterpret_cast<VT*>(&s_kv[buf][0][st_row * RS + st_col]) = st.k;
    *reinterpret_cast<VT*>(&s_kv[buf][1][st_row * RS + st_col]) = st.v;
  };

  float m[kTiles], l[kTiles];
  f32x4 acc[kTiles][EPL];
  int col_keys[kTiles];  // keys the column's row sees (0 for a column past the item's rows)

  // one block from LDS buffer buf: tokens t0 .. t0+15, of which `valid` are in the context
  auto compute = [&](int buf, int t0, int valid) {
    const char* kb = s_kv[buf][0];
    const char* vb = s_kv[buf][1];
    uint4 kf[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) kf[kc] = *reinterpret_cast<const uint4*>(kb + n * RS + 64 * kc + 16 * j);
    VT vp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      vp[i] = *reinterpret_cast<const VT*>(vb + (4 * j + i) * RS + EPL * 2 * n);
      if (4 * j + i >= valid) vp[i] = VT{};  // past the context: zero (0 * NaN)
    }
    const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vp[0]);
    const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vp[1]);
    const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vp[2]);
    const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vp[3]);
    i16x4 av[EPL];  // V^T operand tiles, shared by the four column tiles
#pragma unroll
    for (int w = 0; w < WPL; ++w) {
      av[2 * w] = __builtin_bit_cast(i16x4, make_uint2(pair_lo(w0[w], w1[w]), pair_lo(w2[w], w3[w])));
      av[2 * w + 1] = __builtin_bit_cast(i16x4, make_uint2(pair_hi(w0[w], w1[w]), pair_hi(w2[w], w3[w])));
    }
    // In phases over the four tiles, so independent tiles overlap: scores,
    // block maxima, one rescale decision, probabilities, value products.
    f32x4 sc[kTiles];
#pragma unroll
    for (int c = 0; c < kTiles; ++c) sc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
#pragma unroll
      for (int c = 0; c < kTiles; ++c)
        sc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[kc]), qf[c][kc],
                                                        sc[c], 0, 0, 0);
    }
    float x[kTiles][4], ms[kTiles];
    bool grew = false;
#pragma unroll
    for (int c = 0; c < kTiles; ++c) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 4 * j + i;
        x[c][i] = t < col_keys[c] ? sc[c][i] * p.scale_log2 : -INFINITY;
      }
      const float mb = max_over_rows(fmaxf(fmaxf(x[c][0], x[c][1]), fmaxf(x[c][2], x[c][3])));
      const bool up = mb > m[c] + kRescaleLog2;  // -inf + 8 = -inf: the first live block moves it
      const float mn = up ? mb : m[c];
      ms[c] = (mn == -INFINITY) ? 0.f : mn;
      grew |= up;
      x[c][0] -= ms[c];
      x[c][1] -= ms[c];
      x[c][2] -= ms[c];
      x[c][3] -= ms[c];
      const float old = m[c];
      m[c] = mn;
      ms[c] = old - ms[c];  // exponent of the rescale factor
    }
    if (__ballot(grew)) {  // some column's reference moved: rescale what was accumulated
#pragma unroll
      for (int c = 0; c < kTiles; ++c) {
        const float alpha = exp2_fast(ms[c]);
        l[c] *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[c][e] *= alpha;
      }
    }
    i16x4 pt[kTiles];
#pragma unroll
    for (int c = 0; c < kTiles; ++c) {
      const uint32_t p01 = pack_bf16x2(exp2_fast(x[c][0]), exp2_fast(x[c][1]));
      const uint32_t p23 = pack_bf16x2(exp2_fast(x[c][2]), exp2_fast(x[c][3]));
      l[c] += (bf16_lo(p01) + bf16_hi(p01)) + (bf16_lo(p23) + bf16_hi(p23));
      pt[c] = __builtin_bit_cast(i16x4, make_uint2(p01, p23));
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
#pragma unroll
      for (int c = 0; c < kTiles; ++c)
        acc[c][e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av[e], pt[c], acc[c][e], 0, 0, 0);
    }
  };

  if (tid == 0) s_ticket[0] = atomicAdd(&p.sched[2], 1);
  __syncthreads();
  int tk = __builtin_amdgcn_readfirstlane(s_ticket[0]);

  Stage stg[NPF];
  int buf = 0;
  for (int parity = 1; tk < total; parity ^= 1) {
    int next_tk = 0;
    if (tid == 0) next_tk = atomicAdd(&p.sched[2], 1);
    Item it;
    make_item(tk, it);
    load_q(it);
#pragma unroll
    for (int u = 0; u < NPF; ++u) issue(it, u, stg[u]);
#pragma unroll
    for (int c = 0; c < kTiles; ++c) {
      m[c] = -INFINITY;
      l[c] = 0.f;
      const int r = wave * RPW + c * R + n / G;
      col_keys[c] = r < it.nrows ? max(0, it.key0 + r) : 0;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[c][e] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // Blocks in rounds of NPF: block k's staged registers go to LDS buffer
    // k % 2, the slot is refilled with block k + NPF (a zero-range load past the
    // item), one barrier makes the block visible, and every wave computes it.
    // Two LDS buffers suffice: a wave writing buffer k % 2 has passed block
    // k-1's barrier, which every wave reached after computing block k-2.
    const int rounds = (it.nblk + NPF - 1) / NPF;
    for (int rr = 0; rr < rounds; ++rr) {
#pragma unroll
      for (int u = 0; u < NPF; ++u) {
        const int k = rr * NPF + u;
        const bool live = k < it.nblk;  // uniform over the workgroup
        if (live) stage_to_lds(stg[u], buf);
        issue(it, k + NPF, stg[u]);      // unconditional: the wait counts stay static
        if (live) {
          __syncthreads();
          const int t0 = (it.b_begin + k) * kBlockTokens;
          compute(buf, t0, min(kBlockTokens, it.ctx - t0));
          buf ^= 1;
        }
      }
    }

#pragma unroll
    for (int c = 0; c < kTiles; ++c) {
      const float lt = sum_over_rows(l[c]);
      const int r = wave * RPW + c * R + n / G;
      const int keys = max(0, it.key0 + r);
      const int nparts = max(1, (keys + kPartTokens - 1) / kPartTokens);
      // a row that ends before this partition has nothing here (its own items
      // cover its partitions); only partition 0 of a one-partition row is output
      if (r < it.nrows && it.part < nparts) {
        const int64_t orow = (int64_t)(it.qrow0 + r) * Hq + it.g * G + n % G;
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        if (nparts == 1) {
          uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + orow * D;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[EPL * (4 * j + i) + e] = f32_to_bf16(acc[c][e][i] * inv);
          }
        } else {
          const int64_t pr = orow * p.max_parts + it.part;
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
    if (tid == 0) s_ticket[parity] = next_tk;
    __syncthreads();
    tk = __builtin_amdgcn_readfirstlane(s_ticket[parity]);
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
  const int64_t items = (int64_t)a.pre_cap * a.num_kv_heads;  // upper bound
  const int64_t grid = std::min<int64_t>(items, (int64_t)a.num_cus * per_cu);
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
