// fp32 split-context paged decode attention on the vector ALUs, and the
// log-sum-exp merge of partition results (both dtypes), for gfx950.  The bf16
// partition kernel runs on the matrix cores (decode_mfma.hip); fp32 stays here
// because fp32 data carries half the flops per byte and the vector ALUs keep up.
//
// Attention over K/V reached block by block through a block table, with each
// block's contribution computed separately and accumulated ("vLLM and
// PagedAttention", §2 "Reworking the Attention Computation"; cache layout from
// the kernel sketch there: [num_blocks, 16, num_kv_heads, head_dim]).
//
// Work decomposition (one workgroup = 4 wavefronts of 64 lanes):
//   grid = (kv head g, partition p, sequence s); partition p covers tokens
//   [512 p, 512 p + 512) of the sequence, i.e. 32 blocks.  The workgroup serves
//   all G = Hq / Hkv query heads of KV head g, so every K/V byte is read once.
//   Wave w takes blocks p*32 + w, + 4, + 8, ... and keeps its own online-softmax
//   state; the four waves merge through LDS at the end.
//
// Lane mapping for one 16-token block of one KV head (the slab is 16 rows of
// head_dim elements, rows num_kv_heads*head_dim apart): a token row is split
// over LPT lanes that each load 16 contiguous bytes (dwordx4), so one wave-wide
// load covers TPL = 64 / LPT whole rows and NL = 16 / TPL loads cover the block.
// For head_dim 128: 32 lanes x 16 B = one 512-B row, 2 rows per load, 8 loads per
// block for K and 8 for V.  The q.k dot product is a per-lane partial over 4
// dims followed by a butterfly sum across the row's lanes.
//
// Online softmax in base 2: q is pre-multiplied by scale*log2(e) so scores are
// log2-domain and every exponential is one v_exp_f32.  The running max m is
// uniform across the wave; the running sum l and the accumulator acc stay
// lane-local (each lane sums only its own tokens) and are reduced once at the end.
//
// Masking: tokens past the context in the last block get score -inf and their V
// values are replaced by 0 before the multiply, so NaN/Inf left in unused slots
// never reaches the output.  Block ids outside [0, num_blocks) are not
// dereferenced: such a block counts as fully masked.
//
// Memory-level parallelism: each wave double-buffers two blocks (K and V) in
// registers, issuing block i+1's loads before computing block i.

#include <hip/hip_runtime.h>

#include <algorithm>

#include "../pkv_internal.hpp"
#include "decode_common.hpp"

namespace pkv {

namespace {

template <int D, int G>
__global__ __launch_bounds__(kDecodeThreads) void decode_partition_kernel(DecodeParams p) {
  constexpr int ES = 4;                            // bytes per element (fp32)
  constexpr int EPL = 16 / ES;                     // elements per lane per load
  constexpr int LPT = D * ES / 16;                 // lanes per token row
  constexpr int TPL = kWave / LPT;                 // token rows per wave-wide load
  constexpr int NL = kBlockTokens / TPL;           // loads per block (per cache)
  constexpr int NW = kDecodeWaves;
  static_assert(LPT >= 1 && LPT <= kWave && kWave % LPT == 0, "row must split over lanes");
  static_assert(kBlockTokens % TPL == 0, "block must split over loads");

  const int g = blockIdx.x;
  const int part = blockIdx.y;
  const int s = blockIdx.z;
  const int Hq = p.Hkv * G;

  const int ctx = clamped_ctx(p, s);
  const int nparts = (ctx + kPartTokens - 1) / kPartTokens;
  if (part >= max(nparts, 1)) return;
  const int64_t row0 = (int64_t)s * Hq + (int64_t)g * G;  // first q head of this group

  if (ctx == 0) {  // empty context: zero output
    for (int i = threadIdx.x; i < G * D; i += kDecodeThreads) store_out<false>(p.out, row0 * D + i, 0.f);
    return;
  }

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int dim0 = (lane % LPT) * EPL;
  const int tl = lane / LPT;

  // q for this lane's dims, all G heads, scaled into the log2 domain.
  float qv[G][EPL];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const uint4 r = load16(reinterpret_cast<const char*>(p.q) + ((row0 + j) * D + dim0) * ES);
    widen16<false>(r, qv[j]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[j][e] *= p.scale_log2;
  }

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[j][e] = 0.f;
  }

  const int nblk = (ctx + kBlockTokens - 1) / kBlockTokens;
  const int b_begin = part * kPartBlocks;
  const int b_end = min(b_begin + kPartBlocks, nblk);
  const int32_t* trow = p.tables + (int64_t)s * p.MB;
  const int64_t tok_bytes = (int64_t)p.Hkv * D * ES;
  const int64_t blk_bytes = tok_bytes * kBlockTokens;
  const int64_t lane_off = (int64_t)tl * tok_bytes + ((int64_t)g * D + dim0) * ES;

  auto issue = [&](int b, uint4 (&kr)[NL], uint4 (&vr)[NL], int& valid) {
    const int pb = trow[b];
    const bool ok = (unsigned)pb < (unsigned)p.NB;
    valid = ok ? min(kBlockTokens, ctx - b * kBlockTokens) : 0;
    const int64_t base = (int64_t)(ok ? pb : 0) * blk_bytes + lane_off;
#pragma unroll
    for (int i = 0; i < NL; ++i) kr[i] = load16(p.kc + base + (int64_t)i * TPL * tok_bytes);
#pragma unroll
    for (int i = 0; i < NL; ++i) vr[i] = load16(p.vc + base + (int64_t)i * TPL * tok_bytes);
  };

  auto compute = [&](const uint4 (&kr)[NL], const uint4 (&vr)[NL], int valid) {
    float sc[NL][G];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      float kf[EPL];
      widen16<false>(kr[i], kf);
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) d = fmaf(qv[j][e], kf[e], d);
        sc[i][j] = xor_sum<1, LPT>(d);
      }
    }
    const bool partial = valid < kBlockTokens;
    if (partial) {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        if (i * TPL + tl >= valid) {
#pragma unroll
          for (int j = 0; j < G; ++j) sc[i][j] = -INFINITY;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float mb = sc[0][j];
#pragma unroll
      for (int i = 1; i < NL; ++i) mb = fmaxf(mb, sc[i][j]);
      mb = xor_max<LPT, kWave>(mb);
      const float mn = fmaxf(m[j], mb);
      const float ms = (mn == -INFINITY) ? 0.f : mn;
      const float alpha = exp2_fast(m[j] - ms);
      m[j] = mn;
      l[j] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[j][e] *= alpha;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        sc[i][j] = exp2_fast(sc[i][j] - ms);
        l[j] += sc[i][j];
      }
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      float vf[EPL];
      widen16<false>(vr[i], vf);
      if (partial && i * TPL + tl >= valid) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) vf[e] = 0.f;
      }
#pragma unroll
      for (int j = 0; j < G; ++j) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[j][e] = fmaf(sc[i][j], vf[e], acc[j][e]);
      }
    }
  };

  uint4 ka[NL], va[NL], kb[NL], vb[NL];
  int valid_a = 0, valid_b = 0;
  int b = b_begin + wave;
  if (b < b_end) issue(b, ka, va, valid_a);
  while (b < b_end) {
    int bn = b + NW;
    if (bn < b_end) issue(bn, kb, vb, valid_b);
    compute(ka, va, valid_a);
    b = bn;
    if (b >= b_end) break;
    bn = b + NW;
    if (bn < b_end) issue(bn, ka, va, valid_a);
    compute(kb, vb, valid_b);
    b = bn;
  }

  // Wave totals: sum l and acc over the TPL token groups (m is already uniform).
#pragma unroll
  for (int j = 0; j < G; ++j) {
    l[j] = xor_sum<LPT, kWave>(l[j]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[j][e] = xor_sum<LPT, kWave>(acc[j][e]);
  }

  __shared__ float s_m[NW][G];
  __shared__ float s_l[NW][G];
  __shared__ float s_o[NW][G][D];
  if (tl == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_o[wave][j][dim0 + e] = acc[j][e];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      s_m[wave][j] = m[j];
      s_l[wave][j] = l[j];
    }
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < G * D; idx += kDecodeThreads) {
    const int j = idx / D;
    const int d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][j]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = exp2_fast(s_m[w][j] - M);
        L = fmaf(s_l[w][j], f, L);
        O = fmaf(s_o[w][j][d], f, O);
      }
    }
    const float r = L > 0.f ? O / L : 0.f;
    if (nparts == 1) {
      store_out<false>(p.out, (row0 + j) * D + d, r);
    } else {
      const int64_t pr = (row0 + j) * p.max_parts + part;
      p.part_o[pr * D + d] = r;
      if (d == 0) {
        p.part_m[pr] = M;
        p.part_l[pr] = L;
      }
    }
  }
}

template <bool BF16, int D, bool PER_TOKEN>
__global__ __launch_bounds__(kWave) void lse_merge_kernel(
    void* __restrict__ out, const float* __restrict__ pm, const float* __restrict__ pl,
    const float* __restrict__ po, const int32_t* __restrict__ counts, int32_t Hq,
    int32_t max_parts) {
  merge_row<BF16, D, PER_TOKEN>(blockIdx.x, threadIdx.x, out, pm, pl, po, counts, Hq, max_parts);
}

template <int D, int G>
void launch_partitions_t(const DecodeParams& p, const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((decode_partition_kernel<D, G>),
                     dim3(a.num_kv_heads, a.max_parts, a.num_seqs), dim3(kDecodeThreads), 0, st, p);
}

template <int D>
int launch_partitions_g(const DecodeParams& p, const DecodeArgs& a, hipStream_t st) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: launch_partitions_t<D, 1>(p, a, st); break;
    case 2: launch_partitions_t<D, 2>(p, a, st); break;
    case 4: launch_partitions_t<D, 4>(p, a, st); break;
    case 8: launch_partitions_t<D, 8>(p, a, st); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

template <bool BF16, int D>
void launch_merge_t(const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((lse_merge_kernel<BF16, D, true>), dim3(a.num_tokens * a.num_q_heads), dim3(kWave),
                     0, st, a.out, a.part_m, a.part_l, a.part_o, a.row_slots, a.num_q_heads, a.max_parts);
}

}  // namespace

DecodeParams make_params(const DecodeArgs& a) {
  DecodeParams p;
  p.out = a.out;
  p.q = a.q;
  p.kc = reinterpret_cast<const char*>(a.kc);
  p.vc = reinterpret_cast<const char*>(a.vc);
  p.tables = a.tables;
  p.ctx = a.ctx;
  p.qsl = a.qsl;
  p.scale_log2 = a.scale_log2;
  p.num_seqs = a.num_seqs;
  p.num_tokens = a.num_tokens;
  p.Hkv = a.num_kv_heads;
  p.MB = a.max_blocks;
  p.NB = a.num_blocks;
  p.max_parts = a.max_parts;
  p.ctx_cap = std::min(a.max_blocks * kBlockTokens, a.max_parts * kPartTokens);
  p.sched = a.sched;
  p.dec_recs = reinterpret_cast<const int4*>(a.dec_recs);
  p.pre_recs = reinterpret_cast<const int4*>(a.pre_recs);
  p.row_slots = a.row_slots;
  p.dec_cap = a.dec_cap;
  p.pre_cap = a.pre_cap;
  p.part_m = a.part_m;
  p.part_l = a.part_l;
  p.part_o = a.part_o;
  p.knew = reinterpret_cast<const char*>(a.knew);
  p.vnew = reinterpret_cast<const char*>(a.vnew);
  return p;
}

int launch_decode_partitions(const DecodeArgs& a, void* stream) {
  const DecodeParams p = make_params(a);
  if (a.bf16) return launch_decode_partitions_bf16(p, a, stream);  // matrix cores
  hipStream_t st = (hipStream_t)stream;
  return a.head_dim == 64 ? launch_partitions_g<64>(p, a, st) : launch_partitions_g<128>(p, a, st);
}

int launch_decode_merge(const DecodeArgs& a, void* stream) {
  if (a.max_parts <= 1) return 0;  // every row fits one partition: nothing to merge
  hipStream_t st = (hipStream_t)stream;
  if (a.bf16) {
    if (a.head_dim == 64) launch_merge_t<true, 64>(a, st); else launch_merge_t<true, 128>(a, st);
  } else {
    if (a.head_dim == 64) launch_merge_t<false, 64>(a, st); else launch_merge_t<false, 128>(a, st);
  }
  return (int)hipGetLastError();
}

int launch_lse_merge(void* out, const float* part_m, const float* part_l, const float* part_o,
                     const int32_t* num_parts, int32_t rows, int32_t max_parts, int32_t head_dim,
                     bool bf16, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const dim3 grid(rows), block(kWave);
  if (bf16) {
    if (head_dim == 64)
      hipLaunchKernelGGL((lse_merge_kernel<true, 64, false>), grid, block, 0, st, out, part_m,
                         part_l, part_o, num_parts, 1, max_parts);
    else
      hipLaunchKernelGGL((lse_merge_kernel<true, 128, false>), grid, block, 0, st, out, part_m,
                         part_l, part_o, num_parts, 1, max_parts);
  } else {
    if (head_dim == 64)
      hipLaunchKernelGGL((lse_merge_kernel<false, 64, false>), grid, block, 0, st, out, part_m,
                         part_l, part_o, num_parts, 1, max_parts);
    else
      hipLaunchKernelGGL((lse_merge_kernel<false, 128, false>), grid, block, 0, st, out, part_m,
                         part_l, part_o, num_parts, 1, max_parts);
  }
  return (int)hipGetLastError();
}

}  // namespace pkv
