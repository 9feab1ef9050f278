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
// Work decomposition: grid = (KV head g, partition p, sequence s), 4 wavefronts;
// partition p is tokens [512p, 512p + 512).  Wave w takes blocks p*32 + w, + 4,
// ... and keeps its own online-softmax state; the four waves merge through LDS.
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
// Memory-level parallelism: each wave double-buffers two blocks (K and V, 8 KiB
// at head_dim 128) in registers, issuing block i+1's loads before computing i.
// Loads go through per-block buffer resources (base = the block, range = its
// size): the lane offsets are 32-bit, and a block that must not be read gets a
// zero range, so the prefetch needs no branch.

#include <hip/hip_runtime.h>

#include "../pkv_internal.hpp"
#include "decode_common.hpp"

#ifndef PKV_MFMA_NBUF
#define PKV_MFMA_NBUF 2
#endif
#ifndef PKV_MFMA_WAVES
#define PKV_MFMA_WAVES 3
#endif

namespace pkv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Blocks each wave keeps in flight, and the occupancy the register budget is
// sized for (waves per SIMD).
constexpr int kMfmaPipelineDepth = PKV_MFMA_NBUF;
constexpr int kMfmaWavesPerSimd = PKV_MFMA_WAVES;

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

// Two fp32 values to a packed bf16 pair (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

template <int D, int G>
__global__ __launch_bounds__(kDecodeThreads, kMfmaWavesPerSimd) void decode_partition_mfma_kernel(
    DecodeParams p) {
  constexpr int EPL = D / 16;            // dims per lane in one V row load
  constexpr int WPL = EPL / 2;           // 32-bit words per V row load
  constexpr int NKC = D / 32;            // 16x16x32 MFMAs per block for the scores
  constexpr int NWAVE = kDecodeWaves;
  constexpr int NBUF = kMfmaPipelineDepth;
  using VT = typename VPiece<D>::T;
  static_assert(G >= 1 && G <= 16, "the q heads of one KV head fill at most 16 MFMA columns");

  const int g = blockIdx.x;
  const int part = blockIdx.y;
  const int s = blockIdx.z;
  const int Hq = p.Hkv * G;
  const int ctx = clamped_ctx(p, s);
  const int nparts = (ctx + kPartTokens - 1) / kPartTokens;
  if (part >= max(nparts, 1)) return;
  const int64_t row0 = (int64_t)s * Hq + (int64_t)g * G;  // first q head of this group

  if (ctx == 0) {  // empty context: zero output
    for (int i = threadIdx.x; i < G * D; i += kDecodeThreads) store_out<true>(p.out, row0 * D + i, 0.f);
    return;
  }

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int h = lane & 15;
  const int j = lane >> 4;

  // q as the B operand of the score MFMAs (columns >= G are zero).
  bf16x8 qf[NKC];
  {
    const char* qrow = reinterpret_cast<const char*>(p.q) + (row0 + min(h, G - 1)) * D * 2;
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
      const uint4 r = h < G ? load16(qrow + (32 * c + 8 * j) * 2) : make_uint4(0, 0, 0, 0);
      qf[c] = __builtin_bit_cast(bf16x8, r);
    }
  }

  const int nblk = (ctx + kBlockTokens - 1) / kBlockTokens;
  const int b_begin = part * kPartBlocks;
  const int b_end = min(b_begin + kPartBlocks, nblk);
  const int32_t* trow = p.tables + (int64_t)s * p.MB;
  const int64_t tok_bytes = (int64_t)p.Hkv * D * 2;
  const int64_t blk_bytes = tok_bytes * kBlockTokens;
  // byte offsets of this lane's pieces inside a block (blocks are < 2 GiB)
  const int k_lane = (int)(h * tok_bytes + (g * D + 8 * j) * 2);
  const int v_lane = (int)(4 * j * tok_bytes + (g * D + EPL * h) * 2);

  struct Blk {
    uint4 k[NKC];
    VT v[4];
    int valid;
  };

  // Block ids of this wave's blocks b_begin + wave + NWAVE*k (k < kPartBlocks /
  // NWAVE), one per lane, fetched once: the per-block id is then a lane read.
  const int nmine = max(0, (b_end - b_begin - wave + NWAVE - 1) / NWAVE);
  const int my_id = lane < nmine ? trow[b_begin + wave + NWAVE * lane] : -1;

  // Loads of the wave's k-th block through buffer resources sized to the block:
  // k past the wave's share or an id outside the pool gets a zero-sized
  // resource, so its loads return zeros without touching memory and the
  // prefetch of later blocks needs no branch.
  auto issue = [&](int k, Blk& B) {
    const int pb = k < nmine ? __builtin_amdgcn_readlane(my_id, k) : -1;
    const bool ok = (unsigned)pb < (unsigned)p.NB;
    const int b = b_begin + wave + NWAVE * k;
    B.valid = ok ? min(kBlockTokens, ctx - b * kBlockTokens) : 0;
    const int64_t base = (int64_t)(ok ? pb : 0) * blk_bytes;
    const int nrec = ok ? (int)blk_bytes : 0;
    const __amdgpu_buffer_rsrc_t kr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p.kc + base), (short)0, nrec, kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p.vc + base), (short)0, nrec, kRawBufferWord3);
#pragma unroll
    for (int c = 0; c < NKC; ++c) B.k[c] = buffer_load16(kr, k_lane + 64 * c, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) B.v[i] = buffer_load_piece<VT>(vr, v_lane, i * tok_bytes);
  };

  float m = -INFINITY;   // running max of head h (log2 domain), uniform over j
  float l = 0.f;         // running sum of this lane's tokens' weights
  f32x4 acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};

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
    float mb = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mb = fmaxf(mb, __shfl_xor(mb, 16, kWave));
    mb = fmaxf(mb, __shfl_xor(mb, 32, kWave));
    const float mn = fmaxf(m, mb);
    const float ms = (mn == -INFINITY) ? 0.f : mn;
    if (__ballot(mn != m)) {  // some head's max grew: rescale what was accumulated
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

  // NBUF-deep software pipeline: blocks k+1 .. k+NBUF-1 are in flight while
  // block k is computed.  The trip count is rounded up to whole rounds; the
  // extra blocks have zero-sized resources and are fully masked, so they leave
  // the running state unchanged.
  Blk buf[NBUF];
#pragma unroll
  for (int u = 0; u < NBUF - 1; ++u) issue(u, buf[u]);
  const int rounds = (nmine + NBUF - 1) / NBUF;
  for (int r = 0; r < rounds; ++r) {
#pragma unroll
    for (int u = 0; u < NBUF; ++u) {
      issue(r * NBUF + u + NBUF - 1, buf[(u + NBUF - 1) % NBUF]);
      compute(buf[u]);
    }
  }

  // Wave totals of head h: l summed over the four lane groups (m is already uniform).
  l += __shfl_xor(l, 16, kWave);
  l += __shfl_xor(l, 32, kWave);

  __shared__ float s_m[NWAVE][G];
  __shared__ float s_l[NWAVE][G];
  __shared__ float s_o[NWAVE][G][D];
  if (h < G) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_o[wave][h][EPL * (4 * j + i) + e] = acc[e][i];
    }
    if (j == 0) {
      s_m[wave][h] = m;
      s_l[wave][h] = l;
    }
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < G * D; idx += kDecodeThreads) {
    const int hh = idx / D;
    const int d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) M = fmaxf(M, s_m[w][hh]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NWAVE; ++w) {
        const float f = exp2_fast(s_m[w][hh] - M);
        L = fmaf(s_l[w][hh], f, L);
        O = fmaf(s_o[w][hh][d], f, O);
      }
    }
    const float r = L > 0.f ? O / L : 0.f;
    if (nparts == 1) {
      store_out<true>(p.out, (row0 + hh) * D + d, r);
    } else {
      const int64_t pr = (row0 + hh) * p.max_parts + part;
      p.part_o[pr * D + d] = r;
      if (d == 0) {
        p.part_m[pr] = M;
        p.part_l[pr] = L;
      }
    }
  }
}

template <int D, int G>
void launch_mfma_t(const DecodeParams& p, const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((decode_partition_mfma_kernel<D, G>),
                     dim3(a.num_kv_heads, a.max_parts, a.num_seqs), dim3(kDecodeThreads), 0, st, p);
}

template <int D>
int launch_mfma_g(const DecodeParams& p, const DecodeArgs& a, hipStream_t st) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: launch_mfma_t<D, 1>(p, a, st); break;
    case 2: launch_mfma_t<D, 2>(p, a, st); break;
    case 4: launch_mfma_t<D, 4>(p, a, st); break;
    case 8: launch_mfma_t<D, 8>(p, a, st); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

}  // namespace

int launch_decode_partitions_bf16(const DecodeParams& p, const DecodeArgs& a, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  return a.head_dim == 64 ? launch_mfma_g<64>(p, a, st) : launch_mfma_g<128>(p, a, st);
}

}  // namespace pkv
