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
// Unlike a decode row, a chunk's rows make a dense tile, so this kernel runs on
// the 32x32x16 matrix instructions (the fastest bf16 shape here).  A workgroup
// item is 256/G consecutive rows x the G q heads of one KV head over one or two
// partitions of keys (the plan's span: two when the batch has enough items to
// keep every compute unit busy, which halves the partial results written and
// merged); each of the eight waves owns one 32-column tile (column n
// = row n/G of the wave's 32/G rows, head n%G).
// Keys go in steps of 32 tokens (two blocks):
//  * scores S^T[t][n] = sum_d K[t][d] q[n][d]: v_mfma_f32_32x32x16_bf16, D/16
//    per tile; A = K (lane: token lane%32, dims 8*(lane/32) .. +7 of the
//    16-dim step, read from LDS), B = q^T (lane: column lane%32, same dims).
//    C: lane (n, h = lane/32), register i <-> token 8*(i/4) + 4h + i%4.
//  * online softmax per column (base 2, lazy reference max as in decode);
//  * values O^T[d][n] += sum_t V^T[d][t] P^T[t][n]: two 16-token k-steps of
//    D/32 MFMAs per tile.  B = P^T is the score registers i = 8s .. 8s+7 of
//    k-step s, rounded to bf16: element e <-> token 16s + 8*(e/4) + 4h + e%4.
//    A = V^T takes the same tokens for the same elements, dim 32E + lane%32
//    for output tile E: two transposing LDS reads (ds_read_b64_tr_b16) per
//    tile and k-step gather them from the token-major V rows in LDS.
//    C: lane (n, h), register i of tile E <-> dim 32E + 8*(i/4) + 4h + i%4.
// Each column keeps its own causal mask (token < the keys its row sees), so the
// diagonal block needs no special case.
//
// K and V of each step are loaded once per workgroup, straight into LDS
// (buffer loads with the LDS destination: 16 bytes per lane, 1 KiB per wave
// instruction, no registers and no LDS write instructions on the way), and
// read by every wave.  In LDS a block's K or V slice is kept in 16-byte units
// (8 dims of one token) laid out so that both read patterns are free of bank
// conflicts without padding (see s_k / s_v).  Rows past the context land as
// zeros (the block's buffer resource ends at the context), so a V row there
// never meets a zero weight as 0 * NaN.  Each wave computes the scores of step
// q + 1 while it runs step q's softmax and value products, so the matrix cores
// work during the vector code.  There is one barrier per four steps, over nine
// step buffers: while the steps q .. q + 3 run (reading the buffers of steps
// q .. q + 4), steps q + 5 .. q + 8 load into the buffers of q - 4 .. q - 1,
// last read before the previous barrier, and each wave waits for its own loads
// before the next barrier.  Fewer barriers let the eight waves drift apart, so
// their LDS reads and their arithmetic overlap rather than all waves reading
// at once after each barrier (one barrier per two steps over seven buffers
// measured 3-4% slower).  The load stream runs across item boundaries: the
// workgroup keeps the record and the q operand of the next item, so a new item
// starts with its first steps and q already loaded.
//
// Workgroups take items from the prefill tickets: the first two are static
// (blockIdx.x and blockIdx.x + gridDim.x), the rest come from the counter.  A row whose
// keys one item covers gets its output written directly; other rows' partials
// go to the workspace for the merge, one slot per item (slot part / span).

#include <hip/hip_runtime.h>

#include <algorithm>

#include "../pkv_internal.hpp"
#include "decode_common.hpp"

namespace pkv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kStepTokens = 2 * kBlockTokens;  // tokens per step (two blocks)
// Waves per workgroup; the item's 256 columns are split among them in 32-column
// tiles.  Eight waves (two per SIMD) let one wave's softmax and LDS reads
// overlap another's matrix products.
constexpr int kPrefillWaves = 8;
constexpr int kPrefillThreads = kPrefillWaves * kWave;
constexpr int kColTiles = 8 / kPrefillWaves;   // 32-column tiles per wave
constexpr int kPrefillSteps = 4;               // steps per barrier interval
// LDS buffers of one step each: while steps q .. q+3 are computed (reading the
// buffers of steps q .. q+4), steps q+5 .. q+8 load into the buffers of
// q-4 .. q-1; 9 x 16 KiB at head_dim 128.
constexpr int kPrefillBufs = 9;

// Transposing LDS read of 16-bit data (gfx950): each lane names 8 bytes (four
// 16-bit values); within each group of 16 lanes, lane i receives value i%4 of
// lanes 4j + i/4, j = 0..3, as its values j.  With lane 4j + a of a group
// pointing at four consecutive dims 4a .. 4a+3 of token row j, lane i gets dim
// i of the four token rows.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const char* p) {
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(uint2, r);
}
// Sum of a packed bf16 pair, added to acc (one dot-product instruction).
__device__ __forceinline__ float add_bf16_pair(uint32_t w, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, 0x3F803F80u), acc,
                                         false);
}
// Direct-to-LDS buffer load (gfx950): each lane's 16 bytes at voff + soff of
// the resource land at lds + 16 * lane (lds uniform over the wave); bytes past
// the resource's range land as zeros.  Counted by vmcnt like any vector load.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, char* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

template <int D, int G>
__global__ __launch_bounds__(kPrefillThreads, 1) void prefill_mfma_kernel(DecodeParams p) {
  constexpr int NT = D / 32;               // 32-dim tiles of the output; V dims per lane
  constexpr int NKC = D / 16;              // 16-dim steps of the scores
  constexpr int CT = kColTiles;
  constexpr int R = 32 / G;                // rows per column tile
  constexpr int RPW = CT * R;              // rows per wave
  constexpr int BLKB = kBlockTokens * D * 2;  // LDS bytes of one block's K (or V) slice
  constexpr int NS = kPrefillSteps;
  static_assert(G >= 1 && G <= 32 && 32 % G == 0, "a tile holds whole rows of G heads");

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n = lane & 31;                 // column of a tile; token / dim slot of operands
  const int hh = lane >> 5;                // lane half
  const int Hq = p.Hkv * G;
  const uint32_t tok_bytes = (uint32_t)p.Hkv * D * 2;
  const uint32_t blk_bytes = tok_bytes * kBlockTokens;
  const int total = min(p.sched[3], p.pre_cap * p.Hkv);
  const int grid = (int)gridDim.x;

  // [buffer][two blocks of 16 token rows]: step q in buffer q % kPrefillBufs.
  // A block's slice is stored in 16-byte units (8 dims of one token): unit
  // c * 16 + u holds dims 8c .. 8c+7 of token row u for K, and of token row
  // u ^ (4 * (c % 4)) for V.  Both read patterns below then spread over all
  // banks (K: 16 lanes read 16 rows of one unit column, 256 contiguous bytes;
  // V: the transposing reads take four rows of four unit columns per 16 lanes),
  // and a 1 KiB direct-to-LDS load (16 bytes per lane) fills four unit columns.
  __shared__ __attribute__((aligned(16))) char s_k[kPrefillBufs][2 * BLKB];
  __shared__ __attribute__((aligned(16))) char s_v[kPrefillBufs][2 * BLKB];
  __shared__ int s_ticket[2];

  struct Item {
    int s, part, span, g, ctx, qrow0, nrows, key0, b_begin, nblk, nsteps;
    int ids;        // lane k: the id of the item's block k (k < nblk)
    bool valid;
  };
  // Records are written by the plan launch and read-only here: read through the
  // constant address space (scalar loads; waiting for them never waits for the
  // vector loads in flight).
  auto make_item = [&](int tk, Item& it) {
    // the record's address does not wait for the count of tickets: a ticket
    // past it reads a record that is not used (no blocks, no rows)
    it.valid = tk < total;
    const int t = min(tk, p.pre_cap * p.Hkv - 1);
    const __attribute__((address_space(4))) int* r =
        (const __attribute__((address_space(4))) int*)(const void*)p.pre_recs + 8 * (t / p.Hkv);
    it.g = t % p.Hkv;
    it.s = r[0];
    it.part = r[1];
    it.ctx = r[2];
    it.qrow0 = r[3];
    it.nrows = r[4];
    it.key0 = r[5];                                       // row i sees max(0, key0 + i) keys
    it.span = r[6];                                       // partitions covered: 1 or 2
    const int key_last = max(0, it.key0 + it.nrows - 1);  // keys the item's last row sees
    const int k_begin = it.part * kPartTokens;
    const int k_end = min(k_begin + it.span * kPartTokens, key_last);
    it.b_begin = it.part * kPartBlocks;
    it.nblk = it.valid ? max(0, (k_end - k_begin + kBlockTokens - 1) / kBlockTokens) : 0;
    // steps of two blocks, padded to a multiple of NS so that every item starts
    // an interval, and to at least 8: the load stream runs up to eight steps
    // ahead of the interval being computed and must never run past the next
    // item; padding steps load nothing and compute nothing
    it.nsteps = max(8, (max(1, (it.nblk + 1) / 2) + NS - 1) / NS * NS);
    {
      // the item's block ids, one per lane (an item spans at most 64 blocks),
      // loaded once; each step then takes its id from a lane, with no memory wait
      const __amdgpu_buffer_rsrc_t tr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<int*>(p.tables + (int64_t)it.s * p.MB + it.b_begin), (short)0, it.nblk * 4, kRawBufferWord3);
      it.ids = __builtin_amdgcn_raw_buffer_load_b32(tr, lane * 4, 0, 0);
    }
  };
  // q operands (B of the scores) of this wave's columns; rows past the item read
  // zeros through the resource bound.
  auto load_q = [&](const Item& it, bf16x8 (&qv)[CT][NKC]) {
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(reinterpret_cast<const char*>(p.q) + (int64_t)it.qrow0 * Hq * D * 2), (short)0,
        it.valid ? it.nrows * Hq * D * 2 : 0, kRawBufferWord3);
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const int r = wave * RPW + c * R + n / G;
      const int off = ((r * Hq + it.g * G + n % G) * D + 8 * hh) * 2;
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) qv[c][kc] = __builtin_bit_cast(bf16x8, buffer_load16(qr, off + 32 * kc, 0));
    }
  };

  // Loads straight into LDS: a wave instruction moves 1 KiB, 16 bytes per lane,
  // into four unit columns of one block's K or V slice (lane i: unit column
  // i / 16, position i % 16).  A step takes 4 CPB such instructions (K and V,
  // two blocks, CPB per block slice); this wave issues LPW of them, all in one
  // block slice: tensor ld_v (K or V), block ld_b of the step, unit columns
  // 4 (ld_piece + j) .. +3 for j < LPW.
  constexpr int CPB = D / 32;                      // 1 KiB pieces per block slice
  constexpr int LPW = 4 * CPB / kPrefillWaves;     // load instructions per wave and step
  static_assert(LPW >= 1 && 4 * CPB % kPrefillWaves == 0 && CPB % LPW == 0, "whole block slices per wave");
  const int ld_first = wave * LPW;
  const bool ld_v = ld_first >= 2 * CPB;
  const int ld_b = (ld_first / CPB) % 2;
  const int ld_piece = ld_first % CPB;
  // per lane and instruction: the byte offset in the block (token row, dims);
  // the KV head's offset goes in the scalar offset
  int ld_off[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int c = 4 * (ld_piece + j) + lane / 16;  // unit column: dims 8c .. 8c+7
    const int u = lane % 16;
    const int row = ld_v ? u ^ (4 * (c % 4)) : u;
    ld_off[j] = row * (int)tok_bytes + c * 16;
  }
  const char* ld_pool = ld_v ? p.vc : p.kc;
  // The load stream's position: an item (copied) and a step of it.  Each step's
  // block id comes from a lane of the item's id register; with each id, the
  // number of the block's rows inside the context.
  struct Cursor {
    int ids;
    int nblk, ctx_rel, g, step, nsteps;
  };
  auto cursor_of = [&](const Item& it) {
    Cursor c;
    c.ids = it.ids;
    c.nblk = it.nblk;
    c.ctx_rel = it.ctx - it.b_begin * kBlockTokens;  // context tokens from the item's first block
    c.g = it.g;
    c.step = 0;
    c.nsteps = it.nsteps;
    return c;
  };
  // Loads of the cursor's step into LDS buffer buf.  Each block's buffer
  // resource ends at the context (rows past it land as zeros, so a V row there
  // never meets a zero weight as 0 * NaN) and is empty past the item's blocks
  // or for an id outside the pool.
  auto issue_step = [&](const Cursor& c, int buf) {
    const int k = 2 * c.step + ld_b;
    const int id = __builtin_amdgcn_readlane(c.ids, min(k, kWave - 1));
    const bool ok = k < c.nblk && (unsigned)id < (unsigned)p.NB;
    const int lim = min(kBlockTokens, c.ctx_rel - k * kBlockTokens);
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(ld_pool + (uint64_t)(uint32_t)(ok ? id : 0) * blk_bytes), (short)0,
        ok ? lim * (int)tok_bytes : 0, kRawBufferWord3);
    char* dst = (ld_v ? s_v[buf] : s_k[buf]) + ld_b * BLKB + ld_piece * 1024;
#pragma unroll
    for (int j = 0; j < LPW; ++j) buffer_load_lds16(r, dst + 1024 * j, ld_off[j], c.g * D * 2);
  };

  bf16x8 qf[CT][NKC], qn[CT][NKC];   // q operands of the current and the next item
  float m[CT], l[CT], mref[CT];      // lazy reference max (log2 units), its finite form
  f32x16 acc[CT][NT];
  int col_keys[CT];                   // keys the column's row sees (0 past the item's rows)
  int min_keys;                       // the least of them over the wave (uniform)

  // This lane's K operand in a step buffer: token n (block n / 16, row n % 16),
  // dims 16 kc + 8 hh .. +7 = unit column 2 kc + hh, at k_lane + 512 kc.
  const int k_lane = (n >> 4) * BLKB + hh * 256 + (n & 15) * 16;

  // Scores of the step in LDS buffer buf (the matrix products only).
  auto scores = [&](int buf, f32x16 (&sc)[CT]) {
    const char* kb = s_k[buf] + k_lane;
#pragma unroll
    for (int c = 0; c < CT; ++c) sc[c] = f32x16{};
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const bf16x8 kf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kb + 512 * kc));
#pragma unroll
      for (int c = 0; c < CT; ++c) sc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c][kc], sc[c], 0, 0, 0);
    }
  };
  // This lane's addresses in a V buffer for the transposing reads: lane
  // 16g + 4j + a names token row 4*(g/2) + j of an 8-row group (rows 0..7 of
  // a block: v_lane, rows 8..15: v_lane_hi), dims 16*(g%2) + 4a .. +3 of the
  // output tile, so that lane 16g + i receives dim 16*(g%2) + i = lane%32 of
  // token rows 4*(g/2) + 0..3 = 4*hh + 0..3.  Those dims are unit column
  // 4e + cl of output tile e (cl = 2*(g%2) + a/2; bytes 8*(a%2) of the unit),
  // found at unit (4e + cl) * 16 + (row ^ 4*cl): e adds 1 KiB.
  const int v_cl = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int v_row = 4 * hh + ((lane >> 2) & 3);
  const int v_lane = (v_cl * 16 + (v_row ^ (4 * v_cl))) * 16 + (lane & 1) * 8;
  const int v_lane_hi = (v_cl * 16 + ((v_row + 8) ^ (4 * v_cl))) * 16 + (lane & 1) * 8;

  // Softmax and value products of a step from its scores and LDS buffer buf:
  // tokens t0 .. t0+31 (V rows past the context hold zeros); with them, in
  // the same straight-line code, the score products of the next step (K in
  // LDS buffer kbuf, into sn), so that the matrix and vector work interleave.
  auto softmax_values = [&](f32x16 (&sc)[CT], int buf, int t0, int kbuf, f32x16 (&sn)[CT]) {
    const char* vb = s_v[buf];
    const char* kb = s_k[kbuf] + k_lane;
    // softmax per column in base 2: register i holds token 8*(i/4) + 4*hh + i%4.
    // Only steps that reach past some column's keys (the causal edge, the end
    // of the context) need the per-element mask, which sets the raw score to
    // -inf; every step then takes the scale into the exponent's fused
    // multiply-add (-inf stays -inf: the scale is positive).
    const bool masked = t0 + kStepTokens > min_keys;  // uniform over the wave
    float rmax[CT];
    bool over = false;
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      if (masked) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int t = t0 + 8 * (i / 4) + 4 * hh + (i % 4);
          sc[c][i] = t < col_keys[c] ? sc[c][i] : -INFINITY;
        }
      }
      float r = sc[c][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) r = fmaxf(r, sc[c][i]);
      rmax[c] = r;
      // this half's tokens exceed the column's reference by more than the lazy
      // margin (always at the first live step: the reference is -inf; the scale
      // is positive, so the max commutes with it)
      over |= r * p.scale_log2 > m[c] + kRescaleLog2;
    }
    if (__ballot(over)) {  // move the references of the columns that exceed them
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const float mb = max_over_halves(rmax[c] * p.scale_log2);  // both halves of the column
        const bool up = mb > m[c] + kRescaleLog2;
        const float mn = up ? mb : m[c];
        const float mr = (mn == -INFINITY) ? 0.f : mn;
        const float alpha = exp2_fast(m[c] - mr);  // 1 where the reference stays, 0 from -inf
        mref[c] = mr;
        m[c] = mn;
        l[c] *= alpha;
#pragma unroll
        for (int e = 0; e < NT; ++e) acc[c][e] *= alpha;
      }
    }
    auto weight = [&](int c, int i) { return exp2_fast(fmaf(sc[c][i], p.scale_log2, -mref[c])); };
#pragma unroll
    for (int c = 0; c < CT; ++c) sn[c] = f32x16{};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      // P^T operand of k-step s (rounded weights summed into l)
      bf16x8 pt[CT];
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        uint32_t w[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          w[d] = pack_bf16x2(weight(c, 8 * s + 2 * d), weight(c, 8 * s + 2 * d + 1));
          l[c] = add_bf16_pair(w[d], l[c]);
        }
        pt[c] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
      }
      // half of the next step's score products
#pragma unroll
      for (int kc = s * NKC / 2; kc < (s + 1) * NKC / 2; ++kc) {
        const bf16x8 kf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kb + 512 * kc));
#pragma unroll
        for (int c = 0; c < CT; ++c) sn[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c][kc], sn[c], 0, 0, 0);
      }
      // V^T operand of tile e: element j <-> token 16s + 8*(j/4) + 4*hh + j%4,
      // dim 32e + lane%32 (token rows 16s + 4*hh + 0..3, then 8 rows on)
#pragma unroll
      for (int e = 0; e < NT; ++e) {
        const uint2 lo = lds_read_tr16(vb + v_lane + s * BLKB + 1024 * e);
        const uint2 hi = lds_read_tr16(vb + v_lane_hi + s * BLKB + 1024 * e);
        const bf16x8 av = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
        for (int c = 0; c < CT; ++c) acc[c][e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pt[c], acc[c][e], 0, 0, 0);
      }
    }
  };

  auto begin_item = [&](const Item& it) {
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      m[c] = -INFINITY;
      mref[c] = 0.f;
      l[c] = 0.f;
      const int r = wave * RPW + c * R + n / G;
      col_keys[c] = r < it.nrows ? max(0, it.key0 + r) : 0;
#pragma unroll
      for (int e = 0; e < NT; ++e) acc[c][e] = f32x16{};
    }
    int mk = col_keys[0];
#pragma unroll
    for (int c = 1; c < CT; ++c) mk = min(mk, col_keys[c]);
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) mk = min(mk, __shfl_xor(mk, o, kWave));
    min_keys = __builtin_amdgcn_readfirstlane(mk);
  };

  auto finish_item = [&](const Item& it) {
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const float lt = sum_over_halves(l[c]);
      const int r = wave * RPW + c * R + n / G;
      const int keys = max(0, it.key0 + r);
      const int nparts = max(1, (keys + kPartTokens - 1) / kPartTokens);
      const int nslots = (nparts + it.span - 1) / it.span;  // this row's items, one partial each
      // a row that ends before this partition has nothing here (its own items
      // cover its partitions); a row one item covers gets its output directly,
      // the others a partial in slot part / span
      if (r < it.nrows && it.part < nparts) {
        const int64_t orow = (int64_t)(it.qrow0 + r) * Hq + it.g * G + n % G;
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        // registers 4k .. 4k+3 of tile e hold dims 32e + 8k + 4*hh + 0..3: one
        // vector store of four consecutive dims each
        if (nslots == 1) {
          char* o = reinterpret_cast<char*>(p.out) + orow * D * 2;
#pragma unroll
          for (int e = 0; e < NT; ++e) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const f32x16& a = acc[c][e];
              *reinterpret_cast<uint2*>(o + (32 * e + 8 * k + 4 * hh) * 2) =
                  make_uint2(pack_bf16x2(a[4 * k] * inv, a[4 * k + 1] * inv),
                             pack_bf16x2(a[4 * k + 2] * inv, a[4 * k + 3] * inv));
            }
          }
        } else {
          const int64_t pr = orow * p.max_parts + it.part / it.span;
          float* o = p.part_o + pr * D;
#pragma unroll
          for (int e = 0; e < NT; ++e) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const f32x16& a = acc[c][e];
              *reinterpret_cast<float4*>(o + 32 * e + 8 * k + 4 * hh) =
                  make_float4(a[4 * k] * inv, a[4 * k + 1] * inv, a[4 * k + 2] * inv, a[4 * k + 3] * inv);
            }
          }
          if (hh == 0) {
            p.part_m[pr] = m[c];
            p.part_l[pr] = lt;
          }
        }
      }
    }
  };

  // The item queue: cur (being computed) and n1 (record known, q loaded into
  // qn); the ticket after n1 is fetched while cur runs.  The loads run up to
  // eight steps ahead of the interval being computed: into n1 near the end of
  // cur, never past it.
  Item cur, n1;
  make_item(blockIdx.x, cur);
  if (!cur.valid) return;
  load_q(cur, qf);

  // The load stream runs ahead of the computation: in cur, then in n1
  // (cs_n1).  Stepping past the end of n1 (which has at least eight steps, so
  // this does not happen with the stream's lookahead) would leave it pending (cs_wait) until the item switch makes the next
  // n1; that happens before the next issue.  An invalid item has no
  // blocks (zero-sized loads).
  Cursor cs = cursor_of(cur);
  bool cs_n1 = false, cs_wait = false;
  auto issue_next = [&](int buf) {
    issue_step(cs, buf);
    if (__builtin_expect(++cs.step == cs.nsteps, 0)) {
      if (cs_n1) {
        cs_wait = true;
      } else {
        cs = cursor_of(n1);
        cs_n1 = true;
      }
    }
  };

  // Four steps per barrier: while steps q .. q + 3 run (reading the LDS
  // buffers of steps q .. q + 4; step j + 1's scores are computed during step
  // j's softmax and values), steps q + 5 .. q + 8 load into the buffers of
  // q - 4 .. q - 1, last read before the previous barrier.  The loads are
  // issued after the first and the second step's vector code, not right after
  // the barrier, where every wave would queue for the compute unit's scalar
  // unit with the same address work at once.  __syncthreads() waits for every
  // load of this wave (its fence orders all earlier memory operations, the
  // direct-to-LDS loads included) before the barrier, so the next interval
  // finds steps q + 4 .. q + 8 in LDS.
  static_assert(NS == 4 && kPrefillBufs == 9, "four steps per barrier, five more buffers");
#pragma unroll
  for (int u = 0; u < 5; ++u) issue_next(u);  // steps 0 .. 4 (cur has at least eight)
  // the next item is read once the first loads are on their way
  make_item(blockIdx.x + grid, n1);
  load_q(n1, qn);
  __syncthreads();  // steps 0 .. 4 in LDS (and n1's loads landed)
  int buf = 0, tpar = 0;  // LDS buffer of step 0 of cur
  f32x16 sc[2][CT];       // scores of steps of either parity
  for (;;) {  // one item per iteration
    int fetched;  // thread 0: the ticket after n1, written to LDS at cur's last step
    if (tid == 0) fetched = atomicAdd(&p.sched[2], 1);  // offset added where it is read
    begin_item(cur);
    if (cur.nblk > 0) scores(buf, sc[0]);
    // Buffers rotate over nine: step q + k in rot(buf, k) relative to the interval.
    auto rot = [](int b, int k) { return b + k >= kPrefillBufs ? b + k - kPrefillBufs : b + k; };
    for (int q = 0; q < cur.nsteps; q += 4) {
      const int b1 = rot(buf, 1), b2 = rot(buf, 2), b3 = rot(buf, 3), b4 = rot(buf, 4);
      if (q + 4 == cur.nsteps && tid == 0) s_ticket[tpar] = fetched;
      const int t0 = (cur.b_begin + 2 * q) * kBlockTokens;
      if (2 * q < cur.nblk) softmax_values(sc[0], buf, t0, b1, sc[1]);
      issue_next(rot(buf, 5));            // step q + 5
      issue_next(rot(buf, 6));            // step q + 6
      if (2 * q + 2 < cur.nblk) softmax_values(sc[1], b1, t0 + kStepTokens, b2, sc[0]);
      issue_next(rot(buf, 7));            // step q + 7
      issue_next(rot(buf, 8));            // step q + 8
      if (2 * q + 4 < cur.nblk) softmax_values(sc[0], b2, t0 + 2 * kStepTokens, b3, sc[1]);
      if (2 * q + 6 < cur.nblk) softmax_values(sc[1], b3, t0 + 3 * kStepTokens, b4, sc[0]);
      __syncthreads();  // this interval's loads have landed (the fence waits for them)
      buf = b4;
    }
    // Switch to n1.  Its q was loaded at the start of this item; the empty asm
    // makes the wait for those loads happen here, once, before the output
    // stores are in flight (left to the compiler, it lands before the score
    // products inside the step loop, every other step).
#pragma unroll
    for (int c = 0; c < CT; ++c) {
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        qf[c][kc] = qn[c][kc];
        asm volatile("" : "+v"(qf[c][kc]));
      }
    }
    finish_item(cur);
    const int tk = 2 * grid + __builtin_amdgcn_readfirstlane(s_ticket[tpar]);
    tpar ^= 1;
    cur = n1;
    if (!cur.valid) break;
    make_item(tk, n1);
    load_q(n1, qn);
    if (cs_wait) {  // the stream stepped past the old n1: it continues in the new one
      cs = cursor_of(n1);
      cs_wait = false;
    } else {
      cs_n1 = false;  // the stream's item (the old n1) is now cur
    }
  }
}

template <int D, int G>
int launch_prefill_t(const DecodeArgs& a, hipStream_t st) {
  const DecodeParams p = make_params(a);
  const int64_t items = (int64_t)a.pre_cap * a.num_kv_heads;  // upper bound
  const int64_t grid = std::min<int64_t>(items, (int64_t)a.num_cus);
  hipLaunchKernelGGL((prefill_mfma_kernel<D, G>), dim3((unsigned)std::max<int64_t>(grid, 1)),
                     dim3(kPrefillThreads), 0, st, p);
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
