// Device helpers shared by the gfx950 kernels: bf16 <-> fp32, 16-byte vector
// access, wavefront reductions and the log2-domain exponential.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kWave = 64;           // CDNA wavefront width
constexpr int kBlockTokens = 16;    // tokens per KV block
constexpr int kPartTokens = 512;    // tokens per split-context partition
constexpr int kPartBlocks = kPartTokens / kBlockTokens;

// bf16 is the upper half of an fp32: widening is a shift (low half) or a mask (high half).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even; NaN stays NaN (quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Lazy rescaling of the online softmax: the running reference max moves only
// when a block's max exceeds it by more than this many powers of two, so
// weights 2^(x - ref) stay below 2^8 and the accumulators are rescaled rarely.
// The result is the same softmax: the reference cancels between the weighted
// sum and the sum of weights (and between partials in the log-sum-exp merge).
constexpr float kRescaleLog2 = 8.f;

// 2^x on the hardware exponential unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Widen one 16-byte load of storage into fp32 values (8 for bf16, 4 for fp32).
template <bool BF16>
__device__ __forceinline__ void widen16(const uint4& r, float* f) {
  if constexpr (BF16) {
    f[0] = bf16_lo(r.x); f[1] = bf16_hi(r.x);
    f[2] = bf16_lo(r.y); f[3] = bf16_hi(r.y);
    f[4] = bf16_lo(r.z); f[5] = bf16_hi(r.z);
    f[6] = bf16_lo(r.w); f[7] = bf16_hi(r.w);
  } else {
    f[0] = __uint_as_float(r.x); f[1] = __uint_as_float(r.y);
    f[2] = __uint_as_float(r.z); f[3] = __uint_as_float(r.w);
  }
}

__device__ __forceinline__ uint4 load16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Raw buffer resources (gfx9 descriptor, stride 0): loads at byte offsets at or
// past the resource's range return zeros without a memory access.
constexpr int kRawBufferWord3 = 0x00020000;

// Cache policy of a buffer load (its aux operand): kStreamLoad sets the
// nontemporal hint (`nt`) for data each launch reads once, the K/V blocks.
// Measured on the partition kernel (interleaved A/B on one box): 6-15% shorter
// launches, and a plain read of 32 KiB blocks in random order goes from 6.1 to
// 6.8 TB/s with it.
constexpr int kCachedLoad = 0;
constexpr int kStreamLoad = 2;

template <int kPolicy = kCachedLoad>
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kPolicy));
}

template <typename T, int kPolicy = kCachedLoad>
struct BufferPiece;
template <int kPolicy>
struct BufferPiece<uint4, kPolicy> {
  static __device__ __forceinline__ uint4 load(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return buffer_load16<kPolicy>(r, voff, soff);
  }
};
template <int kPolicy>
struct BufferPiece<uint2, kPolicy> {
  static __device__ __forceinline__ uint2 load(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kPolicy));
  }
};
template <typename T, int kPolicy = kCachedLoad>
__device__ __forceinline__ T buffer_load_piece(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return BufferPiece<T, kPolicy>::load(r, voff, soff);
}

// Reductions over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48)
// with the gfx950 lane-swap instructions (vector ALU, no LDS round trip).
// v_permlane16_swap(x, x) yields, per lane, the lane's own value and its xor-16
// partner's in its two results; v_permlane32_swap(x, x) the same for xor 32.
// All 64 lanes must be active.
__device__ __forceinline__ float max_over_rows(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_rows(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// The same over the two 32-lane halves only (lane and lane ^ 32).
__device__ __forceinline__ float max_over_halves(float v) {
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_halves(float v) {
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Butterfly sum / max over lanes that differ only in the bits of [lo_mask, 64).
template <int FROM, int TO>
__device__ __forceinline__ float xor_sum(float v) {
#pragma unroll
  for (int off = FROM; off < TO; off <<= 1) v += __shfl_xor(v, off, kWave);
  return v;
}
template <int FROM, int TO>
__device__ __forceinline__ float xor_max(float v) {
#pragma unroll
  for (int off = FROM; off < TO; off <<= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

}  // namespace pkv
