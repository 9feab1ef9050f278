// LDS operand-read probe: the chunked-prefill kernel's K and V operand reads by
// themselves, the ceiling its step loop is compared with.
//
// Measurement code (libpkvprobe.so), not part of the attention library.  One
// workgroup per compute unit holds five step buffers of 32 token rows at
// head_dim 128 in one of two layouts: padded rows (K rows of 272 bytes, V rows
// of 320; the kernel's layout before its loads went straight into LDS), or, with
// mode bit 4, the kernel's unit-column layouts (16-byte units of 8 dims of one
// token; K unit c * 16 + u holds token row u, V unit c * 16 + u token row
// u ^ 4 (c % 4); two 16-row blocks of 4 KiB per buffer).  Each wave repeats,
// per iteration, the reads one wave makes in one 32-token step of that kernel:
//
//  * K (mode bit 1): eight 16-byte reads per lane, lane n % 32 reading token
//    row n % 32, dims 16 kc + 8 (n / 32) .. +7 (the A operand of the score
//    products, 8 KiB per wave);
//  * V (mode bit 2): sixteen transposing 8-byte reads per lane
//    (ds_read_b64_tr_b16; the A operand of the value products, 8 KiB per
//    wave), with the kernel's lane addressing.
//
// Each burst is issued whole before any of its data is used (a scheduling
// barrier keeps the compiler from spacing the reads out), and every lane folds
// what it read into registers that are stored at the end, so no read can be
// dropped.  Per wave, the cycles of the loop (s_memtime) are written out.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kRowK = 128 * 2 + 16;
constexpr int kRowV = 128 * 2 + 64;
constexpr int kBufs = 5;
constexpr int kLdsBytes = kBufs * 32 * (kRowK + kRowV);

typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint2 read_tr16(const char* p) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p)));
}

template <int NW, bool UNITS>
__global__ __launch_bounds__(NW * 64, 1) void probe_lds_reads_kernel(int32_t iters, int32_t mode, uint32_t* __restrict__ sink,
                                                                    unsigned long long* __restrict__ cycles) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  for (int i = threadIdx.x; i < kLdsBytes / 4; i += NW * 64) reinterpret_cast<uint32_t*>(lds)[i] = i * 2654435761u;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int n = lane & 31, hh = lane >> 5;
  const int v_lane = (4 * hh + ((lane >> 2) & 3)) * kRowV + (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
  // unit-column layout: lane 16g + 4j + a reads unit column cl = 2 (g % 2) + a / 2
  // (+ 4 e), token row 4 hh + j (+ 8 for the second half of a block)
  const int cl = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int vrow = 4 * hh + ((lane >> 2) & 3);
  const int v_unit_lo = (cl * 16 + (vrow ^ (4 * cl))) * 16 + (lane & 1) * 8;
  const int v_unit_hi = (cl * 16 + ((vrow + 8) ^ (4 * cl))) * 16 + (lane & 1) * 8;
  constexpr int kUnitBuf = 2 * 4096;            // bytes of one step's K (or V) in the unit layout
  uint4 fk[8] = {};
  uint2 fv[16] = {};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    asm volatile("" ::: "memory");
    const int buf = it % kBufs;
    if (mode & 1) {
      const char* kb = UNITS ? lds + buf * kUnitBuf + (n >> 4) * 4096 + hh * 256 + (n & 15) * 16
                             : lds + buf * 32 * kRowK + n * kRowK + 16 * hh;
      constexpr int kstep = UNITS ? 512 : 32;
      uint4 x[8];
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) x[kc] = *reinterpret_cast<const uint4*>(kb + kstep * kc);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) {
        fk[kc].x ^= x[kc].x; fk[kc].y ^= x[kc].y; fk[kc].z ^= x[kc].z; fk[kc].w ^= x[kc].w;
      }
    }
    if (mode & 2) {
      uint2 y[16];
      if constexpr (UNITS) {
        const char* vb = lds + kBufs * kUnitBuf + buf * kUnitBuf;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            y[8 * s + 2 * e] = read_tr16(vb + v_unit_lo + 4096 * s + 1024 * e);
            y[8 * s + 2 * e + 1] = read_tr16(vb + v_unit_hi + 4096 * s + 1024 * e);
          }
        }
      } else {
        const char* vb = lds + kBufs * 32 * kRowK + buf * 32 * kRowV + v_lane;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            y[8 * s + 2 * e] = read_tr16(vb + 16 * s * kRowV + 64 * e);
            y[8 * s + 2 * e + 1] = read_tr16(vb + (16 * s + 8) * kRowV + 64 * e);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 16; ++i) { fv[i].x ^= y[i].x; fv[i].y ^= y[i].y; }
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  uint32_t acc = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) acc ^= fk[i].x ^ fk[i].y ^ fk[i].z ^ fk[i].w;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc ^= fv[i].x ^ fv[i].y;
  sink[blockIdx.x * NW * 64 + threadIdx.x] = acc;
  if (lane == 0) cycles[blockIdx.x * NW + (threadIdx.x >> 6)] = t1 - t0;
}

template <int NW>
int launch(int32_t iters, int32_t mode, int32_t grid, uint32_t* sink, unsigned long long* cycles, hipStream_t st) {
  if (mode & 4)
    hipLaunchKernelGGL((probe_lds_reads_kernel<NW, true>), dim3(grid), dim3(NW * 64), 0, st, iters, mode, sink, cycles);
  else
    hipLaunchKernelGGL((probe_lds_reads_kernel<NW, false>), dim3(grid), dim3(NW * 64), 0, st, iters, mode, sink, cycles);
  return (int)hipGetLastError();
}

}  // namespace

// Runs `iters` iterations of the operand reads selected by `mode` (1: K, 2: V,
// 3: both; + 4: the unit-column layouts instead of padded rows) in `grid`
// workgroups of `waves` waves (4, 8 or 16).  sink: device, grid * waves * 64
// uint32; cycles: device, grid * waves uint64 (loop cycles per wave).  Returns 0, or a HIP error code (1 for a bad mode, wave count or
// size).
extern "C" int pkv_probe_lds_reads(int32_t mode, int32_t waves, int32_t iters, int32_t grid, void* sink, void* cycles,
                                   void* stream) {
  if (mode < 1 || mode > 7 || (mode & 3) == 0 || iters < 1 || grid < 1 || !sink || !cycles) return 1;
  uint32_t* s = static_cast<uint32_t*>(sink);
  unsigned long long* c = static_cast<unsigned long long*>(cycles);
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (waves) {
    case 4: return launch<4>(iters, mode, grid, s, c, st);
    case 8: return launch<8>(iters, mode, grid, s, c, st);
    case 16: return launch<16>(iters, mode, grid, s, c, st);
    default: return 1;
  }
}
