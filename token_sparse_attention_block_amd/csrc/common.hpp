// Shared device helpers for the gfx950 kernels of libjano.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jano {

constexpr int kWave = 64;  // CDNA wavefront width

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Value of `x` held by lane (lane + delta) of the same wave (undefined source
// lanes read lane's own value). Used for the +w neighbour.
__device__ __forceinline__ double shfl_down_f64(double x, int delta) {
  return __shfl_down(x, delta, kWave);
}

__device__ __forceinline__ float shfl_xor_f32(float x, int mask) {
  return __shfl_xor(x, mask, kWave);
}

// Number of set bits of `mask` in lanes below the calling lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  const int lane = __lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const uint32_t u = __shfl_up(v, off, kWave);
    if (lane >= off) v += u;
  }
  return v;
}

}  // namespace jano
