// Calibration kernel: the bf16 matrix-core rate this part sustains under full
// load. Every wave runs a register-only loop of independent MFMAs (no memory
// traffic and no other instructions inside the loop), so the measured rate is
// the ceiling any MFMA kernel can reach on the part at the clock it holds
// under that load, as opposed to the published peak at the nominal clock.
//   shape 0: v_mfma_f32_16x16x32_bf16, 32 per iteration over 8 accumulators
//   shape 1: v_mfma_f32_32x32x16_bf16, 16 per iteration over 4 accumulators
// Both do 524288 flop per wave per iteration.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../../include/jano_calib.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 512;               // 8 waves: two per SIMD

template <int SHAPE>
__global__ __launch_bounds__(kThreads) void mfma_loop_kernel(int iters, float seed, float *sink,
                                                             long long *cycles) {
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(seed * static_cast<float>(threadIdx.x + e));
    b[e] = static_cast<__bf16>(seed * static_cast<float>(threadIdx.x - e));
  }
  f32x4 acc4[8];
  f32x16 acc16[4];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc4[k] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc16[k][r] = 0.f;
  const long long t0 = __builtin_amdgcn_s_memtime();
  for (int i = 0; i < iters; ++i) {
    if constexpr (SHAPE == 0) {
#pragma unroll
      for (int m = 0; m < 32; ++m)
        acc4[m % 8] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc4[m % 8], 0, 0, 0);
    } else {
#pragma unroll
      for (int m = 0; m < 16; ++m)
        acc16[m % 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc16[m % 4], 0, 0, 0);
    }
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += acc4[k][0] + acc4[k][1] + acc4[k][2] + acc4[k][3];
#pragma unroll
  for (int k = 0; k < 4; ++k) s += acc16[k][0] + acc16[k][7] + acc16[k][15];
  // never true for the seeds used; keeps the accumulators (and the loop) live
  if (s == 12345.678f) sink[blockIdx.x * kThreads + threadIdx.x] = s;
  if (cycles != nullptr && threadIdx.x % 64 == 0)
    cycles[blockIdx.x * (kThreads / 64) + threadIdx.x / 64] = t1 - t0;
}

}  // namespace

extern "C" int jano_calib_mfma_loop(int shape, int workgroups, int iters, float *sink,
                                    long long *cycles, void *stream) {
  if (shape < 0 || shape > 1 || workgroups < 1 || iters < 1 || sink == nullptr) return 1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // 96 KB of dynamic LDS (unused) holds the kernel to one workgroup per CU
  constexpr unsigned kLds = 96 * 1024;
  if (shape == 0)
    hipLaunchKernelGGL(mfma_loop_kernel<0>, dim3(workgroups), dim3(kThreads), kLds, st, iters, 1e-3f,
                       sink, cycles);
  else
    hipLaunchKernelGGL(mfma_loop_kernel<1>, dim3(workgroups), dim3(kThreads), kLds, st, iters, 1e-3f,
                       sink, cycles);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
