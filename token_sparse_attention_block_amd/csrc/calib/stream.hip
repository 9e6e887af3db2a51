// Calibration kernels: the HBM rates plain streaming reaches on this part, a
// measured ceiling for the row copies (read + write) and for the analyzer
// (read only), to set beside the published 8 TB/s.
//   mode 0: dst = src, 16-byte non-temporal loads and stores
//   mode 1: src is only read (16-byte non-temporal loads) and summed per
//           thread; the sum is stored only in a case that does not occur
// Grid-stride: each pass of a workgroup covers 4 x 256 consecutive 16-byte
// pieces, so every thread has four loads in flight.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../../include/jano_calib.h"

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 4;

template <int MODE>
__global__ __launch_bounds__(kThreads) void stream_kernel(const f4 *__restrict__ src, f4 *__restrict__ dst,
                                                          size_t n, float *sink) {
  const size_t stride = static_cast<size_t>(gridDim.x) * kThreads * kUnroll;
  float s = 0.f;
  for (size_t base = static_cast<size_t>(blockIdx.x) * kThreads * kUnroll; base < n; base += stride) {
    f4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t i = base + u * kThreads + threadIdx.x;
      v[u] = i < n ? __builtin_nontemporal_load(&src[i]) : f4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t i = base + u * kThreads + threadIdx.x;
      if constexpr (MODE == 0) {
        if (i < n) __builtin_nontemporal_store(v[u], &dst[i]);
      } else {
        s += v[u].x + v[u].y + v[u].z + v[u].w;
      }
    }
  }
  if (MODE == 1 && s == 12345.678f) sink[blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

extern "C" int jano_calib_stream(int mode, const void *src, void *dst, size_t bytes, int workgroups,
                                 float *sink, void *stream) {
  if (mode < 0 || mode > 1 || src == nullptr || bytes == 0 || bytes % 16 != 0 || workgroups < 1 ||
      reinterpret_cast<uintptr_t>(src) % 16 != 0)
    return 1;
  if (mode == 0 && (dst == nullptr || reinterpret_cast<uintptr_t>(dst) % 16 != 0)) return 1;
  if (mode == 1 && sink == nullptr) return 1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t n = bytes / 16;
  const f4 *s = static_cast<const f4 *>(src);
  if (mode == 0)
    hipLaunchKernelGGL(stream_kernel<0>, dim3(workgroups), dim3(kThreads), 0, st, s, static_cast<f4 *>(dst), n,
                       sink);
  else
    hipLaunchKernelGGL(stream_kernel<1>, dim3(workgroups), dim3(kThreads), 0, st, s, nullptr, n, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
