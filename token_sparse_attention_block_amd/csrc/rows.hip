// Row gather (adaptive token activation) and KV-cache row scatter (gfx950).
//
// Method (Jano pages, nl methodology §2 and contributions item 2; zh §2.2
// item 3): only the tokens due at a step are computed, and the key/value pairs
// of the frozen tokens stay in a cache; here the fresh rows of the active
// tokens are written into a persistent full-sequence cache at their token
// positions, so the cache always holds every token's latest K/V.
//
// Both kernels are pure HBM streams: one workgroup per row, sized to the row
// (one 16-byte dwordx4 chunk per thread up to 1024 threads, so a 10 KB row of
// 40 heads x 128 dims is copied by 640 threads in a single pass), rows of H*d
// bf16. A scalar path covers rows whose byte size or base addresses are not
// 16-byte aligned.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace jano {
namespace {

constexpr int kRowThreads = 256;     // scalar fallback
constexpr int kMaxRowThreads = 1024;

// threads per workgroup for rows of `chunks` 16-byte chunks
int row_threads(int chunks) { return std::min(kMaxRowThreads, (chunks + 63) / 64 * 64); }

__global__ __launch_bounds__(kMaxRowThreads) void gather_rows_v16(const u32x4 *__restrict__ src,
                                                               const int32_t *__restrict__ idx,
                                                               u32x4 *__restrict__ dst, int chunks) {
  const long long row = blockIdx.x;
  const long long srow = idx[row];
  const u32x4 *s = src + srow * chunks;
  u32x4 *d = dst + row * chunks;
  for (int c = threadIdx.x; c < chunks; c += blockDim.x)
    __builtin_nontemporal_store(__builtin_nontemporal_load(s + c), d + c);
}

__global__ __launch_bounds__(kRowThreads) void gather_rows_u16(const uint16_t *__restrict__ src,
                                                               const int32_t *__restrict__ idx,
                                                               uint16_t *__restrict__ dst,
                                                               long long D) {
  const long long row = blockIdx.x;
  const long long srow = idx[row];
  for (long long c = threadIdx.x; c < D; c += kRowThreads) dst[row * D + c] = src[srow * D + c];
}

// blockIdx.y selects K (0) or V (1)
__global__ __launch_bounds__(kMaxRowThreads) void scatter_kv_v16(const u32x4 *__restrict__ kn,
                                                              const u32x4 *__restrict__ vn,
                                                              const int32_t *__restrict__ idx,
                                                              u32x4 *__restrict__ kc,
                                                              u32x4 *__restrict__ vc, int chunks) {
  const long long row = blockIdx.x;
  const long long drow = idx[row];
  const u32x4 *s = (blockIdx.y == 0 ? kn : vn) + row * chunks;
  u32x4 *d = (blockIdx.y == 0 ? kc : vc) + drow * chunks;
  for (int c = threadIdx.x; c < chunks; c += blockDim.x)
    __builtin_nontemporal_store(__builtin_nontemporal_load(s + c), d + c);
}

__global__ __launch_bounds__(kRowThreads) void scatter_kv_u16(const uint16_t *__restrict__ kn,
                                                              const uint16_t *__restrict__ vn,
                                                              const int32_t *__restrict__ idx,
                                                              uint16_t *__restrict__ kc,
                                                              uint16_t *__restrict__ vc,
                                                              long long D) {
  const long long row = blockIdx.x;
  const long long drow = idx[row];
  const uint16_t *s = blockIdx.y == 0 ? kn : vn;
  uint16_t *d = blockIdx.y == 0 ? kc : vc;
  for (long long c = threadIdx.x; c < D; c += kRowThreads) d[drow * D + c] = s[row * D + c];
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

hipError_t launch_gather_rows(const uint16_t *X, int64_t D, const int32_t *idx, int64_t n,
                              uint16_t *out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if ((D * 2) % 16 == 0 && aligned16(X) && aligned16(out)) {
    const int chunks = static_cast<int>(D * 2 / 16);
    hipLaunchKernelGGL(gather_rows_v16, dim3(static_cast<unsigned>(n)), dim3(row_threads(chunks)), 0, s,
                       reinterpret_cast<const u32x4 *>(X), idx, reinterpret_cast<u32x4 *>(out),
                       chunks);
  } else {
    hipLaunchKernelGGL(gather_rows_u16, dim3(static_cast<unsigned>(n)), dim3(kRowThreads), 0, s, X,
                       idx, out, static_cast<long long>(D));
  }
  return hipGetLastError();
}

hipError_t launch_scatter_kv(const uint16_t *Kn, const uint16_t *Vn, const int32_t *idx, int64_t n,
                             uint16_t *Kc, uint16_t *Vc, int64_t HD, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if ((HD * 2) % 16 == 0 && aligned16(Kn) && aligned16(Vn) && aligned16(Kc) && aligned16(Vc)) {
    const int chunks = static_cast<int>(HD * 2 / 16);
    hipLaunchKernelGGL(scatter_kv_v16, dim3(static_cast<unsigned>(n), 2), dim3(row_threads(chunks)), 0, s,
                       reinterpret_cast<const u32x4 *>(Kn), reinterpret_cast<const u32x4 *>(Vn), idx,
                       reinterpret_cast<u32x4 *>(Kc), reinterpret_cast<u32x4 *>(Vc), chunks);
  } else {
    hipLaunchKernelGGL(scatter_kv_u16, dim3(static_cast<unsigned>(n), 2), dim3(kRowThreads), 0, s,
                       Kn, Vn, idx, Kc, Vc, static_cast<long long>(HD));
  }
  return hipGetLastError();
}

}  // namespace jano
