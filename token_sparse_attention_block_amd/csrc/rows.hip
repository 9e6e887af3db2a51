// Row gather (adaptive token activation), KV-cache row scatter, and the
// write-back + sampler step of the token outputs (gfx950).
//
// Method (Jano pages, nl methodology §2 and contributions item 2; zh §2.2
// item 3): only the tokens due at a step are computed, and the key/value pairs
// of the frozen tokens stay in a cache; here the fresh rows of the active
// tokens are written into a persistent full-sequence cache at their token
// positions, so the cache always holds every token's latest K/V.
//
// Write-back (Jano pages, nl "three groups": the static group rests and its
// result is remembered; zh: static regions use the cache instead; ko §2:
// skipped parts keep the previous state in memory): the fresh model output of
// the active tokens replaces their rows of a full-sequence output buffer, and
// every token takes one Euler step x += dt * out with its latest output, so
// frozen tokens advance with the output cached at their last update.
//
// All kernels are pure HBM streams: one workgroup per row, sized to the row
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

// single-tensor row scatter: dst[idx[row]] = src[row]
__global__ __launch_bounds__(kMaxRowThreads) void scatter_rows_v16(const u32x4 *__restrict__ src,
                                                                const int32_t *__restrict__ idx,
                                                                u32x4 *__restrict__ dst, int chunks) {
  const long long row = blockIdx.x;
  const long long drow = idx[row];
  const u32x4 *s = src + row * chunks;
  u32x4 *d = dst + drow * chunks;
  for (int c = threadIdx.x; c < chunks; c += blockDim.x)
    __builtin_nontemporal_store(__builtin_nontemporal_load(s + c), d + c);
}

// The pages' layout of one interleaved step ([nl] methodology §2, [fr] §2.B):
// row r of Kcat/Vcat is the fresh row r of an active token for r < n_act and
// the cached row frozen[r - n_act] of a frozen token after that; positions
// are not restored. blockIdx.y selects K (0) or V (1).
__global__ __launch_bounds__(kMaxRowThreads) void concat_kv_v16(
    const u32x4 *__restrict__ kn, const u32x4 *__restrict__ vn, const u32x4 *__restrict__ kc,
    const u32x4 *__restrict__ vc, const int32_t *__restrict__ frozen, long long n_act,
    u32x4 *__restrict__ kcat, u32x4 *__restrict__ vcat, int chunks) {
  const long long row = blockIdx.x;
  const bool isk = blockIdx.y == 0;
  const u32x4 *s = row < n_act ? (isk ? kn : vn) + row * chunks
                               : (isk ? kc : vc) + static_cast<long long>(frozen[row - n_act]) * chunks;
  u32x4 *d = (isk ? kcat : vcat) + row * chunks;
  for (int c = threadIdx.x; c < chunks; c += blockDim.x)
    __builtin_nontemporal_store(__builtin_nontemporal_load(s + c), d + c);
}

__global__ __launch_bounds__(kRowThreads) void concat_kv_u16(
    const uint16_t *__restrict__ kn, const uint16_t *__restrict__ vn, const uint16_t *__restrict__ kc,
    const uint16_t *__restrict__ vc, const int32_t *__restrict__ frozen, long long n_act,
    uint16_t *__restrict__ kcat, uint16_t *__restrict__ vcat, long long D) {
  const long long row = blockIdx.x;
  const bool isk = blockIdx.y == 0;
  const uint16_t *s = row < n_act ? (isk ? kn : vn) + row * D
                                  : (isk ? kc : vc) + static_cast<long long>(frozen[row - n_act]) * D;
  uint16_t *d = (isk ? kcat : vcat) + row * D;
  for (long long c = threadIdx.x; c < D; c += kRowThreads) d[c] = s[c];
}

// rows of at most 32 chunks: several rows per workgroup, one thread per chunk
constexpr int kSmallRowThreads = 256;
__global__ __launch_bounds__(kSmallRowThreads) void scatter_rows_small_v16(const u32x4 *__restrict__ src,
                                                                       const int32_t *__restrict__ idx,
                                                                       u32x4 *__restrict__ dst,
                                                                       int chunks, long long n) {
  const int rows_per_wg = kSmallRowThreads / chunks;
  const int t = threadIdx.x;
  if (t >= rows_per_wg * chunks) return;
  const long long row = static_cast<long long>(blockIdx.x) * rows_per_wg + t / chunks;
  if (row >= n) return;
  const int c = t % chunks;
  const long long drow = idx[row];
  __builtin_nontemporal_store(__builtin_nontemporal_load(src + row * chunks + c), dst + drow * chunks + c);
}

__global__ __launch_bounds__(kRowThreads) void scatter_rows_u16(const uint16_t *__restrict__ src,
                                                                const int32_t *__restrict__ idx,
                                                                uint16_t *__restrict__ dst,
                                                                long long D) {
  const long long row = blockIdx.x;
  const long long drow = idx[row];
  for (long long c = threadIdx.x; c < D; c += kRowThreads) dst[drow * D + c] = src[row * D + c];
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

constexpr int kEulerThreads = 256;
constexpr int kEulerMaxBlocks = 8192;

// x[e] = fma(dt, v[e], x[e]) over a flat array, 8 elements per thread and step
__global__ __launch_bounds__(kEulerThreads) void euler_v8(const u32x4 *__restrict__ v,
                                                          f32x4 *__restrict__ x, long long n8,
                                                          float dt) {
  for (long long i = static_cast<long long>(blockIdx.x) * kEulerThreads + threadIdx.x; i < n8;
       i += static_cast<long long>(gridDim.x) * kEulerThreads) {
    const u32x4 w = __builtin_nontemporal_load(v + i);
    f32x4 a = x[2 * i], b = x[2 * i + 1];
    a.x = fmaf(dt, bf16_lo(w.x), a.x);
    a.y = fmaf(dt, bf16_hi(w.x), a.y);
    a.z = fmaf(dt, bf16_lo(w.y), a.z);
    a.w = fmaf(dt, bf16_hi(w.y), a.w);
    b.x = fmaf(dt, bf16_lo(w.z), b.x);
    b.y = fmaf(dt, bf16_hi(w.z), b.y);
    b.z = fmaf(dt, bf16_lo(w.w), b.z);
    b.w = fmaf(dt, bf16_hi(w.w), b.w);
    __builtin_nontemporal_store(a, x + 2 * i);
    __builtin_nontemporal_store(b, x + 2 * i + 1);
  }
}

__global__ __launch_bounds__(kEulerThreads) void euler_scalar(const uint16_t *__restrict__ v,
                                                              float *__restrict__ x, long long lo,
                                                              long long hi, float dt) {
  for (long long e = lo + static_cast<long long>(blockIdx.x) * kEulerThreads + threadIdx.x; e < hi;
       e += static_cast<long long>(gridDim.x) * kEulerThreads)
    x[e] = fmaf(dt, __uint_as_float(static_cast<uint32_t>(v[e]) << 16), x[e]);
}

int euler_blocks(long long work) {
  const long long b = (work + kEulerThreads - 1) / kEulerThreads;
  return static_cast<int>(b < 1 ? 1 : (b > kEulerMaxBlocks ? kEulerMaxBlocks : b));
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

hipError_t launch_scatter_rows(const uint16_t *src, int64_t D, const int32_t *idx, int64_t n,
                               uint16_t *dst, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if ((D * 2) % 16 == 0 && aligned16(src) && aligned16(dst)) {
    const int chunks = static_cast<int>(D * 2 / 16);
    if (chunks <= 32) {
      const long long per = kSmallRowThreads / chunks;
      hipLaunchKernelGGL(scatter_rows_small_v16, dim3(static_cast<unsigned>((n + per - 1) / per)),
                         dim3(kSmallRowThreads), 0, s, reinterpret_cast<const u32x4 *>(src), idx,
                         reinterpret_cast<u32x4 *>(dst), chunks, static_cast<long long>(n));
      return hipGetLastError();
    }
    hipLaunchKernelGGL(scatter_rows_v16, dim3(static_cast<unsigned>(n)), dim3(row_threads(chunks)), 0, s,
                       reinterpret_cast<const u32x4 *>(src), idx, reinterpret_cast<u32x4 *>(dst), chunks);
  } else {
    hipLaunchKernelGGL(scatter_rows_u16, dim3(static_cast<unsigned>(n)), dim3(kRowThreads), 0, s, src,
                       idx, dst, static_cast<long long>(D));
  }
  return hipGetLastError();
}

hipError_t launch_concat_kv(const uint16_t *Kn, const uint16_t *Vn, int64_t n_act, const uint16_t *Kc,
                            const uint16_t *Vc, const int32_t *frozen, int64_t n_frozen, uint16_t *Kcat,
                            uint16_t *Vcat, int64_t HD, hipStream_t s) {
  const int64_t rows = n_act + n_frozen;
  if (rows == 0) return hipSuccess;
  const bool fresh_ok = n_act == 0 || (aligned16(Kn) && aligned16(Vn));
  if ((HD * 2) % 16 == 0 && fresh_ok && aligned16(Kc) && aligned16(Vc) && aligned16(Kcat) &&
      aligned16(Vcat)) {
    const int chunks = static_cast<int>(HD * 2 / 16);
    hipLaunchKernelGGL(concat_kv_v16, dim3(static_cast<unsigned>(rows), 2), dim3(row_threads(chunks)), 0, s,
                       reinterpret_cast<const u32x4 *>(Kn), reinterpret_cast<const u32x4 *>(Vn),
                       reinterpret_cast<const u32x4 *>(Kc), reinterpret_cast<const u32x4 *>(Vc), frozen,
                       static_cast<long long>(n_act), reinterpret_cast<u32x4 *>(Kcat),
                       reinterpret_cast<u32x4 *>(Vcat), chunks);
  } else {
    hipLaunchKernelGGL(concat_kv_u16, dim3(static_cast<unsigned>(rows), 2), dim3(kRowThreads), 0, s, Kn, Vn,
                       Kc, Vc, frozen, static_cast<long long>(n_act), Kcat, Vcat, static_cast<long long>(HD));
  }
  return hipGetLastError();
}

hipError_t launch_euler(const uint16_t *v, float *x, int64_t total, float dt, hipStream_t s) {
  long long done = 0;
  if (aligned16(v) && aligned16(x)) {
    const long long n8 = total / 8;
    if (n8 > 0)
      hipLaunchKernelGGL(euler_v8, dim3(euler_blocks(n8)), dim3(kEulerThreads), 0, s,
                         reinterpret_cast<const u32x4 *>(v), reinterpret_cast<f32x4 *>(x), n8, dt);
    done = n8 * 8;
  }
  if (done < total)
    hipLaunchKernelGGL(euler_scalar, dim3(euler_blocks(total - done)), dim3(kEulerThreads), 0, s, v, x,
                       done, static_cast<long long>(total), dt);
  return hipGetLastError();
}

}  // namespace jano
