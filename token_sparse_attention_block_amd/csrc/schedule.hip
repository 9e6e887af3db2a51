// Interleaved-step schedule: compaction of the tokens due at one step into an
// ascending index list (gfx950).
//
// Method (Jano pages, nl methodology §2; zh §2.2 item 2): warm-up and
// cool-down steps recompute every token; in the interleaved phase Active
// tokens are recomputed every step, Moderate ones intermittently and Static
// ones rarely. Here a token of level L is due when (step - W) is a multiple
// of period[L-1]; the host turns that into a per-level `due` flag.
//
// One workgroup of 1024 threads walks the tokens in slices of 1024*kUnroll.
// Within a slice every wave ballots its 64 predicates per sub-slice, counts
// with popcount, and places each due token with mbcnt (number of due lanes
// below it); wave totals are scanned in LDS in token order. Writes are
// contiguous per wave, so the list comes out ascending with no sort.
#include "common.hpp"
#include "kernels.hpp"

namespace jano {
namespace {

constexpr int kSchedThreads = 1024;
constexpr int kSchedWaves = kSchedThreads / kWave;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(const uint8_t *__restrict__ levels,
                                                                 SchedGeom g,
                                                                 int32_t *__restrict__ idx,
                                                                 int32_t *__restrict__ n_act) {
  __shared__ int wcount[kUnroll * kSchedWaves];
  __shared__ int woffset[kUnroll * kSchedWaves + 1];
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const int HWt = g.Ht * g.Wt;
  const int rF = g.bF / g.pF, rH = g.bH / g.pH, rW = g.bW / g.pW;  // tokens per block edge
  int running = 0;
  for (int base = 0; base < g.N; base += kSchedThreads * kUnroll) {
    bool due[kUnroll];
    uint64_t mask[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int n = base + u * kSchedThreads + tid;
      bool d = false;
      if (n < g.N) {
        const int f = n / HWt, rem = n - f * HWt;
        const int h = rem / g.Wt, w = rem - h * g.Wt;
        const int b = ((f / rF) * g.nBH + h / rH) * g.nBW + w / rW;
        const int lv = levels[b];
        d = (lv >= 1 && lv <= 3) ? g.due[lv - 1] != 0 : false;
      }
      due[u] = d;
      mask[u] = __ballot(d);
    }
    if (lane == 0) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) wcount[u * kSchedWaves + wv] = __popcll(mask[u]);
    }
    __syncthreads();
    if (tid == 0) {
      int acc = 0;
      for (int i = 0; i < kUnroll * kSchedWaves; ++i) {
        woffset[i] = acc;
        acc += wcount[i];
      }
      woffset[kUnroll * kSchedWaves] = acc;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (due[u]) {
        const int n = base + u * kSchedThreads + tid;
        idx[running + woffset[u * kSchedWaves + wv] + lanes_below(mask[u])] = n;
      }
    }
    running += woffset[kUnroll * kSchedWaves];
    __syncthreads();
  }
  if (tid == 0) *n_act = running;
}

__global__ __launch_bounds__(1024) void check_idx_kernel(const int32_t *__restrict__ idx,
                                                         long long n, long long N,
                                                         int32_t *__restrict__ flag) {
  bool bad = false;
  for (long long i = threadIdx.x; i < n; i += blockDim.x) {
    const int v = idx[i];
    if (v < 0 || v >= N) bad = true;
    if (i > 0 && v <= idx[i - 1]) bad = true;
  }
  const int any_bad = __syncthreads_or(bad ? 1 : 0);
  if (threadIdx.x == 0) *flag = any_bad ? -3 /* JANO_E_RANGE */ : 0;
}

}  // namespace

hipError_t launch_schedule(const uint8_t *levels, const SchedGeom &g, int32_t *idx,
                           int32_t *n_act, hipStream_t s) {
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kSchedThreads), 0, s, levels, g, idx, n_act);
  return hipGetLastError();
}

hipError_t launch_check_idx(const int32_t *idx, int64_t n, int64_t N, int32_t *flag,
                            hipStream_t s) {
  hipLaunchKernelGGL(check_idx_kernel, dim3(1), dim3(1024), 0, s, idx, static_cast<long long>(n),
                     static_cast<long long>(N), flag);
  return hipGetLastError();
}

}  // namespace jano
