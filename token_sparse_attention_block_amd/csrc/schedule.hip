// Interleaved-step schedule: compaction of the tokens due at one step into an
// ascending index list (gfx950).
//
// Method (Jano pages, nl methodology §2; zh §2.2 item 2): warm-up and
// cool-down steps recompute every token; in the interleaved phase Active
// tokens are recomputed every step, Moderate ones intermittently and Static
// ones rarely. Here a token of level L is due when (step - W) is a multiple
// of period[L-1]; the host turns that into a per-level `due` flag.
//
// One workgroup of 1024 threads walks the tokens in slices of 1024*kPerThread.
// The block levels are staged in LDS. Each thread owns kPerThread consecutive
// tokens: it derives (f, h, w) and the block coordinates once and then steps
// them with counters (no division per token), collects a due bit-mask,
// and the slice's per-thread counts are prefix-summed (wave scans plus one
// pass over the wave totals). Each thread then writes its due tokens at its
// offset, so the list comes out ascending with no sort.
#include "common.hpp"
#include "kernels.hpp"

namespace jano {
namespace {

constexpr int kSchedThreads = 1024;
constexpr int kSchedWaves = kSchedThreads / kWave;
constexpr int kPerThread = 16;
constexpr int kMaxLevels = 16384;   // the analyzer's block limit

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(const uint8_t *__restrict__ levels,
                                                                 SchedGeom g, int B,
                                                                 int32_t *__restrict__ idx,
                                                                 int32_t *__restrict__ n_act) {
  __shared__ uint8_t lv[kMaxLevels];
  __shared__ uint32_t wsum[kSchedWaves];
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  for (int b = tid; b < B; b += kSchedThreads) lv[b] = levels[b];
  const int HWt = g.Ht * g.Wt;
  const int rF = g.bF / g.pF, rH = g.bH / g.pH, rW = g.bW / g.pW;  // tokens per block edge
  const bool due1 = g.due[0] != 0, due2 = g.due[1] != 0, due3 = g.due[2] != 0;
  __syncthreads();
  int running = 0;
  for (int base = 0; base < g.N; base += kSchedThreads * kPerThread) {
    const int n0 = base + tid * kPerThread;
    uint32_t mask = 0;
    if (n0 < g.N) {
      int f = n0 / HWt;
      const int rem = n0 - f * HWt;
      int h = rem / g.Wt;
      int w = rem - h * g.Wt;
      int bf = f / rF, fi = f - bf * rF;
      int bh = h / rH, hi = h - bh * rH;
      int bw = w / rW, wi = w - bw * rW;
#pragma unroll
      for (int u = 0; u < kPerThread; ++u) {
        if (n0 + u < g.N) {
          const int l = lv[(bf * g.nBH + bh) * g.nBW + bw];
          const bool d = (l == 1 && due1) || (l == 2 && due2) || (l == 3 && due3);
          mask |= static_cast<uint32_t>(d) << u;
        }
        // advance to the next token in (f, h, w) order
        if (++wi == rW) { wi = 0; ++bw; }
        if (++w == g.Wt) {
          w = 0; bw = 0; wi = 0;
          if (++hi == rH) { hi = 0; ++bh; }
          if (++h == g.Ht) {
            h = 0; bh = 0; hi = 0;
            if (++fi == rF) { fi = 0; ++bf; }
            ++f;
          }
        }
      }
    }
    const uint32_t cnt = __popc(mask);
    const uint32_t incl = wave_inclusive_scan(cnt);
    if (lane == kWave - 1) wsum[wv] = incl;
    __syncthreads();
    uint32_t before = 0, total = 0;
    for (int j = 0; j < kSchedWaves; ++j) {
      const uint32_t v = wsum[j];
      before += j < wv ? v : 0u;
      total += v;
    }
    int pos = running + static_cast<int>(before + incl - cnt);
    while (mask) {
      const int u = __builtin_ctz(mask);
      mask &= mask - 1;
      idx[pos++] = n0 + u;
    }
    running += static_cast<int>(total);
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
  const int B = g.nBF * g.nBH * g.nBW;
  if (B > kMaxLevels) return hipErrorInvalidValue;
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kSchedThreads), 0, s, levels, g, B, idx, n_act);
  return hipGetLastError();
}

hipError_t launch_check_idx(const int32_t *idx, int64_t n, int64_t N, int32_t *flag,
                            hipStream_t s) {
  hipLaunchKernelGGL(check_idx_kernel, dim3(1), dim3(1024), 0, s, idx, static_cast<long long>(n),
                     static_cast<long long>(N), flag);
  return hipGetLastError();
}

}  // namespace jano
