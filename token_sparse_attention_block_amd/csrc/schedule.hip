// Interleaved-step schedule: compaction of the tokens due at one step into an
// ascending index list (gfx950).
//
// Method (Jano pages, nl methodology §2; zh §2.2 item 2): warm-up and
// cool-down steps recompute every token; in the interleaved phase Active
// tokens are recomputed every step, Moderate ones intermittently and Static
// ones rarely. Here a token of level L is due when (step - W) is a multiple
// of period[L-1]; the host turns that into a per-level `due` flag.
//
// The tokens are cut into chunks of kSchedChunk consecutive tokens, one
// workgroup each, with no communication between workgroups. A workgroup
// first finds where its chunk's indices start in the list: the number of due
// tokens before its first token n0. Every block contributes its due flag times
// the number of its tokens that precede n0, a closed form in the block's
// token box and n0's (f, h, w), so the workgroup sums that over all blocks
// (a fixed-order reduction: deterministic). It then marks its own tokens
// (each thread kSchedTok consecutive ones, stepped with counters rather than
// divisions), scans the per-thread counts and writes the due tokens at their
// offsets, so the list comes out ascending with no sort. The workgroup of the
// last chunk also writes the total. Each workgroup stages the block levels
// in LDS first (at most kMaxLevels bytes).
#include "common.hpp"
#include "kernels.hpp"

namespace jano {
namespace {

constexpr int kSchedThreads = 256;
constexpr int kSchedWaves = kSchedThreads / kWave;
constexpr int kSchedTok = 4;                              // tokens per thread
constexpr int kSchedChunk = kSchedThreads * kSchedTok;    // tokens per workgroup
constexpr int kMaxLevels = 16384;   // the analyzer's block limit

__device__ __forceinline__ bool is_due(int level, const SchedGeom &g) {
  return (level == 1 && g.due[0] != 0) || (level == 2 && g.due[1] != 0) ||
         (level == 3 && g.due[2] != 0);
}

// sum of v over the workgroup, in a fixed order; every thread gets it
__device__ __forceinline__ uint32_t wg_sum(uint32_t v, uint32_t *red) {
  const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
  v = wave_inclusive_scan(v);
  if (lane == kWave - 1) red[wv] = v;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int j = 0; j < kSchedWaves; ++j) t += red[j];
  __syncthreads();
  return t;
}

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(const uint8_t *__restrict__ levels,
                                                                 SchedGeom g, int B,
                                                                 int32_t *__restrict__ idx,
                                                                 int32_t *__restrict__ n_act) {
  __shared__ uint32_t red[kSchedWaves];
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  // block levels staged in LDS: 16-byte loads where the array allows, the
  // tail (and an unaligned array) byte by byte
  __shared__ __attribute__((aligned(16))) uint8_t lv[kMaxLevels];
  const int n16 = (reinterpret_cast<uintptr_t>(levels) & 15) == 0 ? B / 16 : 0;
  for (int i = tid; i < n16; i += kSchedThreads)
    reinterpret_cast<uint4 *>(lv)[i] = reinterpret_cast<const uint4 *>(levels)[i];
  for (int b = 16 * n16 + tid; b < B; b += kSchedThreads) lv[b] = levels[b];
  __syncthreads();
  const int HWt = g.Ht * g.Wt;
  const int rF = g.bF / g.pF, rH = g.bH / g.pH, rW = g.bW / g.pW;  // tokens per block edge
  const int n0 = blockIdx.x * kSchedChunk;
  const int f0 = n0 / HWt, h0 = (n0 - f0 * HWt) / g.Wt, w0 = n0 - f0 * HWt - h0 * g.Wt;

  // 1. due tokens before n0, one block row (bf, bh) per thread: a due block
  //    of width nw contributes nw per token row of the block row that lies
  //    wholly before n0, plus its columns before w0 in n0's own token row
  uint32_t before = 0;
  for (int r = tid; r < g.nBF * g.nBH; r += kSchedThreads) {
    const int bf = r / g.nBH, bh = r - bf * g.nBH;
    const int fa = bf * rF, fb = min(fa + rF, g.Ft);
    const int ha = bh * rH, hb = min(ha + rH, g.Ht);
    const int nh = hb - ha;
    const bool in_f = f0 >= fa && f0 < fb;
    const bool in_h = in_f && h0 >= ha && h0 < hb;
    const uint32_t rows_before = static_cast<uint32_t>(min(max(f0 - fa, 0), fb - fa) * nh +
                                                       (in_f ? min(max(h0 - ha, 0), nh) : 0));
    const uint8_t *row = lv + r * g.nBW;
    uint32_t width = 0, part = 0;
    for (int bw = 0, wa = 0; bw < g.nBW; ++bw, wa += rW) {
      if (!is_due(row[bw], g)) continue;
      const int nw = min(wa + rW, g.Wt) - wa;
      width += static_cast<uint32_t>(nw);
      if (in_h) part += static_cast<uint32_t>(min(max(w0 - wa, 0), nw));
    }
    before += width * rows_before + part;
  }
  const uint32_t start = wg_sum(before, red);

  // 2. this thread's kSchedTok tokens
  const int nt = n0 + tid * kSchedTok;
  uint32_t mask = 0;
  if (nt < g.N) {
    int f = nt / HWt;
    const int rem = nt - f * HWt;
    int h = rem / g.Wt;
    int w = rem - h * g.Wt;
    int bf = f / rF, fi = f - bf * rF;
    int bh = h / rH, hi = h - bh * rH;
    int bw = w / rW, wi = w - bw * rW;
#pragma unroll
    for (int u = 0; u < kSchedTok; ++u) {
      if (nt + u < g.N) {
        const bool d = is_due(lv[(bf * g.nBH + bh) * g.nBW + bw], g);
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
  // 3. offsets within the chunk: scan of the per-thread counts
  const uint32_t cnt = __popc(mask);
  const uint32_t incl = wave_inclusive_scan(cnt);
  if (lane == kWave - 1) red[wv] = incl;
  __syncthreads();
  uint32_t wave_before = 0, total = 0;
#pragma unroll
  for (int j = 0; j < kSchedWaves; ++j) {
    const uint32_t v = red[j];
    wave_before += j < wv ? v : 0u;
    total += v;
  }
  int pos = static_cast<int>(start + wave_before + incl - cnt);
  while (mask) {
    const int u = __builtin_ctz(mask);
    mask &= mask - 1;
    idx[pos++] = nt + u;
  }
  if (blockIdx.x == gridDim.x - 1 && tid == 0) *n_act = static_cast<int32_t>(start + total);
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
  if (B > kMaxLevels || g.N < 1) return hipErrorInvalidValue;
  const unsigned chunks = static_cast<unsigned>((g.N + kSchedChunk - 1) / kSchedChunk);
  hipLaunchKernelGGL(schedule_kernel, dim3(chunks), dim3(kSchedThreads), 0, s, levels, g, B, idx,
                     n_act);
  return hipGetLastError();
}

hipError_t launch_check_idx(const int32_t *idx, int64_t n, int64_t N, int32_t *flag,
                            hipStream_t s) {
  hipLaunchKernelGGL(check_idx_kernel, dim3(1), dim3(1024), 0, s, idx, static_cast<long long>(n),
                     static_cast<long long>(N), flag);
  return hipGetLastError();
}

}  // namespace jano
