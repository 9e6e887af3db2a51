// Block-wise complexity analyzer and level bucketing (gfx950).
//
// Method (Jano pages, zh technical summary §2.1; nl methodology §1): split the
// latent into 3D frame x height x width blocks, take temporal and spatial
// gradients of the first K warm-up latents, difference them twice along the
// step axis, and turn the variation into one score per block; bucket blocks
// into Static / Moderate / Active.
//
// Score of block b: mean over (axis a in {F,H,W} with extent >= 2,
// k = 1..K-2, channel c, position p in b with p+e_a inside the latent) of
// |D_k(c, p+e_a) - D_k(c, p)|, D_k = L_{k+1} - 2 L_k + L_{k-1} in fp64.
//
// Kernel 1 (analyze_stream_kernel) is a single streaming pass over the fp32
// latents. One wave owns one channel, one strip of R latent rows of a block
// row, a chunk of CW (< 64) columns and a chunk of FC frames:
//   * lanes run along W (coalesced 256-byte row loads), so the +w neighbour
//     is one lane over (the lane after the chunk loads the halo column);
//   * each lane keeps its R+1 rows (R owned + 1 halo row) in registers, so
//     the +h neighbour is the next register;
//   * frames are streamed, so the +f neighbour is the previous iteration's
//     registers (one halo frame is read past the chunk).
// Every input value is read from HBM once; halos are re-read from cache.
// D and the terms are formed in fp64 (for fp32 latents D is exact), summed
// per lane, reduced over the block's lanes with a fixed shuffle tree and
// written as one fp64 partial per (channel, strip, block): no atomics, so the
// result is deterministic.
//
// Kernel 2 (block_scores_kernel, one thread per block) sums the partials in a
// fixed order, divides by the closed-form term count and rounds the score to
// fp32. Kernels 1 and 2 are jano_analyze_scores.
//
// The FFT complexity baseline (jano_fft_scores, an alternative index source
// whose scores go through the same levels) is fft_scores_kernel.
//
// Levels (jano_levels): kernel 3 (rank_levels_kernel) gives every block its
// exact rank in the (score, block id) order and the level that rank falls in;
// kernel 4 (level_counts_kernel, one workgroup) counts the tokens of each
// level, with each block's token count in closed form from the grid.
//
// Grid mapping of kernel 1: workgroups are renumbered XCD-aware and waves are
// ordered column chunk fastest, then strip, then frame chunk, so the waves
// that re-read each other's halo cache lines run on one XCD (one L2) at the
// same time.
#include "common.hpp"
#include "kernels.hpp"

namespace jano {
namespace {

constexpr int kAnalyzeWaves = 1;          // waves per workgroup of kernel 1 (single-wave
                                          // workgroups refill freed slots at the finest grain)
constexpr int kXcds = 8;                  // accelerator dies (each with an L2) per GPU
constexpr int kRankThreads = 1024;        // kernel 3 workgroup size
constexpr int kRankSplit = 32;            // kernel 3 threads per block (one per 16 bytes of a 512-byte row)
constexpr int kCountThreads = 1024;       // kernel 4 is one workgroup
constexpr int kMaxBlocks = 16384;         // kernel 3 keeps all scores in LDS (a multiple of 128)
#ifndef JANO_ANALYZE_TARGET_WAVES
#define JANO_ANALYZE_TARGET_WAVES 2304    // about 1.1 x the waves one pass of the GPU holds
#endif
constexpr int kTargetWaves = JANO_ANALYZE_TARGET_WAVES;  // waves wanted in the grid

__device__ __forceinline__ void flush_block_sum(double acc, const AnalyzeGeom &g, int lane,
                                                int w0, int c, int sg, int bf, int bh,
                                                double *__restrict__ part) {
  // segmented tree reduction over the bW lanes of each block column
  const int pos = lane % g.bW;
  for (int off = 1; off < g.bW; off <<= 1) {
    const double v = shfl_down_f64(acc, off);
    if (pos + off < g.bW) acc += v;
  }
  const int w = w0 + lane;
  if (pos == 0 && lane < g.CW && w < g.W) {
    const int b = (bf * g.nBH + bh) * g.nBW + w / g.bW;
    part[(static_cast<size_t>(c) * g.G + sg) * g.B + b] = acc;
  }
}

// Value held by lane + 1 (DPP wavefront shift, a plain VALU move). Lane 63
// receives 0; it never owns a gradient term (a wave owns at most 63 columns).
__device__ __forceinline__ double from_next_lane(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const int lo = __builtin_amdgcn_mov_dpp(static_cast<int>(u), 0x130, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_mov_dpp(static_cast<int>(u >> 32), 0x130, 0xF, 0xF, true);
  return __builtin_bit_cast(double, (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) |
                                        static_cast<uint32_t>(lo));
}

// One (K, R) strip of one wave, streamed over its frame chunk. FULL: all R+1
// rows (R owned + the +h halo row) lie inside the latent, so no row needs a
// predicate; otherwise rows past the bottom edge are excluded term by term.
template <int KT, int R, bool FULL>
__device__ __forceinline__ void stream_strip(__amdgpu_buffer_rsrc_t rsrc, const AnalyzeGeom &g,
                                             const uint32_t (&lane_off)[R + 1], int c, int f0,
                                             int f_last, int f_end, int rows_loaded,
                                             int rows_owned, bool own, bool has_wn, int lane,
                                             int w0, int sg, int bh, double *__restrict__ part) {
  constexpr int KD = KT - 2;
  const uint32_t plane_b = static_cast<uint32_t>(g.H) * g.W * 4u;
  const uint32_t kstride_b = static_cast<uint32_t>(g.C) * g.F * plane_b;
  const uint32_t cbase_b = static_cast<uint32_t>(c) * g.F * plane_b;

  double acc = 0.0;

  // The next frame's loads are issued before the current frame is computed,
  // so memory latency overlaps the fp64 work. Frames alternate between two
  // register sets (x, D), so nothing is copied from one frame to the next.
  auto load_frame = [&](int f, float (&xn)[KT][R + 1]) {
    const uint32_t fb = cbase_b + static_cast<uint32_t>(f) * plane_b;
#pragma unroll
    for (int k = 0; k < KT; ++k)
#pragma unroll
      for (int r = 0; r <= R; ++r)
        xn[k][r] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rsrc, lane_off[r], fb + k * kstride_b, 0));
  };
  // processes frame f held in x (D_prev: the previous frame's D), prefetching
  // frame f+1 into xn and leaving this frame's D in D_cur
  auto frame = [&](int f, float (&x)[KT][R + 1], float (&xn)[KT][R + 1],
                   const double (&D_prev)[KD][R + 1], double (&D)[KD][R + 1]) {
    if (f < f_end) load_frame(f + 1, xn);
#pragma unroll
    for (int k = 0; k < KD; ++k)
#pragma unroll
      for (int r = 0; r <= R; ++r)
        D[k][r] = (static_cast<double>(x[k + 2][r]) - 2.0 * static_cast<double>(x[k + 1][r])) +
                  static_cast<double>(x[k][r]);
    if (f > f0) {
      // temporal terms of frame f-1 (pairs f-1 -> f), booked to block of f-1
      double t = 0.0;
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int k = 0; k < KD; ++k)
          if (FULL || r < rows_owned) t += fabs(D[k][r] - D_prev[k][r]);
      if (own) acc += t;
      const int bprev = (f - 1) / g.bF;
      if (f > f_last || f / g.bF != bprev) {
        flush_block_sum(acc, g, lane, w0, c, sg, bprev, bh, part);
        acc = 0.0;
      }
    }
    if (f <= f_last) {
      double th = 0.0, tw = 0.0;   // +h terms, +w terms
#pragma unroll
      for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int k = 0; k < KD; ++k) {
          const double right = from_next_lane(D[k][r]);   // +w neighbour
          if (FULL || r < rows_owned) tw += fabs(right - D[k][r]);
          if (FULL || r + 1 < rows_loaded) th += fabs(D[k][r + 1] - D[k][r]);
        }
      }
      if (own) acc += th;
      if (has_wn) acc += tw;
    }
  };

  float xa[KT][R + 1], xb[KT][R + 1];
  double Da[KD][R + 1], Db[KD][R + 1];
#pragma unroll
  for (int k = 0; k < KD; ++k)
#pragma unroll
    for (int r = 0; r <= R; ++r) Db[k][r] = 0.0;
  load_frame(f0, xa);
  for (int f = f0; f <= f_end; f += 2) {
    frame(f, xa, xb, Db, Da);
    if (f + 1 > f_end) break;
    frame(f + 1, xb, xa, Da, Db);
  }
  if (f_end == f_last) flush_block_sum(acc, g, lane, w0, c, sg, f_last / g.bF, bh, part);
}

template <int KT, int R>
__global__ __launch_bounds__(kAnalyzeWaves * kWave) void analyze_stream_kernel(
    const float *__restrict__ lat, AnalyzeGeom g, double *__restrict__ part, int total_waves) {
  // Workgroups are dispatched round-robin over the XCDs, each with its own
  // L2. Renumber them so that consecutive logical workgroups -- which read
  // each other's halo rows, columns and frames -- run on the same XCD.
  const int nwg = gridDim.x, xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int logical = xcd * (nwg / kXcds) + min(xcd, nwg % kXcds) + slot;
  // wave index made provably uniform, so everything derived from it stays in
  // scalar registers (buffer offsets must be scalar)
  const int wave = __builtin_amdgcn_readfirstlane(logical * kAnalyzeWaves + (threadIdx.x / kWave));
  if (wave >= total_waves) return;  // uniform per wave
  const int lane = threadIdx.x % kWave;

  // column chunk fastest, then strip, then frame chunk, then channel
  const int nStrips = g.nBH * g.G;
  int q = wave;
  const int wc = q % g.nWC;
  q /= g.nWC;
  const int strip = q % nStrips;
  q /= nStrips;
  const int fc = q % g.nFC;
  const int c = q / g.nFC;

  const int bh = strip / g.G, sg = strip % g.G;
  const int h0 = bh * g.bH + sg * R;
  const int w0 = wc * g.CW;
  const int w = w0 + lane;
  const bool own = lane < g.CW && w < g.W;      // owns gradient terms
  const bool has_wn = own && (w + 1 < g.W);
  const int rows_loaded = min(R + 1, g.H - h0);  // may be <= 0 for empty strips
  const int rows_owned = min(R, g.H - h0);

  const int f0 = fc * g.FC;
  const int f_last = min(f0 + g.FC, g.F) - 1;   // last owned frame
  const int f_end = min(f0 + g.FC, g.F - 1);    // last loaded frame (halo)

  // Loads go through a buffer resource (wave-uniform base, 32-bit offsets).
  // Every load is issued unconditionally from a clamped in-bounds offset;
  // clamped rows and columns hold real latent values and every term that
  // would use them is excluded, so they need no masking.
  const uint32_t bytes = static_cast<uint32_t>(static_cast<size_t>(g.K) * g.C * g.F * g.H * g.W * 4);
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(lat), 0, bytes, 0x00020000);
  uint32_t lane_off[R + 1];
#pragma unroll
  for (int r = 0; r <= R; ++r)
    lane_off[r] = static_cast<uint32_t>(min(h0 + r, g.H - 1) * g.W + min(w, g.W - 1)) * 4u;

  if (rows_loaded == R + 1)
    stream_strip<KT, R, true>(rsrc, g, lane_off, c, f0, f_last, f_end, rows_loaded, rows_owned,
                              own, has_wn, lane, w0, sg, bh, part);
  else
    stream_strip<KT, R, false>(rsrc, g, lane_off, c, f0, f_last, f_end, rows_loaded, rows_owned,
                               own, has_wn, lane, w0, sg, bh, part);
}

// Slow path for shapes the streaming kernel does not cover (K > 8, odd block
// heights, blocks wider than a wave): one thread per (channel, block), direct
// global reads. Same definition, same partial layout with G = 1.
__global__ __launch_bounds__(256) void analyze_generic_kernel(const float *__restrict__ lat,
                                                              AnalyzeGeom g,
                                                              double *__restrict__ part) {
  const long long t = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= static_cast<long long>(g.C) * g.B) return;
  const int c = static_cast<int>(t / g.B);
  const int b = static_cast<int>(t % g.B);
  const int bw = b % g.nBW, bh = (b / g.nBW) % g.nBH, bf = b / (g.nBW * g.nBH);
  const size_t plane = static_cast<size_t>(g.H) * g.W;
  const size_t kstride = static_cast<size_t>(g.C) * g.F * plane;
  auto Dat = [&](int k, int f, int h, int w) {
    const float *p = lat + (static_cast<size_t>(c) * g.F + f) * plane + static_cast<size_t>(h) * g.W + w;
    return (static_cast<double>(p[(k + 1) * kstride]) - 2.0 * static_cast<double>(p[k * kstride])) +
           static_cast<double>(p[(k - 1) * kstride]);
  };
  double acc = 0.0;
  for (int f = bf * g.bF; f < min((bf + 1) * g.bF, g.F); ++f)
    for (int h = bh * g.bH; h < min((bh + 1) * g.bH, g.H); ++h)
      for (int w = bw * g.bW; w < min((bw + 1) * g.bW, g.W); ++w)
        for (int k = 1; k + 1 < g.K; ++k) {
          const double d0 = Dat(k, f, h, w);
          if (f + 1 < g.F) acc += fabs(Dat(k, f + 1, h, w) - d0);
          if (h + 1 < g.H) acc += fabs(Dat(k, f, h + 1, w) - d0);
          if (w + 1 < g.W) acc += fabs(Dat(k, f, h, w + 1) - d0);
        }
  part[static_cast<size_t>(c) * g.B + b] = acc;
}

__device__ __forceinline__ long long axis_terms(int lo, int hi, int ext) {
  // positions in [lo, hi) that have a +1 neighbour inside [0, ext)
  return max(0, min(hi, ext - 1) - lo);
}

__device__ __forceinline__ int axis_tokens(int j, int per_block, int ntok) {
  return max(0, min((j + 1) * per_block, ntok) - j * per_block);
}

// Kernel 2: per-block score (fixed-order sum of the partials over channels
// and strips, divided by the closed-form term count, rounded to fp32). One
// thread per block.
__global__ __launch_bounds__(256) void block_scores_kernel(const double *__restrict__ part,
                                                           AnalyzeGeom g,
                                                           float *__restrict__ scores) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= g.B) return;
  const int B = g.B, CG = g.C * g.G;
  double t = 0.0;
  constexpr int kJ = 16;   // loads in flight per thread; summed in j order
  for (int j0 = 0; j0 < CG; j0 += kJ) {
    double v[kJ];
#pragma unroll
    for (int jj = 0; jj < kJ; ++jj)
      v[jj] = j0 + jj < CG ? part[static_cast<size_t>(j0 + jj) * B + b] : 0.0;
#pragma unroll
    for (int jj = 0; jj < kJ; ++jj) t += v[jj];
  }
  const int bw = b % g.nBW, bh = (b / g.nBW) % g.nBH, bf = b / (g.nBW * g.nBH);
  const int f0 = bf * g.bF, f1 = min(f0 + g.bF, g.F);
  const int h0 = bh * g.bH, h1 = min(h0 + g.bH, g.H);
  const int w0 = bw * g.bW, w1 = min(w0 + g.bW, g.W);
  const long long ef = f1 - f0, eh = h1 - h0, ew = w1 - w0;
  const long long pos = (g.F >= 2 ? axis_terms(f0, f1, g.F) * eh * ew : 0) +
                        (g.H >= 2 ? axis_terms(h0, h1, g.H) * ef * ew : 0) +
                        (g.W >= 2 ? axis_terms(w0, w1, g.W) * ef * eh : 0);
  const long long n = pos * (g.K - 2) * g.C;
  scores[b] = n > 0 ? static_cast<float>(t / static_cast<double>(n)) : 0.0f;
}

// Kernel 3: the level of every block from its exact rank in the (score,
// block id) order -- the number of blocks with a smaller score, or an equal
// score and a smaller id. kRankSplit = 32 threads count one block's rank; each
// workgroup stages all score bits in LDS (scores are >= 0, so their fp32 bit
// patterns order like the values), padded to whole rows of 128 with
// 0xFFFFFFFF, which no score reaches. Lane p of a block's 32 reads scores
// 4p .. 4p+3 of every 128-score row (together one contiguous 512-byte row, no
// bank conflicts). Rows wholly below block b count "score <= s", rows above
// count "score < s", and the row holding b compares ids element by element.
// Integer counts make the result exact and independent of scheduling.
__global__ __launch_bounds__(kRankThreads) void rank_levels_kernel(const float *__restrict__ scores,
                                                                   int B, int nS, int nSM,
                                                                   uint8_t *__restrict__ levels) {
  __shared__ __attribute__((aligned(16))) uint32_t sc[kMaxBlocks];
  const int tid = threadIdx.x;
  const int nrows = (B + 127) / 128;
  // stage the score bits: eight independent loads in flight per thread
  for (int i0 = tid; i0 < nrows * 128; i0 += 8 * kRankThreads) {
    uint32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * kRankThreads;
      v[u] = i < B ? __float_as_uint(scores[i]) : 0xFFFFFFFFu;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * kRankThreads;
      if (i < nrows * 128) sc[i] = v[u];
    }
  }
  __syncthreads();
  const int b = blockIdx.x * (kRankThreads / kRankSplit) + tid / kRankSplit;
  const int part = tid % kRankSplit;
  int cnt = 0;
  if (b < B) {
    const uint32_t s = sc[b];
    const int rb = b / 128;
    const uint32_t *p = &sc[4 * part];
    for (int r = 0; r < rb; ++r) {
      const uint4 t = *reinterpret_cast<const uint4 *>(p + 128 * r);
      cnt += (t.x <= s) + (t.y <= s) + (t.z <= s) + (t.w <= s);
    }
    {
      const uint4 t = *reinterpret_cast<const uint4 *>(p + 128 * rb);
      const int j = 128 * rb + 4 * part;
      const uint32_t tv[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        cnt += j + e < b ? (tv[e] <= s) : (j + e > b ? (tv[e] < s) : 0);
    }
    for (int r = rb + 1; r < nrows; ++r) {
      const uint4 t = *reinterpret_cast<const uint4 *>(p + 128 * r);
      cnt += (t.x < s) + (t.y < s) + (t.z < s) + (t.w < s);
    }
  }
#pragma unroll
  for (int off = kRankSplit / 2; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off, kWave);
  if (b < B && part == 0) levels[b] = static_cast<uint8_t>(cnt < nS ? 1 : (cnt < nSM ? 2 : 3));
}

// Kernel 4 (one workgroup): tokens per level; a block holds the tokens of its
// (possibly ragged) extent in the token grid.
__global__ __launch_bounds__(kCountThreads) void level_counts_kernel(const uint8_t *__restrict__ levels,
                                                                     AnalyzeGeom g,
                                                                     int32_t *__restrict__ counts) {
  __shared__ uint32_t part[3][kCountThreads / kWave];
  const int tid = threadIdx.x;
  const int tpbF = g.bF / g.pF, tpbH = g.bH / g.pH, tpbW = g.bW / g.pW;
  const int Ft = g.F / g.pF, Ht = g.H / g.pH, Wt = g.W / g.pW;
  uint32_t my[3] = {0u, 0u, 0u};
  // all of this thread's levels are loaded before any is used (one wait)
  constexpr int kPer = kMaxBlocks / kCountThreads;
  int lvr[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int b = tid + k * kCountThreads;
    lvr[k] = b < g.B ? levels[b] : 0;
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int b = tid + k * kCountThreads;
    if (b >= g.B) break;
    const int bw = b % g.nBW, bh = (b / g.nBW) % g.nBH, bf = b / (g.nBW * g.nBH);
    const uint32_t tok = static_cast<uint32_t>(axis_tokens(bf, tpbF, Ft) * axis_tokens(bh, tpbH, Ht) *
                                               axis_tokens(bw, tpbW, Wt));
#pragma unroll
    for (int i = 0; i < 3; ++i) my[i] += lvr[k] == i + 1 ? tok : 0u;
  }
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const uint32_t wsum = __shfl(wave_inclusive_scan(my[i]), kWave - 1, kWave);
    if (tid % kWave == 0) part[i][tid / kWave] = wsum;
  }
  __syncthreads();
  if (tid < 3) {
    uint32_t t = 0;
    for (int w = 0; w < kCountThreads / kWave; ++w) t += part[tid][w];
    counts[tid] = static_cast<int32_t>(t);
  }
}

template <int KT, int R>
hipError_t launch_stream(const float *lat, const AnalyzeGeom &g, double *part, hipStream_t s) {
  const int total = g.C * g.nFC * g.nWC * g.nBH * g.G;
  const int blocks = (total + kAnalyzeWaves - 1) / kAnalyzeWaves;
  hipLaunchKernelGGL((analyze_stream_kernel<KT, R>), dim3(blocks), dim3(kAnalyzeWaves * kWave), 0,
                     s, lat, g, part, total);
  return hipGetLastError();
}

template <int KT>
hipError_t launch_stream_r(const float *lat, const AnalyzeGeom &g, double *part, hipStream_t s) {
  switch (g.R) {
    case 8: return launch_stream<KT, 8>(lat, g, part, s);
    case 4: return launch_stream<KT, 4>(lat, g, part, s);
    default: return launch_stream<KT, 2>(lat, g, part, s);
  }
}

// ---------------------------------------------------------------------------
// FFT complexity baseline (jano_fft_scores), an alternative index source.
// Per block: the energy of the block's 3D DFT outside the DC term, of the
// latest warm-up latent, over n^2 (n = the block's pixels inside the latent),
// averaged over the channels. By Parseval that quantity is the block's
// population variance, so the kernel takes the variance directly, no
// transform: one pass of fp64 sums of (x - x0) and (x - x0)^2, with x0 the
// block's first value (shifting by a value of the block keeps the difference
// of the two sums well conditioned, and a constant block gives exactly 0).
// One workgroup per block row (bf, bh); threads run over (channel, block
// column) pairs with the column fastest, so neighbouring lanes read
// neighbouring 16-byte pieces of one latent row (VEC: bW a multiple of 4,
// 16-byte aligned rows). Each block's channel sum is taken in channel order
// from LDS, so the result is deterministic.
// ---------------------------------------------------------------------------
constexpr int kFftThreads = 512;           // one pass over a 720p block row's 320 (channel, column) pairs
constexpr int kFftCols = 1024;             // block columns per pass over a block row
constexpr int kFftPairs = 2048;            // (channel, block column) variances held in LDS

template <bool VEC>
__global__ __launch_bounds__(kFftThreads) void fft_scores_kernel(const float *__restrict__ lat,
                                                                  AnalyzeGeom g,
                                                                  float *__restrict__ scores) {
  __shared__ double var[kFftPairs];
  __shared__ double acc[kFftCols];
  const int brow = blockIdx.x;                       // bf * nBH + bh
  const int bf = brow / g.nBH, bh = brow % g.nBH;
  const int f0 = bf * g.bF, f1 = min(g.F, f0 + g.bF);
  const int h0 = bh * g.bH, h1 = min(g.H, h0 + g.bH);
  const size_t plane = static_cast<size_t>(g.H) * g.W;
  const float *L = lat + static_cast<size_t>(g.K - 1) * g.C * g.F * plane;
  for (int bw0 = 0; bw0 < g.nBW; bw0 += kFftCols) {
    const int nw = min(kFftCols, g.nBW - bw0);
    for (int j = threadIdx.x; j < nw; j += kFftThreads) acc[j] = 0.0;
    const int cpp = kFftPairs / nw;                  // channels per pass (>= 2)
    for (int c0 = 0; c0 < g.C; c0 += cpp) {
      const int cn = min(cpp, g.C - c0);
      __syncthreads();                               // the previous pass's var reads are done
      for (int p = threadIdx.x; p < cn * nw; p += kFftThreads) {
        const int c = c0 + p / nw, bw = bw0 + p % nw;
        const int w0 = bw * g.bW, w1 = min(g.W, w0 + g.bW);
        const float *Lc = L + static_cast<size_t>(c) * g.F * plane + static_cast<size_t>(h0) * g.W + w0;
        const double x0 = static_cast<double>(Lc[static_cast<size_t>(f0) * plane]);
        double s1 = 0.0, s2 = 0.0;
        for (int f = f0; f < f1; ++f) {
#pragma unroll 8
          for (int h = 0; h < h1 - h0; ++h) {
            const float *row = Lc + f * plane + static_cast<size_t>(h) * g.W;
            if constexpr (VEC) {
              // bW a multiple of 4 and rows 16-byte aligned; a ragged last
              // block still ends on a multiple of 4 because W is one too
              for (int w = 0; w < w1 - w0; w += 4) {
                const f32x4 v = *reinterpret_cast<const f32x4 *>(row + w);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const double d = static_cast<double>(v[e]) - x0;
                  s1 += d;
                  s2 += d * d;
                }
              }
            } else {
              for (int w = 0; w < w1 - w0; ++w) {
                const double d = static_cast<double>(row[w]) - x0;
                s1 += d;
                s2 += d * d;
              }
            }
          }
        }
        const double n = static_cast<double>((f1 - f0) * (h1 - h0) * (w1 - w0));
        var[p] = fmax(s2 - s1 * (s1 / n), 0.0) / n;
      }
      __syncthreads();
      for (int j = threadIdx.x; j < nw; j += kFftThreads) {
        double a = acc[j];
        for (int cc = 0; cc < cn; ++cc) a += var[cc * nw + j];
        acc[j] = a;                                  // only this thread touches acc[j]
      }
    }
    for (int j = threadIdx.x; j < nw; j += kFftThreads)
      scores[static_cast<size_t>(brow) * g.nBW + bw0 + j] = static_cast<float>(acc[j] / g.C);
  }
}

}  // namespace

bool analyze_plan(int K, int C, int F, int H, int W, int bF, int bH, int bW, int pF, int pH,
                  int pW, AnalyzeGeom *g) {
  if (K < 3 || C < 1 || F < 1 || H < 1 || W < 1 || bF < 1 || bH < 1 || bW < 1 || pF < 1 ||
      pH < 1 || pW < 1)
    return false;
  if (F % pF || H % pH || W % pW || bF % pF || bH % pH || bW % pW) return false;
  AnalyzeGeom a{};
  a.K = K; a.C = C; a.F = F; a.H = H; a.W = W;
  a.bF = bF; a.bH = bH; a.bW = bW; a.pF = pF; a.pH = pH; a.pW = pW;
  a.nBF = (F + bF - 1) / bF;
  a.nBH = (H + bH - 1) / bH;
  a.nBW = (W + bW - 1) / bW;
  const long long B = static_cast<long long>(a.nBF) * a.nBH * a.nBW;
  if (B > kMaxBlocks) return false;
  a.B = static_cast<int>(B);
  a.R = (bH % 8 == 0) ? 8 : (bH % 4 == 0) ? 4 : (bH % 2 == 0) ? 2 : 1;
  const long long lat_bytes = static_cast<long long>(K) * C * F * H * W * 4;
  a.fast = K <= 8 && a.R >= 2 && bW <= kWave - 1 && lat_bytes < (1LL << 32);
  if (a.fast) {
    a.G = bH / a.R;
    a.CW = ((kWave - 1) / bW) * bW;
    a.nWC = (W + a.CW - 1) / a.CW;
    const long long waves0 = static_cast<long long>(C) * a.nBH * a.G * a.nWC;
    const long long want = (kTargetWaves + waves0 - 1) / waves0;     // frame chunks wanted
    const int per = static_cast<int>((a.nBF + want - 1) / want);      // blocks per chunk
    a.FC = max(1, per) * bF;
    a.nFC = (F + a.FC - 1) / a.FC;
  } else {
    a.R = bH; a.G = 1; a.CW = 0; a.nWC = 1; a.FC = F; a.nFC = 1;
  }
  *g = a;
  return true;
}

size_t analyze_ws_bytes(const AnalyzeGeom &g) {
  // fp64 partials [C*G][B]
  return static_cast<size_t>(g.C) * g.G * g.B * sizeof(double);
}

hipError_t launch_analyze_scores(const float *lat, const AnalyzeGeom &g, float *scores, void *ws,
                                 hipStream_t s) {
  double *part = static_cast<double *>(ws);
  hipError_t e = hipSuccess;
  if (g.fast) {
    switch (g.K) {
      case 3: e = launch_stream_r<3>(lat, g, part, s); break;
      case 4: e = launch_stream_r<4>(lat, g, part, s); break;
      case 5: e = launch_stream_r<5>(lat, g, part, s); break;
      case 6: e = launch_stream_r<6>(lat, g, part, s); break;
      case 7: e = launch_stream_r<7>(lat, g, part, s); break;
      default: e = launch_stream_r<8>(lat, g, part, s); break;
    }
  } else {
    const long long n = static_cast<long long>(g.C) * g.B;
    hipLaunchKernelGGL(analyze_generic_kernel, dim3(static_cast<unsigned>((n + 255) / 256)),
                       dim3(256), 0, s, lat, g, part);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(block_scores_kernel, dim3((g.B + 255) / 256), dim3(256), 0, s, part, g, scores);
  return hipGetLastError();
}

hipError_t launch_fft_scores(const float *lat, const AnalyzeGeom &g, float *scores, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(g.nBF * g.nBH));
  const bool vec = g.bW % 4 == 0 && g.W % 4 == 0 && reinterpret_cast<uintptr_t>(lat) % 16 == 0;
  if (vec)
    hipLaunchKernelGGL(fft_scores_kernel<true>, grid, dim3(kFftThreads), 0, s, lat, g, scores);
  else
    hipLaunchKernelGGL(fft_scores_kernel<false>, grid, dim3(kFftThreads), 0, s, lat, g, scores);
  return hipGetLastError();
}

hipError_t launch_levels(const float *scores, const AnalyzeGeom &g, int nS, int nSM, uint8_t *levels,
                         int32_t *counts, hipStream_t s) {
  constexpr int per_wg = kRankThreads / kRankSplit;
  hipLaunchKernelGGL(rank_levels_kernel, dim3((g.B + per_wg - 1) / per_wg), dim3(kRankThreads), 0, s,
                     scores, g.B, nS, nSM, levels);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(level_counts_kernel, dim3(1), dim3(kCountThreads), 0, s, levels, g, counts);
  return hipGetLastError();
}

}  // namespace jano
