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
// Kernel 2 (levels_kernel, one workgroup) sums the partials in a fixed order,
// divides by the closed-form term count, rounds the score to fp32, finds the
// two level thresholds of the (score, block id) order by radix select, writes
// the levels and counts tokens per level.
#include "common.hpp"
#include "kernels.hpp"

namespace jano {
namespace {

constexpr int kAnalyzeWaves = 4;          // waves per workgroup of kernel 1
constexpr int kLevelsThreads = 1024;      // kernel 2 is one workgroup
constexpr int kMaxBlocks = 16384;         // kernel 2 keeps all keys in LDS
constexpr int kTargetWaves = 4096;        // enough waves to fill 256 CUs

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

template <int KT, int R>
__global__ __launch_bounds__(kAnalyzeWaves * kWave) void analyze_stream_kernel(
    const float *__restrict__ lat, AnalyzeGeom g, double *__restrict__ part, int total_waves) {
  constexpr int KD = KT - 2;  // number of second differences
  const int wave = blockIdx.x * kAnalyzeWaves + (threadIdx.x / kWave);
  if (wave >= total_waves) return;  // uniform per wave
  const int lane = threadIdx.x % kWave;

  const int nStrips = g.nBH * g.G;
  int q = wave;
  const int strip = q % nStrips;
  q /= nStrips;
  const int wc = q % g.nWC;
  q /= g.nWC;
  const int fc = q % g.nFC;
  const int c = q / g.nFC;

  const int bh = strip / g.G, sg = strip % g.G;
  const int h0 = bh * g.bH + sg * R;
  const int w0 = wc * g.CW;
  const int w = w0 + lane;
  const bool col_ok = lane <= g.CW && w < g.W;  // loads (includes the halo lane)
  const bool own = lane < g.CW && w < g.W;      // owns gradient terms
  const bool has_wn = own && (w + 1 < g.W);
  const int rows_loaded = min(R + 1, g.H - h0);  // may be <= 0 for empty strips
  const int rows_owned = min(R, g.H - h0);

  const int f0 = fc * g.FC;
  const int f_last = min(f0 + g.FC, g.F) - 1;   // last owned frame
  const int f_end = min(f0 + g.FC, g.F - 1);    // last loaded frame (halo)

  const size_t plane = static_cast<size_t>(g.H) * g.W;
  const size_t kstride = static_cast<size_t>(g.C) * g.F * plane;
  // Loads are unconditional from clamped (always in-bounds) addresses and
  // masked afterwards, so all (R+1)*K loads of a frame are in flight at once.
  const float *base = lat + static_cast<size_t>(c) * g.F * plane + min(w, g.W - 1);
  int rowoff[R + 1];
#pragma unroll
  for (int r = 0; r <= R; ++r) rowoff[r] = min(h0 + r, g.H - 1) * g.W;

  double Dprev[KD][R];
#pragma unroll
  for (int k = 0; k < KD; ++k)
#pragma unroll
    for (int r = 0; r < R; ++r) Dprev[k][r] = 0.0;
  double acc = 0.0;

  for (int f = f0; f <= f_end; ++f) {
    const float *p = base + static_cast<size_t>(f) * plane;
    float x[KT][R + 1];
#pragma unroll
    for (int r = 0; r <= R; ++r)
#pragma unroll
      for (int k = 0; k < KT; ++k) x[k][r] = p[k * kstride + rowoff[r]];
#pragma unroll
    for (int r = 0; r <= R; ++r) {
      const bool ok = col_ok && r < rows_loaded;
#pragma unroll
      for (int k = 0; k < KT; ++k) x[k][r] = ok ? x[k][r] : 0.0f;
    }
    double D[KD][R + 1];
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
          if (r < rows_owned) t += fabs(D[k][r] - Dprev[k][r]);
      if (own) acc += t;
      const int bprev = (f - 1) / g.bF;
      if (f > f_last || f / g.bF != bprev) {
        flush_block_sum(acc, g, lane, w0, c, sg, bprev, bh, part);
        acc = 0.0;
      }
    }
    if (f <= f_last) {
      double t = 0.0;
#pragma unroll
      for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int k = 0; k < KD; ++k) {
          const double right = shfl_down_f64(D[k][r], 1);   // +w neighbour
          if (r < rows_owned && has_wn) t += fabs(right - D[k][r]);
          if (r + 1 < rows_loaded) t += fabs(D[k][r + 1] - D[k][r]);  // +h
          Dprev[k][r] = D[k][r];
        }
      }
      if (own) acc += t;
    }
  }
  if (f_end == f_last) flush_block_sum(acc, g, lane, w0, c, sg, f_last / g.bF, bh, part);
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

// Finds, for each of two target ranks, the 64-bit key (score bits, block id)
// at that rank. keys[] holds the fp32 score bits (non-negative scores are
// ordered like their bit patterns). Radix select, 8 bits per pass: build the
// digit histogram of the candidates in LDS, then 512 threads scan the two
// 256-bin histograms in parallel to find the digit holding each target.
__device__ void select_two(const uint32_t *keys, int B, const int target[2], uint64_t thr[2],
                           uint32_t (*hist)[256], uint32_t *sh) {
  const int tid = threadIdx.x;
  const int lane = tid % kWave, wv = tid / kWave, nw = blockDim.x / kWave;
  // sh[0..1] prefix, sh[2..3] remaining rank, sh[4..5] found id,
  // sh[8..8+2*nw) per-wave scratch
  uint32_t *wtot = sh + 8;
  if (tid < 2) {
    sh[tid] = 0u;
    sh[2 + tid] = static_cast<uint32_t>(target[tid]);
  }
  __syncthreads();
  uint32_t mask = 0u;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 2 * 256; i += blockDim.x) hist[i / 256][i % 256] = 0u;
    __syncthreads();
    const uint32_t p0 = sh[0], p1 = sh[1];
    for (int b = tid; b < B; b += blockDim.x) {
      const uint32_t u = keys[b];
      const uint32_t dgt = (u >> shift) & 255u;
      if ((u & mask) == p0) atomicAdd(&hist[0][dgt], 1u);
      if ((u & mask) == p1) atomicAdd(&hist[1][dgt], 1u);
    }
    __syncthreads();
    // threads 0..511: target t = tid / 256, bin = tid % 256 (4 waves per target)
    uint32_t h = 0, incl = 0;
    if (tid < 512) {
      h = hist[tid / 256][tid % 256];
      incl = wave_inclusive_scan(h);
      if (lane == kWave - 1) wtot[wv] = incl;
    }
    __syncthreads();
    if (tid < 512) {
      const int t = tid / 256;
      uint32_t before = 0;
      for (int j = t * 4; j < wv; ++j) before += wtot[j];
      const uint32_t excl = before + incl - h;
      const uint32_t k = sh[2 + t];
      if (h > 0 && excl <= k && k < excl + h) {
        sh[t] |= static_cast<uint32_t>(tid % 256) << shift;
        sh[6 + t] = k - excl;
      }
    }
    mask |= 255u << shift;
    __syncthreads();
    if (tid < 2) sh[2 + tid] = sh[6 + tid];
    __syncthreads();
  }
  // the target is the k-th (in id order) block whose bits equal the prefix
  if (tid < 2) sh[4 + tid] = 0xFFFFFFFFu;
  uint32_t run0 = 0, run1 = 0;
  for (int b0 = 0; b0 < B; b0 += blockDim.x) {
    const int b = b0 + tid;
    const uint32_t u = b < B ? keys[b] : 0u;
    const bool e0 = b < B && u == sh[0];
    const bool e1 = b < B && u == sh[1];
    const uint64_t m0 = __ballot(e0), m1 = __ballot(e1);
    __syncthreads();
    if (lane == 0) {
      wtot[wv] = __popcll(m0);
      wtot[nw + wv] = __popcll(m1);
    }
    __syncthreads();
    uint32_t before0 = run0, before1 = run1, tot0 = 0, tot1 = 0;
    for (int j = 0; j < nw; ++j) {
      if (j < wv) {
        before0 += wtot[j];
        before1 += wtot[nw + j];
      }
      tot0 += wtot[j];
      tot1 += wtot[nw + j];
    }
    if (e0 && before0 + lanes_below(m0) == sh[2]) sh[4] = static_cast<uint32_t>(b);
    if (e1 && before1 + lanes_below(m1) == sh[3]) sh[5] = static_cast<uint32_t>(b);
    run0 += tot0;
    run1 += tot1;
  }
  __syncthreads();
  for (int t = 0; t < 2; ++t)
    thr[t] = (static_cast<uint64_t>(sh[t]) << 32) | static_cast<uint64_t>(sh[4 + t]);
  __syncthreads();
}

__global__ __launch_bounds__(kLevelsThreads) void levels_kernel(const double *__restrict__ part,
                                                                AnalyzeGeom g, int nS, int nSM,
                                                                float *__restrict__ scores,
                                                                uint8_t *__restrict__ levels,
                                                                int32_t *__restrict__ counts) {
  __shared__ uint32_t keys[kMaxBlocks];
  __shared__ uint32_t hist[2][256];
  __shared__ uint32_t sh[8 + 2 * (kLevelsThreads / kWave)];
  __shared__ int tok[3];
  const int tid = threadIdx.x;
  const int B = g.B, CG = g.C * g.G;
  const int tpbF = g.bF / g.pF, tpbH = g.bH / g.pH, tpbW = g.bW / g.pW;
  const int Ft = g.F / g.pF, Ht = g.H / g.pH, Wt = g.W / g.pW;
  if (tid < 3) tok[tid] = 0;

  for (int b = tid; b < B; b += blockDim.x) {
    double t = 0.0;
    for (int j = 0; j < CG; ++j) t += part[static_cast<size_t>(j) * B + b];
    const int bw = b % g.nBW, bh = (b / g.nBW) % g.nBH, bf = b / (g.nBW * g.nBH);
    const int f0 = bf * g.bF, f1 = min(f0 + g.bF, g.F);
    const int h0 = bh * g.bH, h1 = min(h0 + g.bH, g.H);
    const int w0 = bw * g.bW, w1 = min(w0 + g.bW, g.W);
    const long long ef = f1 - f0, eh = h1 - h0, ew = w1 - w0;
    const long long pos = (g.F >= 2 ? axis_terms(f0, f1, g.F) * eh * ew : 0) +
                          (g.H >= 2 ? axis_terms(h0, h1, g.H) * ef * ew : 0) +
                          (g.W >= 2 ? axis_terms(w0, w1, g.W) * ef * eh : 0);
    const long long n = pos * (g.K - 2) * g.C;
    const float s = n > 0 ? static_cast<float>(t / static_cast<double>(n)) : 0.0f;
    scores[b] = s;
    keys[b] = __float_as_uint(s);
  }
  __syncthreads();

  uint64_t thr[2];
  const int target[2] = {nS < B ? nS : 0, nSM < B ? nSM : 0};
  select_two(keys, B, target, thr, hist, sh);
  if (nS >= B) thr[0] = ~0ull;
  if (nSM >= B) thr[1] = ~0ull;

  int my[3] = {0, 0, 0};
  for (int b = tid; b < B; b += blockDim.x) {
    const uint64_t key = (static_cast<uint64_t>(keys[b]) << 32) | static_cast<uint64_t>(b);
    const int lv = key < thr[0] ? 1 : (key < thr[1] ? 2 : 3);
    levels[b] = static_cast<uint8_t>(lv);
    const int bw = b % g.nBW, bh = (b / g.nBW) % g.nBH, bf = b / (g.nBW * g.nBH);
    my[lv - 1] += axis_tokens(bf, tpbF, Ft) * axis_tokens(bh, tpbH, Ht) * axis_tokens(bw, tpbW, Wt);
  }
  for (int i = 0; i < 3; ++i)
    if (my[i]) atomicAdd(&tok[i], my[i]);
  __syncthreads();
  if (tid < 3) counts[tid] = tok[tid];
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
  a.fast = K <= 8 && a.R >= 2 && bW <= kWave - 1;
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
  return static_cast<size_t>(g.C) * g.G * g.B * sizeof(double);
}

hipError_t launch_analyze(const float *lat, const AnalyzeGeom &g, int nS, int nSM, float *scores,
                          uint8_t *levels, int32_t *counts, void *ws, hipStream_t s) {
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
  hipLaunchKernelGGL(levels_kernel, dim3(1), dim3(kLevelsThreads), 0, s, part, g, nS, nSM, scores,
                     levels, counts);
  return hipGetLastError();
}

}  // namespace jano
