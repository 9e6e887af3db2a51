// Active-query flash attention on bf16 MFMA (gfx950).
//
// Method (Jano pages, nl problem statement and methodology §2; fr §1 and
// §2.B): DiT attention is full (non-causal) attention over all tokens; in an
// interleaved step only the active tokens' queries are computed, and they
// attend to every token's key/value, frozen tokens' pairs coming from the
// cache. Key/value order does not matter, so the cache is read in token order.
//
//   out[i,h,:] = sum_j softmax_j(Q[i,h,:] . K[j,h,:] * scale) V[j,h,:]
//
// Design:
//   * grid = (query tiles of BM, heads); x runs fastest, so the workgroups of
//     one head are dispatched together and share that head's K/V in L2/MALL.
//   * 4 waves x 32 queries; each wave keeps its queries' Q fragments in
//     registers for the whole key loop.
//   * Per key tile of BN = 64: K (row-major, padded rows) and V (transposed to
//     [dim][key], padded) are staged in LDS, double-buffered: the global loads
//     of tile j+1 are in flight while tile j is computed.
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys on M, queries on N).
//     In the accumulator layout a lane owns one query column, so the online
//     softmax (running max, rescale, exp2, row sum) is lane-local apart from
//     one exchange with the lane 32 apart that holds the other key half.
//   * O^T += V^T P^T: the bf16-converted P accumulators are the B operand
//     as they stand; the V^T operand is read from the transposed LDS tile in
//     the same key order, so no data moves through LDS for P.
//   * fp32 accumulation, fp32 online softmax in the log2 domain.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace jano {
namespace {

constexpr int kAttnWaves = 4;
constexpr int kQW = 32;                   // queries per wave
constexpr int kBM = kAttnWaves * kQW;     // queries per workgroup
constexpr int kBN = 64;                   // keys per tile
constexpr int kThreads = kAttnWaves * kWave;

template <int D>
struct Lds {
  static constexpr int KS = D + 8;        // K row pitch (bf16 elements)
  static constexpr int VS = kBN + 8;      // V^T row pitch (bf16 elements)
  static constexpr int KSZ = kBN * KS;
  static constexpr int VSZ = D * VS;
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int D>
__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(const uint16_t *__restrict__ Q,
                                                            const uint16_t *__restrict__ K,
                                                            const uint16_t *__restrict__ V,
                                                            uint16_t *__restrict__ out, int nq,
                                                            int N, int H, float scale_log2) {
  using L = Lds<D>;
  constexpr int CPR = D / 8;                       // 16-byte chunks per row
  constexpr int CPT = kBN * CPR / kThreads;        // chunks per thread per tile
  static_assert(CPT * kThreads == kBN * CPR, "tile must split evenly");
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][L::KSZ];
  __shared__ __attribute__((aligned(16))) uint16_t vt[2][L::VSZ];

  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int l32 = lane & 31, hf = lane >> 5;
  const int head = blockIdx.y;
  const size_t rs = static_cast<size_t>(H) * D;     // token row stride (elements)
  const uint16_t *Kh = K + static_cast<size_t>(head) * D;
  const uint16_t *Vh = V + static_cast<size_t>(head) * D;

  // Q fragments: lane holds query (l32) dims [16t + 8hf, +8)
  const int qrow = blockIdx.x * kBM + wave * kQW + l32;
  bf16x8 qf[D / 16];
  {
    const uint16_t *qp = Q + static_cast<size_t>(qrow) * rs + static_cast<size_t>(head) * D + 8 * hf;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (qrow < nq) v = *reinterpret_cast<const u32x4 *>(qp + 16 * t);
      qf[t] = as_bf16x8(v);
    }
  }

  u32x4 kr[CPT], vr[CPT];
  auto load_tile = [&](int j) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * kThreads;
      const int row = c / CPR, col = (c % CPR) * 8;
      const int key = j * kBN + row;
      u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
      if (key < N) {
        a = *reinterpret_cast<const u32x4 *>(Kh + static_cast<size_t>(key) * rs + col);
        b = *reinterpret_cast<const u32x4 *>(Vh + static_cast<size_t>(key) * rs + col);
      }
      kr[i] = a;
      vr[i] = b;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * kThreads;
      const int row = c / CPR, col = (c % CPR) * 8;
      *reinterpret_cast<u32x4 *>(&ks[buf][row * L::KS + col]) = kr[i];
      const uint32_t w[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        vt[buf][(col + e) * L::VS + row] = static_cast<uint16_t>(w[e / 2] >> (16 * (e % 2)));
    }
  };

  const int ntiles = (N + kBN - 1) / kBN;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < ntiles) load_tile(j + 1);
    const uint16_t *kb = ks[buf];
    const uint16_t *vb = vt[buf];

    // S^T[key][query] for the tile's 64 keys (two 32-key blocks)
    f32x16 s[kBN / 32];
#pragma unroll
    for (int mb = 0; mb < kBN / 32; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[mb][r] = 0.0f;
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        const u32x4 a = *reinterpret_cast<const u32x4 *>(&kb[(mb * 32 + l32) * L::KS + 16 * t + 8 * hf]);
        s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), qf[t], s[mb], 0, 0, 0);
      }
    }
    if ((j + 1) * kBN > N) {   // ragged last tile: keys past N get no weight
#pragma unroll
      for (int mb = 0; mb < kBN / 32; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j * kBN + mb * 32 + 8 * (r / 4) + 4 * hf + (r % 4);
          if (key >= N) s[mb][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < kBN / 32; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][r]);
    mx = fmaxf(mx, shfl_xor_f32(mx, 32));
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
#pragma unroll
    for (int mb = 0; mb < kBN / 32; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[mb][r], scale_log2, -m_new));
        s[mb][r] = p;
        l_run += p;
      }

    // O^T[dim][query] += V^T[dim][key] P^T[key][query], 16 keys per MFMA.
    // k-slot 8*hf + e of this lane holds key 16t + 4hf + (e < 4 ? e : e + 4),
    // which is where S^T put it.
#pragma unroll
    for (int t = 0; t < kBN / 16; ++t) {
      const f32x16 &sv = s[t / 2];
      const int r0 = 8 * (t % 2);
      const f32x8 pf = {sv[r0], sv[r0 + 1], sv[r0 + 2], sv[r0 + 3],
                        sv[r0 + 4], sv[r0 + 5], sv[r0 + 6], sv[r0 + 7]};
      const bf16x8 pb = __builtin_convertvector(pf, bf16x8);
      const int kbase = 16 * t + 4 * hf;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const uint16_t *vrow = vb + (db * 32 + l32) * L::VS + kbase;
        const u32x2 lo = *reinterpret_cast<const u32x2 *>(vrow);
        const u32x2 hi = *reinterpret_cast<const u32x2 *>(vrow + 8);
        const u32x4 a = {lo.x, lo.y, hi.x, hi.y};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), pb, o[db], 0, 0, 0);
      }
    }
    if (j + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + shfl_xor_f32(l_run, 32);
  const float inv = 1.0f / l_tot;
  if (qrow < nq) {
    uint16_t *op = out + static_cast<size_t>(qrow) * rs + static_cast<size_t>(head) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 v = {o[db][4 * g4] * inv, o[db][4 * g4 + 1] * inv, o[db][4 * g4 + 2] * inv,
                         o[db][4 * g4 + 3] * inv};
        const bf16x4 b = __builtin_convertvector(v, bf16x4);
        *reinterpret_cast<bf16x4 *>(op + db * 32 + 8 * g4 + 4 * hf) = b;
      }
  }
}

}  // namespace

hipError_t launch_attention(const uint16_t *Q, int64_t nq, const uint16_t *K, const uint16_t *V,
                            int64_t N, int H, int d, float scale, uint16_t *out, hipStream_t s) {
  if (nq == 0) return hipSuccess;
  const float scale_log2 = scale * 1.4426950408889634f;
  const dim3 grid(static_cast<unsigned>((nq + kBM - 1) / kBM), static_cast<unsigned>(H));
  if (d == 128)
    hipLaunchKernelGGL(attn_fwd_kernel<128>, grid, dim3(kThreads), 0, s, Q, K, V, out,
                       static_cast<int>(nq), static_cast<int>(N), H, scale_log2);
  else
    hipLaunchKernelGGL(attn_fwd_kernel<64>, grid, dim3(kThreads), 0, s, Q, K, V, out,
                       static_cast<int>(nq), static_cast<int>(N), H, scale_log2);
  return hipGetLastError();
}

}  // namespace jano
