// Gathered QKV projection of the active tokens with a 3D rotary position
// encoding (gfx950).
//
// Method (Jano pages, nl methodology §2; zh §2.2 item 3): in an interleaved
// step only the active tokens are computed, and their fresh keys/values join
// the cache without positions being restored (fr §2.B), so keys are cached
// with their position encoding applied. The projection and the encoding are
// model details the pages do not give; here
//   [Q | K | V][i, :] = W x[idx[i], :]      W [3*H*d, Dm] bf16, x [N, Dm] bf16
// with fp32 accumulation, then Q and K rotated over the token's (frame, row,
// column): the head dim splits into parts d_f = d - 4*floor(d/6) and
// d_h = d_w = 2*floor(d/6); pair i of a part of size m turns dims (2i, 2i+1)
// of that part by pos * base^(-2i/m). Outputs are bf16 [n_act, H, d].
//
// Design: Y^T = W X_act^T on v_mfma_f32_16x16x32_bf16 (output columns on M,
// tokens on N), so in the accumulator a lane holds four consecutive output
// columns of one token: the rotary pairs are lane-local and each lane stores
// 8 bytes per 16 x 16 tile. Workgroup tile 256 columns x 256 tokens, 8 waves
// of 128 x 64. K advances 32 at a time through 4 LDS stages filled with
// global_load_lds_dwordx4, three tiles in flight; a wave's MFMAs on tile t run
// from registers while tile t+1 is published (barrier) and its fragments are
// read, so LDS latency and the barrier overlap the MFMA work. Token rows are
// gathered through per-lane 32-bit offsets (idx[m] * Dm * 2) from a uniform
// base, weight rows through fixed per-lane offsets: no vector address
// arithmetic per K step. LDS rows are 64 bytes (4 chunks); chunk c of row r
// sits in slot c ^ ((r >> 1) & 3), so the 8 rows one 128-byte LDS pass of a
// fragment read touches fall on 8 different 16-byte bank groups. Workgroups
// are renumbered per XCD and rastered in groups of 2 token tiles (all weight
// tiles of a group, token tile fastest), which keeps the weight tiles the
// concurrent workgroups of an XCD share hot in its L2 (measured against groups
// of 1, 3, 4, 6, 8, 16 and a weight-major raster).
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"
#include "lds_copy.hpp"

namespace jano {
namespace {

constexpr int kPW = 8;                    // waves per workgroup
constexpr int kPBN = 256;                 // output columns per workgroup
constexpr int kPBM = 256;                 // tokens per workgroup
constexpr int kPBK = 32;                  // k per stage
constexpr int kPStages = 4;
constexpr int kPRowB = kPBK * 2;          // 64 bytes per LDS row
constexpr int kPTileB = kPBM * kPRowB;    // 16 KB per operand per stage
constexpr int kPXcds = 8;
constexpr int kPGroupM = 2;              // token tiles per raster group

typedef float f32x4p __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int swz_p(int r) { return (r >> 1) & 3; }

struct ProjGeom {
  int n_act, Dm, Nout, HD, d;
  int Ht, Wt;                             // token grid (rotary positions)
  int rope;                               // 0: no rotary encoding
  float log2_base;
  int df, dh;                             // rotary part sizes (frame, row = column)
  int nTM, nTN;                           // tiles along tokens, along output columns
};

__global__ __launch_bounds__(kPW * kWave) void qkv_proj_kernel(
    const uint16_t *__restrict__ X, const int32_t *__restrict__ idx, const uint16_t *__restrict__ W,
    ProjGeom g, uint16_t *__restrict__ Q, uint16_t *__restrict__ Kn, uint16_t *__restrict__ Vn) {
  __shared__ __attribute__((aligned(1024))) char lds[kPStages][2][kPTileB];   // [stage][W, X]
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int l16 = lane & 15, h4 = lane >> 4;

  // XCD-aware renumbering, then grouped raster (token tiles fastest in a group)
  const int nwg = gridDim.x, lin = blockIdx.x;
  const int xcd = lin % kPXcds, xslot = lin / kPXcds;
  const int logical = xcd * (nwg / kPXcds) + min(xcd, nwg % kPXcds) + xslot;
  const int per_group = kPGroupM * g.nTN;
  const int first_m = (logical / per_group) * kPGroupM;
  const int gsize = min(g.nTM - first_m, kPGroupM);
  const int in_group = logical % per_group;
  const int tm = first_m + in_group % gsize;
  const int tn = in_group / gsize;
  const int m0 = tm * kPBM, n0 = tn * kPBN;

  // per-lane copy offsets (fixed for the whole K loop): two 16-row copies per
  // operand per stage; lane -> row 32*wave + 16*q + lane/4, slot lane%4
  const size_t rowb = static_cast<size_t>(g.Dm) * 2;
  uint32_t offw[2], offx[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r = 32 * wave + 16 * q + lane / 4;
    const int c = (lane % 4) ^ swz_p(r);
    const int nrow = min(n0 + r, g.Nout - 1) - n0;              // clamped weight row
    const int tok = idx[min(m0 + r, g.n_act - 1)];              // gathered token row
    offw[q] = static_cast<uint32_t>(nrow * rowb + 16 * c);
    offx[q] = static_cast<uint32_t>(static_cast<size_t>(tok) * rowb + 16 * c);
  }
  const char *wbase = reinterpret_cast<const char *>(W) + static_cast<size_t>(n0) * rowb;
  const char *xbase = reinterpret_cast<const char *>(X);
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds[0][0]) + 32 * wave * kPRowB);
  auto issue = [&](const int t, const int st) __attribute__((always_inline)) {
    const size_t kb = static_cast<size_t>(t) * kPRowB;
    const uint32_t lw = lds0 + st * 2 * kPTileB, lx = lw + kPTileB;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      copy16_to_lds_s(wbase + kb, offw[q], lw + 16 * q * kPRowB);
      copy16_to_lds_s(xbase + kb, offx[q], lx + 16 * q * kPRowB);
    }
  };

  const int nk = g.Dm / kPBK;
  issue(0, 0);
  if (nk > 1) issue(1, 1);
  if (nk > 2) issue(2, 2);

  const int wn = wave % 2, wm = wave / 2;                        // wave tile: 128 columns x 64 tokens
  const int frag = l16 * kPRowB + 16 * (h4 ^ ((l16 >> 1) & 3));  // row l16 of a 16-row block, k 8*h4..
  f32x4p acc[8][4];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[a][b][r] = 0.0f;

  bf16x8 fa0[8], fb0[4], fa1[8], fb1[4];
  auto load_frags = [&](const int st, bf16x8 (&fa)[8], bf16x8 (&fb)[4]) __attribute__((always_inline)) {
    const char *ws = lds[st][0];
    const char *xs = lds[st][1];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
      fa[nt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(
                                              ws + (128 * wn + 16 * nt) * kPRowB + frag));
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      fb[mt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(
                                              xs + (64 * wm + 16 * mt) * kPRowB + frag));
  };
  auto mfmas = [&](const bf16x8 (&fa)[8], const bf16x8 (&fb)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[nt], fb[mt], acc[nt][mt], 0, 0, 0);
  };
  // publish tile t (its copies and every wave's), then queue tile t + 2
  // (every wave finished reading tile t-1 before this barrier, so tile t+3
  // can take its stage: three tiles in flight)
  auto publish = [&](const int t) __attribute__((always_inline)) {
    if (t + 2 < nk)
      __builtin_amdgcn_s_waitcnt(vmcnt_wait(8));
    else if (t + 1 < nk)
      __builtin_amdgcn_s_waitcnt(vmcnt_wait(4));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (t + 3 < nk) issue(t + 3, (t + 3) % kPStages);
  };
  // tile t's MFMAs run from registers while tile t+1 is published and its
  // fragments are read
  publish(0);
  load_frags(0, fa0, fb0);
  int t = 0;
  for (; t + 2 <= nk; t += 2) {
    mfmas(fa0, fb0);
    publish(t + 1);
    load_frags((t + 1) % kPStages, fa1, fb1);
    mfmas(fa1, fb1);
    if (t + 2 < nk) {
      publish(t + 2);
      load_frags((t + 2) % kPStages, fa0, fb0);
    }
  }
  if (t < nk) mfmas(fa0, fb0);

  // epilogue: lane holds columns n .. n+3 of token m for every (nt, mt).
  // What depends only on the column -- output part, head column, and each
  // rotary pair's axis and frequency (in turns per position) -- is worked
  // out once per column tile; per token only the angle is formed, reduced
  // to [0, 1) turns and fed to the hardware sine and cosine (v_sin_f32 /
  // v_cos_f32 take turns).
  constexpr float kInv2Pi = 0.15915494309189535f;
  int part_of[8], col_of[8], ax_of[8][2];
  float turns_of[8][2];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    const int n = n0 + 128 * wn + 16 * nt + 4 * h4;
    part_of[nt] = n / g.HD;
    col_of[nt] = n % g.HD;
    const int j0 = col_of[nt] % g.d;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int j = j0 + 2 * p;
      int ax, i, mm;
      if (j < g.df) {
        ax = 0; i = j / 2; mm = g.df;
      } else if (j < g.df + g.dh) {
        ax = 1; i = (j - g.df) / 2; mm = g.dh;
      } else {
        ax = 2; i = (j - g.df - g.dh) / 2; mm = g.dh;
      }
      ax_of[nt][p] = ax;
      turns_of[nt][p] = exp2f(-(2.0f * i / mm) * g.log2_base) * kInv2Pi;
    }
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int m = m0 + 64 * wm + 16 * mt + l16;
    if (m >= g.n_act) continue;
    const int tok = idx[m];
    const float pos[3] = {static_cast<float>(tok / (g.Ht * g.Wt)), static_cast<float>((tok / g.Wt) % g.Ht),
                          static_cast<float>(tok % g.Wt)};
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int n = n0 + 128 * wn + 16 * nt + 4 * h4;
      if (n >= g.Nout) continue;
      const int part = part_of[nt], col = col_of[nt];
      float v[4] = {acc[nt][mt][0], acc[nt][mt][1], acc[nt][mt][2], acc[nt][mt][3]};
      if (part < 2 && g.rope) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const float t = pos[ax_of[nt][p]] * turns_of[nt][p];
          const float r = t - floorf(t);
          const float sn = __builtin_amdgcn_sinf(r), cs = __builtin_amdgcn_cosf(r);
          const float x0 = v[2 * p], x1 = v[2 * p + 1];
          v[2 * p] = x0 * cs - x1 * sn;
          v[2 * p + 1] = x0 * sn + x1 * cs;
        }
      }
      const f32x4 vv = {v[0], v[1], v[2], v[3]};
      uint16_t *dst = (part == 0 ? Q : (part == 1 ? Kn : Vn)) + static_cast<size_t>(m) * g.HD + col;
      *reinterpret_cast<bf16x4 *>(dst) = __builtin_convertvector(vv, bf16x4);
    }
  }
}

}  // namespace

bool qkv_proj_supported(int64_t N, int64_t Dm, int H, int d) {
  const int64_t Nout = 3LL * H * d;
  return Dm >= kPBK && Dm % kPBK == 0 && d % 4 == 0 && Nout >= 4 && N * Dm * 2 < (1LL << 32) &&
         Nout * Dm * 2 < (1LL << 31);
}

hipError_t launch_qkv_proj(const uint16_t *X, int64_t Dm, const int32_t *idx, int64_t n_act,
                           const uint16_t *W, int H, int d, int Ht, int Wt, float rope_base,
                           uint16_t *Q, uint16_t *Kn, uint16_t *Vn, hipStream_t s) {
  if (n_act == 0) return hipSuccess;
  ProjGeom g{};
  g.n_act = static_cast<int>(n_act);
  g.Dm = static_cast<int>(Dm);
  g.HD = H * d;
  g.Nout = 3 * g.HD;
  g.d = d;
  g.Ht = Ht;
  g.Wt = Wt;
  g.rope = rope_base > 0.0f;
  g.log2_base = g.rope ? log2f(rope_base) : 0.0f;
  g.dh = 2 * (d / 6);
  g.df = d - 2 * g.dh;
  g.nTM = static_cast<int>((n_act + kPBM - 1) / kPBM);
  g.nTN = (g.Nout + kPBN - 1) / kPBN;
  hipLaunchKernelGGL(qkv_proj_kernel, dim3(static_cast<unsigned>(g.nTM * g.nTN)), dim3(kPW * kWave), 0, s,
                     X, idx, W, g, Q, Kn, Vn);
  return hipGetLastError();
}

}  // namespace jano
