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
// Common design:
//   * grid = (query tiles, heads); each workgroup streams the whole K/V of one
//     head through LDS in tiles of 64 keys while its waves keep their Q
//     fragments in registers for the whole key loop.
//   * S^T = K Q^T on MFMA with keys on M and queries on N: in the accumulator
//     layout a lane owns one query column, so the online softmax (running max,
//     rescale, exp2, row sum) is lane-local apart from a few lane exchanges
//     between the lanes that hold other keys of the same query.
//   * O^T += V^T P^T: the bf16-converted P accumulators are the B operand as
//     they stand and V^T is read from LDS in the same key order, so P never
//     passes through LDS.
//   * fp32 accumulation, fp32 online softmax in the log2 domain.
// attn_fwd_kernel<64> (d = 64) is the simple form: 4 waves x 32 queries,
// v_mfma_f32_32x32x16_bf16, register-staged double-buffered tiles, V
// transposed on the LDS write. attn_fwd_d128_kernel (d = 128) is the tuned
// one, described above its definition.
#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "lds_copy.hpp"

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

// ---------------------------------------------------------------------------
// Shared pieces of the d = 128 kernel. K/V tiles of 64 keys go from global
// memory straight into LDS (global_load_lds_dwordx4, no registers involved),
// four stages deep, two tiles in flight ahead of the one being consumed.
//
// LDS rows are 256 bytes (128 bf16) split in 16 chunks of 16 bytes; chunk c of
// row r is stored at slot c ^ swz(r). The swizzle is applied on the global
// side: the lane that fills LDS slot s fetches the chunk that belongs there.
//
// ds_read_b64_tr_b16 (per 16-lane group): lane j receives element (j % 4) of
// the 4-element row that source lane 4e + j/4 addressed, for e = 0..3. When
// source lane i addresses V[k0 + i/4][d0 + 4*(i%4) .. +3], lane j receives
// V[k0 .. k0+3][d0 + j]: one dim, four consecutive keys -- the V^T operand of
// the PV MFMA, read from row-major V.
// ---------------------------------------------------------------------------
constexpr int kW2 = 8;                      // waves per workgroup
constexpr int kRowB = 256;                  // bytes per K/V row (d = 128)
constexpr int kTileB = kBN * kRowB;         // 16 KB per K or V tile
constexpr float kRescaleSlack = 8.0f;       // log2 headroom before rescaling
constexpr int kWaitVmcnt0 = vmcnt_wait(0);
constexpr int kWaitVmcnt4 = vmcnt_wait(4);

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ int swz_k(int r) { return r & 15; }



constexpr int kStages = 4;
constexpr int kXcdsAttn = 8;    // accelerator dies (each with an L2) per GPU

// ---------------------------------------------------------------------------
// attn_fwd_d128_kernel, v_mfma_f32_16x16x32_bf16: 8 waves x 48 queries (three groups of
// 16 per wave). Every K fragment (16 keys x 32 dims) and V^T fragment (16 dims
// x 32 keys) read from LDS feeds one MFMA per query group, so a wave reuses
// each LDS byte for 48 queries instead of 32.
//   S^T block (16 keys x 16 queries): lane l holds query l%16, keys
//     4*(l/16) + 0..3 of the block.
//   PV step of 32 keys: the B operand P^T of lane l takes keys 4h..4h+3 and
//     16+4h..16+4h+3 (h = l/16) -- registers 0..3 of two consecutive S^T
//     blocks -- and the V^T operand is read with two transposing reads of
//     the same keys for dims 16*db + l%16.
//   K rows use swz(r) = r & 15: the S MFMA reads one chunk of 16 consecutive
//   rows per 16 lanes (ds_read_b128), which then hit 16 different bank
//   groups. V rows use swz(r) = 2*(r & 7): the transposing reads of one half
//   wave cover 8 consecutive rows x 2 chunks, which this spreads over 16 bank
//   groups.
//   Workgroups are renumbered so that each XCD (one L2 each) works through
//   whole heads and the workgroups of a head share its K/V stream in one L2.
//   The two waves that share a SIMD (w and w + 4) take a tile's work in
//   different orders -- S, softmax, PV against PV of the previous tile, S,
//   softmax -- and MFMA phases run at a higher wave priority than the
//   softmax, so one wave's exponents overlap the other's MFMAs.
//   The running max is raised only when a tile's max exceeds it by more than
//   2^8 (kRescaleSlack), so most tiles skip the O rescale; P <= 2^8 stays well
//   inside bf16 and fp32 range, and the final division by the row sum cancels
//   whatever reference point the exponents used. Each lane first compares the
//   max of its own 16 keys; the four lanes of a query exchange maxima (and the
//   wave rescales) only when some lane's keys would raise the running max.
//   Row sums are taken over the bf16 P values the PV product uses, two at a
//   time (v_dot2_f32_bf16 against (1, 1)).
//   K/V copies of full tiles use a wave-uniform base address and per-lane
//   32-bit offsets that do not change from tile to tile; only the last tile,
//   when it extends past N, goes through the clamped per-row path. That tile
//   is also the only one whose scores are masked (keys >= N get -inf).
// ---------------------------------------------------------------------------
typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int swz_v2(int r) { return 2 * (r & 7); }

__device__ __forceinline__ void issue_tile(const uint16_t *Kh, const uint16_t *Vh, size_t rs,
                                               int N, int key0, char *stage_k, char *stage_v,
                                               int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 4 * (2 * wave + i) + lane / 16;
    const int slot = lane % 16;
    const int key = min(key0 + r, N - 1);
    const uint16_t *krow = Kh + static_cast<size_t>(key) * rs;
    const uint16_t *vrow = Vh + static_cast<size_t>(key) * rs;
    copy16_to_lds(krow + 8 * (slot ^ swz_k(r)), lds_addr(stage_k + (4 * (2 * wave + i)) * kRowB));
    copy16_to_lds(vrow + 8 * (slot ^ swz_v2(r)), lds_addr(stage_v + (4 * (2 * wave + i)) * kRowB));
  }
}

// Full tile (all 64 keys < N): per-lane offsets are tile-invariant.
// lds_k / lds_v: LDS byte addresses (wave-uniform) of this wave's first row in the stage
__device__ __forceinline__ void issue_tile_full(const char *kbase, const char *vbase,
                                                const uint32_t (&koff)[2], const uint32_t (&voff)[2],
                                                uint32_t lds_k, uint32_t lds_v) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    copy16_to_lds_s(kbase, koff[i], lds_k + 4 * i * kRowB);
    copy16_to_lds_s(vbase, voff[i], lds_v + 4 * i * kRowB);
  }
}

// Wave priority around the two kinds of work of a tile, fenced so that the
// compiler keeps each phase's instructions inside it. With one wave of a
// SIMD in its MFMA phase and the other in its softmax, the arbiter serves the
// MFMA wave first, so each MFMA issues as soon as the matrix core takes it
// and the softmax's VALU instructions fill the cycles in between.
__device__ __forceinline__ void matrix_phase() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(1);
  __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void vector_phase() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);
}

// G query groups of 16 per wave: G = 3 (384 queries per workgroup) is the
// fast form; G = 2 (256 per workgroup) loses some LDS reuse but fills the
// last round of a launch whose 384-query tiles would leave most CUs idle.
// Keys: tiles [kt0, kt1) of 64 (the whole range unless the launch splits the
// keys). part_o NULL: the normalised bf16 output goes to out. Otherwise the
// key range's unnormalised fp32 output goes to part_o [nq][H][128] and its
// running max (log2 units) and row sum to part_m and part_l [nq][H], for
// combine_kernel to merge.
template <int G, bool SPLIT>
__device__ __forceinline__ void attn_tile_d128(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    uint16_t *__restrict__ out, int nq, int N, int H, float scale_log2, int head, int q0,
    char (*lds)[2][kTileB], int kt0, int kt1, float *__restrict__ part_o,
    float *__restrict__ part_m, float *__restrict__ part_l) {
  constexpr int D = 128;
  constexpr int kQW2 = 16 * G;              // queries per wave
  // LDS fragment reads issued ahead of the MFMAs that use them: the 2-group
  // form has the registers to hold 8 K and 8 V^T fragments in flight (+2% on
  // the 480p shapes against 4 and none); at 3 groups the register file is full
  constexpr int kSAhead = G == 2 ? 8 : 4;
  constexpr int kPVAhead = G == 2 ? 8 : 0;

  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int l16 = lane & 15, h4 = lane >> 4;
  const size_t rs = static_cast<size_t>(H) * D;
  const uint16_t *Kh = K + static_cast<size_t>(head) * D;
  const uint16_t *Vh = V + static_cast<size_t>(head) * D;
  // local tiles 0 .. ntiles-1 are tiles kt0 .. kt1-1; the first nfull are
  // whole (only the range that ends at N can end in a ragged tile). Without
  // a split the range is every key.
  const int ntiles = SPLIT ? kt1 - kt0 : (N + kBN - 1) / kBN;
  const int nfull = SPLIT ? min(kt1, N / kBN) - kt0 : N / kBN;
  if (!SPLIT) kt0 = 0;
  // byte offsets of this lane's two copies within a tile (row r, swizzled chunk)
  uint32_t koff[2], voff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 4 * (2 * wave + i) + lane / 16;
    const int slot = lane % 16;
    koff[i] = static_cast<uint32_t>(r * rs * 2 + 16 * (slot ^ swz_k(r)));
    voff[i] = static_cast<uint32_t>(r * rs * 2 + 16 * (slot ^ swz_v2(r)));
  }
  const size_t tile_bytes = static_cast<size_t>(kBN) * rs * 2;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds[0][0]) + 8 * wave * kRowB);
  auto issue = [&](const int t, const int stg) {
    if (t < nfull)
      issue_tile_full(reinterpret_cast<const char *>(Kh) + (kt0 + t) * tile_bytes,
                      reinterpret_cast<const char *>(Vh) + (kt0 + t) * tile_bytes, koff, voff,
                      lds0 + stg * 2 * kTileB, lds0 + stg * 2 * kTileB + kTileB);
    else
      issue_tile(Kh, Vh, rs, N, (kt0 + t) * kBN, lds[stg][0], lds[stg][1], wave, lane);
  };

  issue(0, 0);
  if (ntiles > 1) issue(1, 1);

  int qrow[G];
  bf16x8 qf[G][D / 32];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    qrow[g] = q0 + wave * kQW2 + 16 * g + l16;
    const uint16_t *qp = Q + static_cast<size_t>(min(qrow[g], nq - 1)) * rs +
                         static_cast<size_t>(head) * D + 8 * h4;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
      qf[g][t] = as_bf16x8(__builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(qp + 32 * t)));
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int t = 0; t < D / 32; ++t) asm volatile("" : : "v"(qf[g][t]));

  // tile-invariant LDS byte offsets
  int kl[D / 32];                            // K: row l16 (+16*kb), chunk 4t + h4
#pragma unroll
  for (int t = 0; t < D / 32; ++t) kl[t] = l16 * kRowB + (((4 * t + h4) ^ swz_k(l16)) << 4);
  // V^T: key k0 + l16/4 (k0 = 32*ks + 16*half + 4*h4), dims 16*db + 4*(l16%4)
  const int vkey = 4 * h4 + l16 / 4;         // key within a 16-key half, < 16
  int vl[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
    vl[db] = vkey * kRowB + 8 * (l16 % 2) + (((2 * db + (l16 % 4) / 2) ^ swz_v2(vkey)) << 4);
  // rows 16*half + 32*ks + vkey share (r & 7) with vkey, so only the row
  // offset changes between the four reads of a dim block

  f32x4v o[G][D / 16];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[g][db][r] = 0.0f;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  float m_run[G], l_run[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.0f;
  }

  // tile j's K/V in LDS for every wave; tile j+2's copies issued
  auto sync = [&](const int j) {
    if (j + 1 < ntiles)
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt4);
    else
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __builtin_amdgcn_s_barrier();
    if (j + 2 < ntiles) issue(j + 2, (j + 2) % kStages);
  };
  // S and softmax of one 64-key tile into pb; RAGGED only for a last tile
  // that extends past N
  auto s_soft = [&](const int j, auto ragged_tag, bf16x8 (&pb)[G][kBN / 32]) {
    constexpr bool RAGGED = decltype(ragged_tag)::value;
    const char *kb = lds[j % kStages][0];
    matrix_phase();

    f32x4v s[G][kBN / 16];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int b = 0; b < kBN / 16; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) s[g][b][r] = 0.0f;
#pragma unroll
    for (int b = 0; b < kBN / 16; ++b)
#pragma unroll
      for (int t = 0; t < D / 32; ++t) {
        const u32x4 a = *reinterpret_cast<const u32x4 *>(kb + b * 16 * kRowB + kl[t]);
#pragma unroll
        for (int g = 0; g < G; ++g)
          s[g][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), qf[g][t], s[g][b], 0, 0, 0);
      }
    // schedule: kSAhead K reads ahead, then one read per G MFMAs, so each
    // read has kSAhead * G MFMAs to land (~190 cycles at G = 3); left to
    // itself the compiler waits on each read right after issuing it
    __builtin_amdgcn_sched_group_barrier(0x100, kSAhead, 0);    // reads ahead
#pragma unroll
    for (int i = 0; i < 16 - kSAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, G, 0);  // G MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kSAhead * G, 0);  // last MFMAs
    vector_phase();

#pragma unroll
    for (int g = 0; g < G; ++g) {
      if constexpr (RAGGED) {
#pragma unroll
        for (int b = 0; b < kBN / 16; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if ((kt0 + j) * kBN + 16 * b + 4 * h4 + r >= N) s[g][b][r] = -INFINITY;
      }
      // this lane's 16 keys of the query; the 4 lanes that share a query
      // exchange maxima only when one of them would raise the running max
      float mx = fmaxf(fmaxf(fmaxf(s[g][0][0], s[g][0][1]), fmaxf(s[g][0][2], s[g][0][3])),
                       fmaxf(fmaxf(s[g][1][0], s[g][1][1]), fmaxf(s[g][1][2], s[g][1][3])));
      mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(s[g][2][0], s[g][2][1]), fmaxf(s[g][2][2], s[g][2][3])),
                           fmaxf(fmaxf(s[g][3][0], s[g][3][1]), fmaxf(s[g][3][2], s[g][3][3]))));
      mx *= scale_log2;
      if (__ballot(mx > m_run[g] + kRescaleSlack)) {
        mx = fmaxf(mx, shfl_xor_f32(mx, 16));
        mx = fmaxf(mx, shfl_xor_f32(mx, 32));
        const bool grow = mx > m_run[g] + kRescaleSlack;
        const float m_new = grow ? mx : m_run[g];
        const float alpha = __builtin_amdgcn_exp2f(m_run[g] - m_new);
        m_run[g] = m_new;
        l_run[g] *= alpha;
#pragma unroll
        for (int db = 0; db < D / 16; ++db)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[g][db][r] *= alpha;
      }
      float ls[kBN / 32] = {0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < kBN / 32; ++ks) {
        f32x8 pf;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pf[e] = __builtin_amdgcn_exp2f(fmaf(s[g][2 * ks + e / 4][e % 4], scale_log2, -m_run[g]));
        pb[g][ks] = __builtin_convertvector(pf, bf16x8);
        // row sum of the bf16 P the PV product uses: pairs dotted with (1, 1)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16x2 pp = {pb[g][ks][2 * e], pb[g][ks][2 * e + 1]};
          ls[ks] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones2, ls[ks], false);
        }
      }
      l_run[g] += ls[0] + ls[1];
    }
  };
  // O += V^T P of the tile in stage st
  auto pv = [&](const int st, const bf16x8 (&pb)[G][kBN / 32]) {
    const char *vb = lds[st][1];
    matrix_phase();
#pragma unroll
    for (int ks = 0; ks < kBN / 32; ++ks)
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4 *)(vb + (32 * ks) * kRowB + vl[db]));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4 *)(vb + (32 * ks + 16) * kRowB + vl[db]));
        const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int g = 0; g < G; ++g)
          o[g][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[g][ks], o[g][db], 0, 0, 0);
      }
    if constexpr (kPVAhead > 0) {
      // the same for the V^T fragments (two transposing reads each)
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kPVAhead, 1);
#pragma unroll
      for (int i = 0; i < 16 - kPVAhead; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, G, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kPVAhead * G, 1);
    }
    vector_phase();
  };
  // Waves w and w + 4 share a SIMD. Waves 0-3 run S, softmax and PV of each
  // tile; waves 4-7 run PV of the previous tile, then S and softmax of this
  // one, carrying P over the barrier (the previous tile's V stays in its
  // stage until the next tile's copies are issued, one barrier later). After
  // the barrier both waves of a SIMD issue MFMAs; then one wave's softmax
  // meets the other's S MFMAs, and the other's softmax meets the first
  // one's PV MFMAs. P of the previous tile is dead before S of this tile is
  // live, so the second order needs no more registers than the first.
  // Both orders pass exactly ntiles barriers (sync), which is what keeps the
  // workgroup's barrier count matched. Which waves share a SIMD decides only
  // how well the phases overlap, never the result.
  if (__builtin_amdgcn_readfirstlane(wave) < kW2 / 2) {
    for (int j = 0; j < nfull; ++j) {
      sync(j);
      bf16x8 pb[G][kBN / 32];
      s_soft(j, std::false_type{}, pb);
      pv(j % kStages, pb);
    }
    if (nfull < ntiles) {
      sync(nfull);
      bf16x8 pb[G][kBN / 32];
      s_soft(nfull, std::true_type{}, pb);
      pv(nfull % kStages, pb);
    }
  } else {
    bf16x8 pb[G][kBN / 32];
    if (nfull > 0) {
      sync(0);
      s_soft(0, std::false_type{}, pb);
      for (int j = 1; j < nfull; ++j) {
        sync(j);
        pv((j - 1) % kStages, pb);
        __builtin_amdgcn_sched_barrier(0);
        s_soft(j, std::false_type{}, pb);
      }
    }
    if (nfull < ntiles) {
      sync(nfull);
      if (nfull > 0) pv((nfull - 1) % kStages, pb);
      s_soft(nfull, std::true_type{}, pb);
    }
    pv((ntiles - 1) % kStages, pb);
  }

#pragma unroll
  for (int g = 0; g < G; ++g) {
    float l_tot = l_run[g] + shfl_xor_f32(l_run[g], 16);
    l_tot += shfl_xor_f32(l_tot, 32);
    if constexpr (SPLIT) {
      // a key range's share: unnormalised output, its max and row sum
      if (qrow[g] < nq) {
        const size_t qh = static_cast<size_t>(qrow[g]) * H + head;
        float *po = part_o + qh * D;
#pragma unroll
        for (int db = 0; db < D / 16; ++db) *reinterpret_cast<f32x4v *>(po + 16 * db + 4 * h4) = o[g][db];
        if (h4 == 0) {
          part_m[qh] = m_run[g];
          part_l[qh] = l_tot;
        }
      }
      continue;
    }
    const float inv = 1.0f / l_tot;
    if (qrow[g] < nq) {
      uint16_t *op = out + static_cast<size_t>(qrow[g]) * rs + static_cast<size_t>(head) * D;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        const f32x4 v = {o[g][db][0] * inv, o[g][db][1] * inv, o[g][db][2] * inv, o[g][db][3] * inv};
        *reinterpret_cast<bf16x4 *>(op + 16 * db + 4 * h4) = __builtin_convertvector(v, bf16x4);
      }
    }
  }
}

// Workgroup i of a phase of n workgroups, renumbered so that the workgroups
// one XCD (one L2) receives -- the hardware deals them out round-robin --
// are consecutive: an XCD works through whole heads in turn.
__device__ __forceinline__ int xcd_order(int i, int n) {
  const int x = i % kXcdsAttn;
  return x * (n / kXcdsAttn) + min(x, n % kXcdsAttn) + i / kXcdsAttn;
}

// One launch of the d = 128 kernel: each head's queries are covered by k3
// tiles of 384 (workgroups 0 .. H*k3-1) and then m2 tiles of 256 (the rest,
// dispatched last), so a launch's last round can be filled with shorter
// workgroups. Both phases are numbered XCD by XCD (xcd_order). FORM 3 and
// FORM 2 are the launches with only one tile size (m2 = 0, or k3 = 0),
// compiled without the other form's code; FORM 0 holds both.
template <int FORM>
__global__ __launch_bounds__(kW2 * kWave) void attn_fwd_d128_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    uint16_t *__restrict__ out, int nq, int N, int H, float scale_log2, int k3, int m2) {
  __shared__ __attribute__((aligned(1024))) char lds[kStages][2][kTileB];
  const int i = blockIdx.x, n3 = H * k3;
  if (FORM == 3 || (FORM == 0 && i < n3)) {
    const int t = xcd_order(i, n3);
    attn_tile_d128<3, false>(Q, K, V, out, nq, N, H, scale_log2, t / k3, 384 * (t % k3), lds, 0, 0, nullptr,
                             nullptr, nullptr);
  } else {
    const int t = xcd_order(i - n3, H * m2);
    attn_tile_d128<2, false>(Q, K, V, out, nq, N, H, scale_log2, t / m2, 384 * k3 + 256 * (t % m2), lds, 0,
                             0, nullptr, nullptr, nullptr);
  }
}

// Key-split launch: every (head, key range, query tile) is one workgroup of
// the 384-query (G = 3) or 256-query (G = 2) form, numbered XCD by XCD with
// the query tile fastest, so the workgroups that stream one head's key range
// share an L2. Key range s of S holds tiles [s*nt/S, (s+1)*nt/S).
template <int G>
__global__ __launch_bounds__(kW2 * kWave) void attn_split_d128_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    int nq, int N, int H, float scale_log2, int tiles, int S, float *__restrict__ ws) {
  __shared__ __attribute__((aligned(1024))) char lds[kStages][2][kTileB];
  const int t = xcd_order(blockIdx.x, H * S * tiles);
  const int head = t / (S * tiles), sp = (t / tiles) % S, qt = t % tiles;
  const int nt = (N + kBN - 1) / kBN;
  const size_t nqh = static_cast<size_t>(nq) * H;
  float *po = ws + static_cast<size_t>(sp) * nqh * 128;
  float *pm = ws + static_cast<size_t>(S) * nqh * 128 + static_cast<size_t>(sp) * nqh;
  float *pl = ws + static_cast<size_t>(S) * nqh * 129 + static_cast<size_t>(sp) * nqh;
  attn_tile_d128<G, true>(Q, K, V, nullptr, nq, N, H, scale_log2, head, 16 * kW2 * G * qt, lds, sp * nt / S,
                          (sp + 1) * nt / S, po, pm, pl);
}

// Merge of the S key ranges' partial results, in range order: with m the
// largest range max, out = sum_s 2^(m_s - m) O_s / sum_s 2^(m_s - m) l_s.
// One thread per 8 output dims of one (query, head).
constexpr int kCombineThreads = 256;
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const float *__restrict__ ws, int nq, int H,
                                                                  int S, uint16_t *__restrict__ out) {
  const size_t nqh = static_cast<size_t>(nq) * H;
  const size_t i = static_cast<size_t>(blockIdx.x) * kCombineThreads + threadIdx.x;
  if (i >= nqh * 16) return;
  const size_t qh = i / 16;
  const int c = static_cast<int>(i % 16);
  const float *pm = ws + static_cast<size_t>(S) * nqh * 128;
  const float *pl = pm + static_cast<size_t>(S) * nqh;
  float m = -INFINITY;
  for (int sp = 0; sp < S; ++sp) m = fmaxf(m, pm[sp * nqh + qh]);
  float l = 0.0f, acc[8] = {};
  for (int sp = 0; sp < S; ++sp) {
    const float w = __builtin_amdgcn_exp2f(pm[sp * nqh + qh] - m);
    l += w * pl[sp * nqh + qh];
    const f32x4v *po = reinterpret_cast<const f32x4v *>(ws + (static_cast<size_t>(sp) * nqh + qh) * 128 + 8 * c);
    const f32x4v a = po[0], b = po[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] += w * a[e];
      acc[4 + e] += w * b[e];
    }
  }
  const float inv = 1.0f / l;
  const f32x8 v = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv,
                   acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
  *reinterpret_cast<bf16x8 *>(out + qh * 128 + 8 * c) = __builtin_convertvector(v, bf16x8);
}

// Tiles of the d = 128 kernel for one launch. One workgroup fills a CU
// (128 KB of LDS), every workgroup streams all N keys, so a 384-query
// workgroup takes one unit of time and a 256-query one kCostG2 units
// (measured 0.69-0.71: two thirds of the matrix and softmax work at the same
// LDS reads per tile). Each XCD runs its share of the 384-query workgroups
// and then of the 256-query ones on its 32 CUs, taking the next workgroup
// whenever a CU frees; the plan with the earliest modelled finish wins
// among all-384 (ragged last tile), all-256, and k3 full 384-query tiles per
// head followed by 256-query tiles for the rest.
constexpr int kCUs = 256;
constexpr int kCUsPerXcd = kCUs / kXcdsAttn;
constexpr double kCostG2 = 0.70;

double xcd_finish(int64_t n3, int64_t n2) {
  const int64_t P = kCUsPerXcd, r = n3 / P, q = n3 % P;
  const double t3 = static_cast<double>(r + (q ? 1 : 0));
  if (n2 == 0) return t3;
  // 256-query workgroups go to the CU that frees first: P - q CUs from time
  // r, q CUs from time r + 1
  double last = 0.0;
  int64_t a = 0, b = 0, left = n2;
  while (left > 0) {
    const double te = r + a * kCostG2;
    const double tl = q ? r + 1 + b * kCostG2 : 1e300;
    if (te <= tl) {
      left -= P - q;
      last = te;
      ++a;
    } else {
      left -= q;
      last = tl;
      ++b;
    }
  }
  return last + kCostG2 > t3 ? last + kCostG2 : t3;
}

double plan_finish(int64_t k3, int64_t m2, int H) {
  const int64_t n3 = k3 * H, n2 = m2 * H;
  return xcd_finish((n3 + kXcdsAttn - 1) / kXcdsAttn, (n2 + kXcdsAttn - 1) / kXcdsAttn);
}

void plan_d128(int64_t nq, int H, int *k3, int *m2) {
  int64_t bk = (nq + 383) / 384, bm = 0;                    // all 384, ragged last tile
  double best = plan_finish(bk, 0, H);
  auto consider = [&](int64_t k, int64_t m) {
    const double f = plan_finish(k, m, H);
    if (f < best - 1e-9) {
      best = f;
      bk = k;
      bm = m;
    }
  };
  consider(0, (nq + 255) / 256);                            // all 256
  const int64_t kfull = nq / 384;
  for (int64_t k = kfull; k >= 1 && k >= kfull - 32; --k) consider(k, (nq - 384 * k + 255) / 256);
  *k3 = static_cast<int>(bk);
  *m2 = static_cast<int>(bm);
}

// Key-split plan, used only when the caller provides a workspace: each
// (head, query tile) is split into S key ranges (S workgroups of 1/S the
// work each) and a combine launch merges them. Modelled like plan_d128, a
// launch of one tile form finishes after ceil(per-XCD workgroups / 32)
// rounds of cost/S; a split plan is taken only when it beats the best
// unsplit plan by more than 15% (the combine, the per-workgroup prologue and
// the partial writes are not in the model). Each key range keeps >= 2 tiles.
constexpr int kMaxSplit = 4;
constexpr double kSplitMargin = 1.15;

void plan_split_d128(int64_t nq, int64_t N, int H, int *G, int *tiles, int *S) {
  int k3, m2;
  plan_d128(nq, H, &k3, &m2);
  const double f1 = plan_finish(k3, m2, H);
  const int64_t nt = (N + kBN - 1) / kBN;
  double best = f1 / kSplitMargin;
  *S = 1;
  *G = 0;
  *tiles = 0;
  for (int g = 3; g >= 2; --g) {
    const int64_t qt = (nq + 128 * g - 1) / (128 * g);
    const double cost = g == 3 ? 1.0 : kCostG2;
    for (int sp = 2; sp <= kMaxSplit; ++sp) {
      if (nt < 2 * sp) break;
      const int64_t per_xcd = (static_cast<int64_t>(H) * qt * sp + kXcdsAttn - 1) / kXcdsAttn;
      const double f = static_cast<double>((per_xcd + kCUsPerXcd - 1) / kCUsPerXcd) * cost / sp;
      if (f < best - 1e-9) {
        best = f;
        *S = sp;
        *G = g;
        *tiles = static_cast<int>(qt);
      }
    }
  }
}

}  // namespace

size_t attention_ws_bytes(int64_t nq, int64_t N, int H, int d) {
  if (d != 128 || nq < 1 || N < 1 || H < 1) return 0;
  int G, tiles, S;
  plan_split_d128(nq, N, H, &G, &tiles, &S);
  return S > 1 ? static_cast<size_t>(S) * nq * H * 130 * sizeof(float) : 0;
}

void attention_tiles_ws(int64_t nq, int64_t N, int H, int d, int32_t plan[4]) {
  attention_tiles(nq, H, d, plan);
  plan[3] = 1;
  if (d != 128) return;
  int G, tiles, S;
  plan_split_d128(nq, N, H, &G, &tiles, &S);
  if (S > 1) {
    plan[0] = G == 3 ? tiles : 0;
    plan[1] = G == 2 ? tiles : 0;
    plan[3] = S;
  }
}

void attention_tiles(int64_t nq, int H, int d, int32_t tiles[3]) {
  tiles[0] = tiles[1] = tiles[2] = 0;
  if (d == 128) {
    int k3, m2;
    plan_d128(nq, H, &k3, &m2);
    tiles[0] = k3;
    tiles[1] = m2;
  } else {
    tiles[2] = static_cast<int32_t>((nq + kBM - 1) / kBM);
  }
}

hipError_t launch_attention(const uint16_t *Q, int64_t nq, const uint16_t *K, const uint16_t *V,
                            int64_t N, int H, int d, float scale, uint16_t *out, float *ws, hipStream_t s) {
  if (nq == 0) return hipSuccess;
  const float scale_log2 = scale * 1.4426950408889634f;
  if (d == 128 && ws != nullptr) {
    int G, tiles, S;
    plan_split_d128(nq, N, H, &G, &tiles, &S);
    if (S > 1) {
      const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(H) * tiles * S));
      if (G == 3)
        hipLaunchKernelGGL(attn_split_d128_kernel<3>, grid, dim3(kW2 * kWave), 0, s, Q, K, V,
                           static_cast<int>(nq), static_cast<int>(N), H, scale_log2, tiles, S, ws);
      else
        hipLaunchKernelGGL(attn_split_d128_kernel<2>, grid, dim3(kW2 * kWave), 0, s, Q, K, V,
                           static_cast<int>(nq), static_cast<int>(N), H, scale_log2, tiles, S, ws);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      const int64_t nthreads = nq * H * 16;
      hipLaunchKernelGGL(combine_kernel, dim3(static_cast<unsigned>((nthreads + kCombineThreads - 1) / kCombineThreads)),
                         dim3(kCombineThreads), 0, s, ws, static_cast<int>(nq), H, S, out);
      return hipGetLastError();
    }
  }
  if (d == 128) {
    int k3, m2;
    plan_d128(nq, H, &k3, &m2);
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(H) * (k3 + m2)));
    auto kernel = m2 == 0 ? attn_fwd_d128_kernel<3> : k3 == 0 ? attn_fwd_d128_kernel<2> : attn_fwd_d128_kernel<0>;
    hipLaunchKernelGGL(kernel, grid, dim3(kW2 * kWave), 0, s, Q, K, V, out, static_cast<int>(nq),
                       static_cast<int>(N), H, scale_log2, k3, m2);
  } else {
    const dim3 grid(static_cast<unsigned>((nq + kBM - 1) / kBM), static_cast<unsigned>(H));
    hipLaunchKernelGGL(attn_fwd_kernel<64>, grid, dim3(kThreads), 0, s, Q, K, V, out,
                       static_cast<int>(nq), static_cast<int>(N), H, scale_log2);
  }
  return hipGetLastError();
}

}  // namespace jano
