// Internal launch interface between the C ABI (capi.hip) and the kernels.
// All launchers assume arguments were validated by the caller and return a
// hipError_t from the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace jano {

// Geometry of one analyzer launch, fully derived on the host.
struct AnalyzeGeom {
  int K, C, F, H, W;
  int bF, bH, bW;
  int pF, pH, pW;
  int nBF, nBH, nBW;
  int B;
  int R;    // latent rows per strip (a strip is one wave's row range)
  int G;    // strips per block row, bH / R
  int CW;   // useful columns per wave (multiple of bW, < 64)
  int nWC;  // column chunks, ceil(W / CW)
  int FC;   // frames per chunk (multiple of bF)
  int nFC;  // frame chunks, ceil(F / FC)
  bool fast;  // streaming stencil kernel instantiated for (K, R)
};

bool analyze_plan(int K, int C, int F, int H, int W, int bF, int bH, int bW, int pF,
                  int pH, int pW, AnalyzeGeom *g);
size_t analyze_ws_bytes(const AnalyzeGeom &g);
// jano_analyze_scores: kernels 1 and 2 (scores [B]; ws holds the partials)
hipError_t launch_analyze_scores(const float *lat, const AnalyzeGeom &g, float *scores, void *ws,
                                 hipStream_t s);
// jano_fft_scores: the FFT complexity baseline's block scores [B]
hipError_t launch_fft_scores(const float *lat, const AnalyzeGeom &g, float *scores, hipStream_t s);
// jano_levels: kernels 3 and 4 (levels [B], tokens per level [3])
hipError_t launch_levels(const float *scores, const AnalyzeGeom &g, int nS, int nSM, uint8_t *levels,
                         int32_t *counts, hipStream_t s);

struct SchedGeom {
  int Ft, Ht, Wt;         // token grid
  int pF, pH, pW;         // patch
  int bF, bH, bW;         // block (latent px)
  int nBF, nBH, nBW;      // block grid
  int N;
  int due[3];             // whether level 1/2/3 is recomputed at this step
};
hipError_t launch_schedule(const uint8_t *levels, const SchedGeom &g, int32_t *idx,
                           int32_t *n_act, hipStream_t s);
hipError_t launch_check_idx(const int32_t *idx, int64_t n, int64_t N, int32_t *flag,
                            hipStream_t s);

hipError_t launch_gather_rows(const uint16_t *X, int64_t D, const int32_t *idx,
                              int64_t n, uint16_t *out, hipStream_t s);
hipError_t launch_scatter_kv(const uint16_t *Kn, const uint16_t *Vn, const int32_t *idx,
                             int64_t n, uint16_t *Kc, uint16_t *Vc, int64_t HD,
                             hipStream_t s);

// out_full-style single-tensor row scatter: dst[idx[i]] = src[i], rows of D bf16
hipError_t launch_scatter_rows(const uint16_t *src, int64_t D, const int32_t *idx, int64_t n,
                               uint16_t *dst, hipStream_t s);
// Kcat = [Kn rows 0..n_act) ; Kc[frozen[0..n_frozen))], same for V; rows of HD bf16
hipError_t launch_concat_kv(const uint16_t *Kn, const uint16_t *Vn, int64_t n_act, const uint16_t *Kc,
                            const uint16_t *Vc, const int32_t *frozen, int64_t n_frozen, uint16_t *Kcat,
                            uint16_t *Vcat, int64_t HD, hipStream_t s);
// x[e] = fma(dt, v[e], x[e]) over total elements (v bf16, x fp32)
hipError_t launch_euler(const uint16_t *v, float *x, int64_t total, float dt, hipStream_t s);
// gathered QKV projection (+ 3D rotary on Q, K); see proj.hip
bool qkv_proj_supported(int64_t N, int64_t Dm, int H, int d);
hipError_t launch_qkv_proj(const uint16_t *X, int64_t Dm, const int32_t *idx, int64_t n_act,
                           const uint16_t *W, int H, int d, int Ht, int Wt, float rope_base,
                           uint16_t *Q, uint16_t *Kn, uint16_t *Vn, hipStream_t s);
// query tiles per head of the attention launch for (nq, H, d): 384-query and
// 256-query tiles (d = 128), 128-query tiles (d = 64)
void attention_tiles(int64_t nq, int H, int d, int32_t tiles[3]);
// with a workspace: plan[0..2] as attention_tiles, plan[3] the key ranges per
// query tile (1: no split); bytes of workspace that plan needs (0: none)
void attention_tiles_ws(int64_t nq, int64_t N, int H, int d, int32_t plan[4]);
size_t attention_ws_bytes(int64_t nq, int64_t N, int H, int d);
// ws NULL: one launch, every workgroup over all keys; otherwise (d = 128) the
// keys may be split over workgroups per the plan, partials in ws (of at least
// attention_ws_bytes) and a combine launch
hipError_t launch_attention(const uint16_t *Q, int64_t nq, const uint16_t *K,
                            const uint16_t *V, int64_t N, int H, int d, float scale,
                            uint16_t *out, float *ws, hipStream_t s);

}  // namespace jano
