// C ABI of libjano: host-side argument validation and kernel launches.
// Every check happens before anything is enqueued, so a non-zero return
// means nothing ran and no output was touched.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/jano.h"
#include "kernels.hpp"

using jano::AnalyzeGeom;

// Scratch memory of jano_analyze_noalloc: the analyzer's partial sums live in
// this fixed array instead of a caller workspace. Each GPU the library runs on
// holds its own copy, at its own address, until the process ends. In host
// code the name `scratch` is only a host-side stand-in, never a device
// address: kernels get the address hipGetSymbolAddress returns for the current
// device (scratch_device_ptr).
static __device__ __align__(256) unsigned char scratch[JANO_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int64_t kMaxRows = 0x7fffffffLL;

bool grid_ok(const jano_grid *g, AnalyzeGeom *out) {
  if (!g) return false;
  return jano::analyze_plan(g->K, g->C, g->F, g->H, g->W, g->bF, g->bH, g->bW, g->pF, g->pH,
                            g->pW, out);
}

bool sched_ok(const jano_sched *sc) {
  if (!sc) return false;
  if (sc->T < 1 || sc->W < 0 || sc->Cd < 0 || sc->W + sc->Cd > sc->T) return false;
  for (int i = 0; i < 3; ++i)
    if (sc->period[i] < 1) return false;
  return true;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? JANO_OK : JANO_E_HIP; }

bool mix_ok(int static_permille, int moderate_permille) {
  return static_permille >= 0 && moderate_permille >= 0 && static_permille + moderate_permille <= 1000;
}

// rank thresholds of the level split: ranks < nS are Static, < nSM Moderate
void split_ranks(int B, int static_permille, int moderate_permille, int *nS, int *nSM) {
  const long long b = B;
  *nS = static_cast<int>((static_permille * b + 500) / 1000);
  *nSM = static_cast<int>(((static_permille + moderate_permille) * b + 500) / 1000);
}

void due_flags(const jano_sched *sc, int step, int due[3]) {
  const bool dense = step < sc->W || step >= sc->T - sc->Cd;
  for (int i = 0; i < 3; ++i) due[i] = dense || ((step - sc->W) % sc->period[i] == 0);
}

int schedule_impl(const uint8_t *levels, const jano_grid *g, const jano_sched *sc, int step,
                  int32_t *idx, int32_t *n_dev, bool frozen, hipStream_t stream) {
  if (!levels || !idx || !n_dev) return JANO_E_INVAL;
  AnalyzeGeom a;
  if (!grid_ok(g, &a) || !sched_ok(sc) || step < 0 || step >= sc->T) return JANO_E_INVAL;
  jano::SchedGeom s{};
  s.Ft = g->F / g->pF;
  s.Ht = g->H / g->pH;
  s.Wt = g->W / g->pW;
  const int64_t N = static_cast<int64_t>(s.Ft) * s.Ht * s.Wt;
  if (N > kMaxRows) return JANO_E_UNSUPPORTED;
  s.N = static_cast<int>(N);
  s.pF = g->pF; s.pH = g->pH; s.pW = g->pW;
  s.bF = g->bF; s.bH = g->bH; s.bW = g->bW;
  s.nBF = a.nBF;
  s.nBH = a.nBH;
  s.nBW = a.nBW;
  due_flags(sc, step, s.due);
  if (frozen)
    for (int i = 0; i < 3; ++i) s.due[i] = !s.due[i];
  return hip_status(jano::launch_schedule(levels, s, idx, n_dev, stream));
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
hipError_t scratch_device_ptr(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

int jano_abi_version(void) { return JANO_ABI_VERSION; }

const char *jano_status_string(int status) {
  switch (status) {
    case JANO_OK: return "ok";
    case JANO_E_INVAL: return "invalid argument";
    case JANO_E_UNSUPPORTED: return "unsupported configuration";
    case JANO_E_RANGE: return "index out of range or not strictly ascending";
    case JANO_E_WORKSPACE: return "workspace missing or too small";
    case JANO_E_HIP: return "HIP launch error";
    case JANO_E_SCRATCH: return "problem larger than the built-in scratch buffer (JANO_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int jano_grid_sizes(const jano_grid *g, int64_t *num_blocks, int64_t *num_tokens) {
  AnalyzeGeom a;
  if (!grid_ok(g, &a)) return JANO_E_INVAL;
  if (num_blocks) *num_blocks = a.B;
  if (num_tokens)
    *num_tokens = static_cast<int64_t>(g->F / g->pF) * (g->H / g->pH) * (g->W / g->pW);
  return JANO_OK;
}

int jano_schedule_count(const int32_t *counts, const jano_sched *sc, int step, int64_t *n_act) {
  if (!counts || !n_act || !sched_ok(sc) || step < 0 || step >= sc->T) return JANO_E_INVAL;
  int due[3];
  due_flags(sc, step, due);
  int64_t n = 0;
  for (int i = 0; i < 3; ++i) {
    if (counts[i] < 0) return JANO_E_INVAL;
    if (due[i]) n += counts[i];
  }
  *n_act = n;
  return JANO_OK;
}

size_t jano_analyze_workspace_bytes(const jano_grid *g) {
  AnalyzeGeom a;
  if (!grid_ok(g, &a)) return 0;
  return jano::analyze_ws_bytes(a);
}

int jano_analyze_scores(const float *lat, const jano_grid *g, float *scores, void *ws,
                        size_t ws_bytes, void *stream) {
  if (!lat || !scores) return JANO_E_INVAL;
  AnalyzeGeom a;
  if (!grid_ok(g, &a)) return JANO_E_INVAL;
  if (!ws || ws_bytes < jano::analyze_ws_bytes(a)) return JANO_E_WORKSPACE;
  return hip_status(jano::launch_analyze_scores(lat, a, scores, ws, static_cast<hipStream_t>(stream)));
}

int jano_fft_scores(const float *lat, const jano_grid *g, float *scores, void *stream) {
  if (!lat || !scores) return JANO_E_INVAL;
  AnalyzeGeom a;
  if (!grid_ok(g, &a)) return JANO_E_INVAL;
  return hip_status(jano::launch_fft_scores(lat, a, scores, static_cast<hipStream_t>(stream)));
}

int jano_levels(const float *scores, const jano_grid *g, int static_permille, int moderate_permille,
                uint8_t *levels, int32_t *level_tok_counts, void *stream) {
  if (!scores || !levels || !level_tok_counts) return JANO_E_INVAL;
  AnalyzeGeom a;
  if (!grid_ok(g, &a) || !mix_ok(static_permille, moderate_permille)) return JANO_E_INVAL;
  int nS, nSM;
  split_ranks(a.B, static_permille, moderate_permille, &nS, &nSM);
  return hip_status(jano::launch_levels(scores, a, nS, nSM, levels, level_tok_counts,
                                        static_cast<hipStream_t>(stream)));
}

int jano_analyze(const float *lat, const jano_grid *g, int static_permille, int moderate_permille,
                 float *scores, uint8_t *levels, int32_t *level_tok_counts, void *ws,
                 size_t ws_bytes, void *stream) {
  if (!lat || !scores || !levels || !level_tok_counts) return JANO_E_INVAL;
  AnalyzeGeom a;
  if (!grid_ok(g, &a) || !mix_ok(static_permille, moderate_permille)) return JANO_E_INVAL;
  if (!ws || ws_bytes < jano::analyze_ws_bytes(a)) return JANO_E_WORKSPACE;
  int nS, nSM;
  split_ranks(a.B, static_permille, moderate_permille, &nS, &nSM);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (jano::launch_analyze_scores(lat, a, scores, ws, s) != hipSuccess) return JANO_E_HIP;
  return hip_status(jano::launch_levels(scores, a, nS, nSM, levels, level_tok_counts, s));
}

int jano_analyze_noalloc(const float *lat, const jano_grid *g, int static_permille,
                         int moderate_permille, float *scores, uint8_t *levels,
                         int32_t *level_tok_counts, void *stream) {
  if (!lat || !scores || !levels || !level_tok_counts) return JANO_E_INVAL;
  AnalyzeGeom a;
  if (!grid_ok(g, &a) || !mix_ok(static_permille, moderate_permille)) return JANO_E_INVAL;
  if (jano::analyze_ws_bytes(a) > sizeof(scratch)) return JANO_E_SCRATCH;
  void *ws = nullptr;
  if (scratch_device_ptr(&ws) != hipSuccess) return JANO_E_HIP;
  int nS, nSM;
  split_ranks(a.B, static_permille, moderate_permille, &nS, &nSM);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (jano::launch_analyze_scores(lat, a, scores, ws, s) != hipSuccess) return JANO_E_HIP;
  return hip_status(jano::launch_levels(scores, a, nS, nSM, levels, level_tok_counts, s));
}

int jano_schedule_frozen(const uint8_t *levels, const jano_grid *g, const jano_sched *sc, int step,
                         int32_t *idx, int32_t *n_frozen_dev, void *stream) {
  return schedule_impl(levels, g, sc, step, idx, n_frozen_dev, true, static_cast<hipStream_t>(stream));
}

int jano_concat_kv(const uint16_t *K_new, const uint16_t *V_new, int64_t n_act, const uint16_t *Kc,
                   const uint16_t *Vc, const int32_t *frozen_idx, int64_t n_frozen, uint16_t *Kcat,
                   uint16_t *Vcat, int64_t HD, void *stream) {
  if (n_act < 0 || n_frozen < 0 || HD < 1 || n_act > kMaxRows || n_frozen > kMaxRows ||
      n_act + n_frozen > kMaxRows)
    return JANO_E_INVAL;
  if (n_act + n_frozen == 0) return JANO_OK;
  if (!Kcat || !Vcat) return JANO_E_INVAL;
  if (n_act > 0 && (!K_new || !V_new)) return JANO_E_INVAL;
  if (n_frozen > 0 && (!Kc || !Vc || !frozen_idx)) return JANO_E_INVAL;
  return hip_status(jano::launch_concat_kv(K_new, V_new, n_act, Kc, Vc, frozen_idx, n_frozen, Kcat, Vcat,
                                           HD, static_cast<hipStream_t>(stream)));
}

int jano_schedule(const uint8_t *levels, const jano_grid *g, const jano_sched *sc, int step,
                  int32_t *idx, int32_t *n_act_dev, void *stream) {
  return schedule_impl(levels, g, sc, step, idx, n_act_dev, false, static_cast<hipStream_t>(stream));
}

int jano_gather_rows(const uint16_t *X, int64_t N, int64_t D, const int32_t *idx, int64_t n_act,
                     uint16_t *X_act, void *stream) {
  if (N < 1 || D < 1 || n_act < 0 || n_act > kMaxRows || N > kMaxRows) return JANO_E_INVAL;
  if (n_act == 0) return JANO_OK;
  if (!X || !idx || !X_act) return JANO_E_INVAL;
  return hip_status(jano::launch_gather_rows(X, D, idx, n_act, X_act, static_cast<hipStream_t>(stream)));
}

int jano_scatter_kv(const uint16_t *K_new, const uint16_t *V_new, const int32_t *idx,
                    int64_t n_act, uint16_t *Kc, uint16_t *Vc, int64_t N, int64_t HD,
                    void *stream) {
  if (N < 1 || HD < 1 || n_act < 0 || n_act > N || N > kMaxRows) return JANO_E_INVAL;
  if (n_act == 0) return JANO_OK;
  if (!K_new || !V_new || !idx || !Kc || !Vc) return JANO_E_INVAL;
  return hip_status(jano::launch_scatter_kv(K_new, V_new, idx, n_act, Kc, Vc, HD,
                                            static_cast<hipStream_t>(stream)));
}

// the key-split workspace of an attention launch: NULL selects the plain
// launch; otherwise it must hold the plan's bytes (none when it does not split)
static int check_attention_ws(int64_t n_q, int64_t N, int H, int d, const void *ws, size_t ws_bytes,
                              float **wsf) {
  *wsf = nullptr;
  if (ws == nullptr) return JANO_OK;
  const size_t need = jano::attention_ws_bytes(n_q, N, H, d);
  if (need == 0) return JANO_OK;
  if (ws_bytes < need || !aligned16(ws)) return JANO_E_WORKSPACE;
  *wsf = static_cast<float *>(const_cast<void *>(ws));
  return JANO_OK;
}

int jano_attention_ws(const uint16_t *Q, int64_t n_q, const uint16_t *Kc, const uint16_t *Vc,
                      int64_t N, int H, int d, float scale, uint16_t *out, void *ws, size_t ws_bytes,
                      void *stream) {
  if (N < 1 || H < 1 || n_q < 0 || N > kMaxRows || n_q > kMaxRows || !isfinite(scale))
    return JANO_E_INVAL;
  if (d != 64 && d != 128) return JANO_E_UNSUPPORTED;
  if (n_q > 0 && (!Q || !out)) return JANO_E_INVAL;
  if (!Kc || !Vc) return JANO_E_INVAL;
  if (!aligned16(Q) || !aligned16(Kc) || !aligned16(Vc) || !aligned16(out)) return JANO_E_INVAL;
  if (H > 65535) return JANO_E_UNSUPPORTED;
  if (n_q == 0) return JANO_OK;
  float *wsf;
  const int w = check_attention_ws(n_q, N, H, d, ws, ws_bytes, &wsf);
  if (w != JANO_OK) return w;
  const float sc = scale > 0.0f ? scale : 1.0f / sqrtf(static_cast<float>(d));
  return hip_status(jano::launch_attention(Q, n_q, Kc, Vc, N, H, d, sc, out, wsf,
                                           static_cast<hipStream_t>(stream)));
}

int jano_attention(const uint16_t *Q, int64_t n_q, const uint16_t *Kc, const uint16_t *Vc,
                   int64_t N, int H, int d, float scale, uint16_t *out, void *stream) {
  return jano_attention_ws(Q, n_q, Kc, Vc, N, H, d, scale, out, nullptr, 0, stream);
}

size_t jano_attention_workspace_bytes(int64_t n_q, int64_t N, int H, int d) {
  if (n_q < 1 || N < 1 || H < 1 || n_q > kMaxRows || N > kMaxRows || H > 65535) return 0;
  return jano::attention_ws_bytes(n_q, N, H, d);
}

int jano_attention_plan_ws(int64_t n_q, int64_t N, int H, int d, int32_t *plan) {
  if (!plan || n_q < 1 || N < 1 || H < 1 || n_q > kMaxRows || N > kMaxRows) return JANO_E_INVAL;
  if (d != 64 && d != 128) return JANO_E_UNSUPPORTED;
  jano::attention_tiles_ws(n_q, N, H, d, plan);
  return JANO_OK;
}

int jano_attention_plan(int64_t n_q, int H, int d, int32_t *tiles_per_head) {
  if (!tiles_per_head || n_q < 1 || H < 1 || n_q > kMaxRows) return JANO_E_INVAL;
  if (d != 64 && d != 128) return JANO_E_UNSUPPORTED;
  jano::attention_tiles(n_q, H, d, tiles_per_head);
  return JANO_OK;
}

int jano_attn_step_ws(const uint16_t *Q_act, const uint16_t *K_new, const uint16_t *V_new,
                      const int32_t *idx, int64_t n_act, uint16_t *Kc, uint16_t *Vc, int64_t N, int H,
                      int d, float scale, uint16_t *out, void *ws, size_t ws_bytes, void *stream) {
  if (N < 1 || H < 1 || n_act < 0 || n_act > N || N > kMaxRows || !isfinite(scale))
    return JANO_E_INVAL;
  if (d != 64 && d != 128) return JANO_E_UNSUPPORTED;
  if (H > 65535) return JANO_E_UNSUPPORTED;
  if (!Kc || !Vc) return JANO_E_INVAL;
  if (n_act == 0) return JANO_OK;
  if (!Q_act || !K_new || !V_new || !idx || !out) return JANO_E_INVAL;
  if (!aligned16(Q_act) || !aligned16(Kc) || !aligned16(Vc) || !aligned16(out)) return JANO_E_INVAL;
  float *wsf;
  const int w = check_attention_ws(n_act, N, H, d, ws, ws_bytes, &wsf);
  if (w != JANO_OK) return w;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t HD = static_cast<int64_t>(H) * d;
  hipError_t e = jano::launch_scatter_kv(K_new, V_new, idx, n_act, Kc, Vc, HD, s);
  if (e != hipSuccess) return JANO_E_HIP;
  const float sc = scale > 0.0f ? scale : 1.0f / sqrtf(static_cast<float>(d));
  return hip_status(jano::launch_attention(Q_act, n_act, Kc, Vc, N, H, d, sc, out, wsf, s));
}

int jano_attn_step(const uint16_t *Q_act, const uint16_t *K_new, const uint16_t *V_new,
                   const int32_t *idx, int64_t n_act, uint16_t *Kc, uint16_t *Vc, int64_t N, int H,
                   int d, float scale, uint16_t *out, void *stream) {
  return jano_attn_step_ws(Q_act, K_new, V_new, idx, n_act, Kc, Vc, N, H, d, scale, out, nullptr, 0,
                           stream);
}

int jano_qkv_proj(const uint16_t *X, int64_t N, int64_t Dm, const int32_t *idx, int64_t n_act,
                  const uint16_t *Wqkv, int H, int d, const jano_grid *g, float rope_base,
                  uint16_t *Q, uint16_t *K_new, uint16_t *V_new, void *stream) {
  if (N < 1 || Dm < 1 || H < 1 || d < 1 || n_act < 0 || n_act > kMaxRows || N > kMaxRows ||
      !isfinite(rope_base))
    return JANO_E_INVAL;
  if (!jano::qkv_proj_supported(N, Dm, H, d)) return JANO_E_UNSUPPORTED;
  int Ht = 1, Wt = 1;
  float base = 0.0f;
  if (g && rope_base > 0.0f) {
    AnalyzeGeom a;
    if (!grid_ok(g, &a) || d < 6 || d % 2) return JANO_E_INVAL;
    const int64_t Ft = g->F / g->pF;
    Ht = g->H / g->pH;
    Wt = g->W / g->pW;
    if (Ft * Ht * Wt != N) return JANO_E_INVAL;
    base = rope_base;
  }
  if (n_act == 0) return JANO_OK;
  if (!X || !idx || !Wqkv || !Q || !K_new || !V_new) return JANO_E_INVAL;
  if (!aligned16(X) || !aligned16(Wqkv) || !aligned16(Q) || !aligned16(K_new) || !aligned16(V_new))
    return JANO_E_INVAL;
  return hip_status(jano::launch_qkv_proj(X, Dm, idx, n_act, Wqkv, H, d, Ht, Wt, base, Q, K_new, V_new,
                                          static_cast<hipStream_t>(stream)));
}

int jano_writeback_step(const uint16_t *out_act, const int32_t *idx, int64_t n_act,
                        uint16_t *out_full, float *x, int64_t N, int64_t P, float dt, void *stream) {
  if (N < 1 || P < 1 || n_act < 0 || n_act > N || N > kMaxRows || !isfinite(dt)) return JANO_E_INVAL;
  if (N > INT64_MAX / P) return JANO_E_INVAL;
  if (!out_full || !x) return JANO_E_INVAL;
  if (n_act > 0 && (!out_act || !idx)) return JANO_E_INVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (jano::launch_scatter_rows(out_act, P, idx, n_act, out_full, s) != hipSuccess) return JANO_E_HIP;
  return hip_status(jano::launch_euler(out_full, x, N * P, dt, s));
}

int jano_check_idx(const int32_t *idx, int64_t n_act, int64_t N, int32_t *flag_dev, void *stream) {
  if (!flag_dev || n_act < 0 || N < 1 || n_act > kMaxRows) return JANO_E_INVAL;
  if (n_act > 0 && !idx) return JANO_E_INVAL;
  return hip_status(jano::launch_check_idx(idx, n_act, N, flag_dev, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
