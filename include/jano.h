/*
 * jano.h -- C ABI of libjano, the MI355X (gfx950) hot path of Jano's
 * convergence-adaptive DiT generation.
 *
 * Method: "Jano: Adaptive Diffusion Generation with Early-stage Convergence
 * Awareness" as summarised on its gist.science pages (nl, fr, pt, zh, ko).
 * Citations below name those pages by language and the section of their
 * technical summary.
 *
 * Conventions (all entry points):
 *   - Tensor arguments are DEVICE pointers to caller-owned memory, densely
 *     packed (C order) with the layout given per argument. Structs and
 *     scalar arguments are host values. bf16 data travels as uint16_t bits.
 *   - `stream` is a hipStream_t (NULL = the default stream). Every call only
 *     enqueues work on that stream and returns without synchronising; kernel
 *     faults surface at the caller's next synchronisation.
 *   - Return value: JANO_OK (0) or a negative JANO_E_* code. Arguments are
 *     validated on the host before anything is enqueued; on a non-zero return
 *     nothing was launched and no output was written (except JANO_E_HIP,
 *     reported when a launch itself fails).
 *   - The library allocates no device memory at run time and keeps no state
 *     between calls; calls on different streams may run concurrently as long
 *     as their outputs do not overlap. The one exception is
 *     jano_analyze_noalloc: its scratch array is a fixed part of the library,
 *     one per GPU, and the library remembers that array's device address after
 *     the first call on each device (see there).
 */
#ifndef JANO_H
#define JANO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define JANO_ABI_VERSION 1

enum {
  JANO_OK = 0,
  JANO_E_INVAL = -1,       /* null pointer, bad size, inconsistent geometry */
  JANO_E_UNSUPPORTED = -2, /* valid but not implemented (e.g. head dim)     */
  JANO_E_RANGE = -3,       /* index list out of range / not ascending       */
  JANO_E_WORKSPACE = -4,   /* workspace missing or too small                */
  JANO_E_HIP = -5,         /* a HIP launch reported an error                */
  JANO_E_SCRATCH = -6      /* problem exceeds the built-in scratch buffer   */
};

/* Size of the fixed per-device scratch array jano_analyze_noalloc uses in
 * place of a workspace (4 MiB: the partial sums of grids up to, e.g., 16
 * channels x 16384 blocks with one strip per block row). */
#define JANO_NOALLOC_SCRATCH_BYTES (4u << 20)

/* Latent history and token geometry.
 *   K x [C, F, H, W]  warm-up latents (K >= 3), fp32
 *   (bF, bH, bW)      analyzer block in latent pixels (frame x height x width)
 *   (pF, pH, pW)      patch: latent pixels per token; F, H, W must be
 *                     multiples of the patch and each block dimension a
 *                     multiple of the patch dimension.
 * Tokens form the grid (F/pF, H/pH, W/pW) in order n = (f*Ht + h)*Wt + w;
 * blocks form the grid ceil(F/bF) x ceil(H/bH) x ceil(W/bW) in order
 * b = (bf*nBH + bh)*nBW + bw (edge blocks may be ragged). A geometry with
 * more than 16384 blocks, or with any size below 1 (K below 3), is rejected
 * with JANO_E_INVAL by every entry point that takes it. */
typedef struct jano_grid {
  int32_t K, C, F, H, W;
  int32_t bF, bH, bW;
  int32_t pF, pH, pW;
} jano_grid;

/* Phases of the interleaved pipeline: steps [0, W) warm-up (dense),
 * [T-Cd, T) cool-down (dense); in between a token of level L (1 Static,
 * 2 Moderate, 3 Active) is recomputed when (step - W) % period[L-1] == 0. */
typedef struct jano_sched {
  int32_t T, W, Cd;
  int32_t period[3];
} jano_sched;

int jano_abi_version(void);
const char *jano_status_string(int status);

/* Host helpers (no device access): number of analyzer blocks and tokens. */
int jano_grid_sizes(const jano_grid *g, int64_t *num_blocks, int64_t *num_tokens);

/* Host helper: number of tokens jano_schedule selects at `step`, from the
 * per-level token counts (host copy of jano_analyze's level_tok_counts). */
int jano_schedule_count(const int32_t *level_tok_counts_host, const jano_sched *sc,
                        int step, int64_t *n_act);

/* Device workspace jano_analyze needs, in bytes (0 on invalid geometry). */
size_t jano_analyze_workspace_bytes(const jano_grid *g);

/*
 * jano_analyze_scores -- block-wise complexity analyzer (scores only).
 * Pages: zh technical summary §2.1 (3D blocks, temporal and spatial gradients,
 * second-order difference over the first K steps, one score per block);
 * fr/pt/ko §2.A.
 *
 *   lat               [K][C][F][H][W] fp32, the latents entering steps 0..K-1
 *                     (finite values)
 *   scores   (out)    [B] fp32: mean |D_k(p+e_a) - D_k(p)| over the axes a
 *                     with extent >= 2, k = 1..K-2, all channels and every p
 *                     in the block with p+e_a inside the latent, where
 *                     D_k = L_{k+1} - 2 L_k + L_{k-1} (formed in fp64)
 *   ws, ws_bytes      device workspace of >= jano_analyze_workspace_bytes
 *                     (contents need no initialisation)
 * Deterministic: the same input gives bit-identical scores.
 */
int jano_analyze_scores(const float *lat, const jano_grid *g, float *scores, void *ws,
                        size_t ws_bytes, void *stream);

/*
 * jano_fft_scores -- the FFT complexity baseline, an alternative index source.
 * Pages: fr §2.A (frequency measures such as the FFT, which the analyzer
 * replaces because they are unreliable on noisy early latents); zh §2.1 (the
 * comparison: an FFT taken directly on the early latents); pt results. The
 * pages give no formula; the measure taken is the energy of each block's 3D
 * DFT outside the DC term, divided by n^2, averaged over the channels.
 *
 *   lat               [K][C][F][H][W] fp32 (finite values); only the latest
 *                     latent, L[K-1], is read
 *   scores   (out)    [B] fp32: per block, the mean over channels of
 *                     sum_{k != 0} |DFT(L[K-1][c] restricted to the block)_k|^2 / n^2
 *                     with n the block's pixels inside the latent -- by
 *                     Parseval the population variance of those pixels, which
 *                     is what is computed (one pass of fp64 sums of each pixel's
 *                     difference from the block's first pixel, and of its square)
 * Rank the scores with jano_levels exactly as the analyzer's. No workspace.
 * Deterministic. Errors: JANO_E_INVAL for null pointers or a bad grid.
 */
int jano_fft_scores(const float *lat, const jano_grid *g, float *scores, void *stream);

/*
 * jano_levels -- level bucketing of block scores.
 * Pages: nl methodology §1 (three convergence levels: static, moderate,
 * active); zh §2.1.
 *
 *   scores            [B] fp32 block scores, finite and >= 0 (as written by
 *                     jano_analyze_scores)
 *   static_permille,  share of blocks (per mille, rounded half up) assigned
 *   moderate_permille Static (lowest scores) and Moderate (next); the rest are
 *                     Active. Each >= 0, sum <= 1000.
 *   levels   (out)    [B] uint8 in {1,2,3}: blocks ranked by (score, block id);
 *                     rank < nS -> 1, rank < nSM -> 2, else 3, with
 *                     nS = (static_permille*B + 500) / 1000 and
 *                     nSM = ((static_permille+moderate_permille)*B + 500) / 1000
 *   level_tok_counts (out) [3] int32: tokens at level 1, 2, 3
 * Needs no workspace.
 */
int jano_levels(const float *scores, const jano_grid *g, int static_permille,
                int moderate_permille, uint8_t *levels, int32_t *level_tok_counts,
                void *stream);

/*
 * jano_analyze -- jano_analyze_scores followed by jano_levels on one stream;
 * arguments as there.
 */
int jano_analyze(const float *lat, const jano_grid *g, int static_permille,
                 int moderate_permille, float *scores, uint8_t *levels,
                 int32_t *level_tok_counts, void *ws, size_t ws_bytes, void *stream);

/*
 * jano_analyze_noalloc -- jano_analyze for callers that cannot allocate
 * device memory or hand over a workspace (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).
 * Arguments, outputs and results as jano_analyze, without ws/ws_bytes: the
 * partial sums live in a fixed array of JANO_NOALLOC_SCRATCH_BYTES inside
 * the library, one per GPU, held until the process ends. The call allocates
 * nothing. The first call on a device looks the array's device address up
 * (with that device current, so the stream must belong to the current
 * device); later calls reuse it.
 *   Returns JANO_E_SCRATCH, with nothing launched, when the grid needs more
 *   than JANO_NOALLOC_SCRATCH_BYTES (jano_analyze_workspace_bytes(g) tells).
 *   Every call on one GPU shares that GPU's array: calls that may overlap in
 *   time on one GPU (different streams, or different threads enqueueing
 *   without ordering) race and must be serialised by the caller. Stream order
 *   is enough: calls enqueued on one stream never overlap. The array needs no
 *   clearing between calls (every word read was written by the same call).
 */
int jano_analyze_noalloc(const float *lat, const jano_grid *g, int static_permille,
                         int moderate_permille, float *scores, uint8_t *levels,
                         int32_t *level_tok_counts, void *stream);

/*
 * jano_schedule -- active index list of one denoising step.
 * Pages: nl methodology §2 (warm-up, interleaved generation with per-level
 * update frequency, cool-down); zh §2.2 item 2; pt/fr/ko §2.B.
 *
 *   levels   [B] uint8 block levels (from jano_analyze)
 *   idx      (out) int32 [capacity >= N]: ascending token indices due at
 *            `step`; entries past n_act are left untouched
 *   n_act_dev (out) one int32 on the device: number of indices written
 *   0 <= step < T.
 */
int jano_schedule(const uint8_t *levels, const jano_grid *g, const jano_sched *sc,
                  int step, int32_t *idx, int32_t *n_act_dev, void *stream);

/*
 * jano_schedule_frozen -- the complement of jano_schedule: ascending indices
 * of the tokens NOT computed at `step` (their keys/values come from the cache),
 * as used by the concatenated layout. Arguments as jano_schedule; empty at
 * warm-up and cool-down steps.
 * Pages: nl methodology §2; zh §2.2 item 3 (frozen tokens' cached K/V).
 */
int jano_schedule_frozen(const uint8_t *levels, const jano_grid *g, const jano_sched *sc,
                         int step, int32_t *idx, int32_t *n_frozen_dev, void *stream);

/*
 * jano_gather_rows -- adaptive token activation: X_act[i,:] = X[idx[i],:].
 * Pages: nl contributions item 2 (adaptive token activation); zh §3 item 2.
 *   X [N][D] bf16, idx [n_act] int32 in [0, N), X_act (out) [n_act][D] bf16.
 * Bit-exact copy. n_act == 0 is a no-op.
 */
int jano_gather_rows(const uint16_t *X, int64_t N, int64_t D, const int32_t *idx,
                     int64_t n_act, uint16_t *X_act, void *stream);

/*
 * jano_scatter_kv -- write fresh K/V rows of the active tokens into the
 * full-sequence cache: Kc[idx[i]] = K_new[i], Vc[idx[i]] = V_new[i].
 * Pages: nl methodology §2 (KV cache of frozen tokens); zh §2.2 item 3.
 *   K_new, V_new [n_act][H*d] bf16; Kc, Vc [N][H*d] bf16, updated in place.
 *   idx must hold distinct indices (duplicates race).
 */
int jano_scatter_kv(const uint16_t *K_new, const uint16_t *V_new, const int32_t *idx,
                    int64_t n_act, uint16_t *Kc, uint16_t *Vc, int64_t N, int64_t HD,
                    void *stream);

/*
 * jano_concat_kv -- the pages' layout of an interleaved step: fresh K/V rows of
 * the active tokens first, then the cached rows of the frozen tokens, with
 * positions not restored (attention does not depend on key order).
 * Pages: nl methodology §2; fr §2.B; ko KV-cache item.
 *   K_new, V_new [n_act][HD] bf16 (fresh rows); Kc, Vc [N][HD] bf16 cache;
 *   frozen_idx [n_frozen] indices into the cache (from jano_schedule_frozen);
 *   Kcat, Vcat (out) [n_act + n_frozen][HD]:
 *     Kcat[r] = K_new[r] for r < n_act, Kc[frozen_idx[r - n_act]] after.
 * The scatter cache (jano_attn_step) gives the same attention output with
 * fewer bytes moved; this call exists to measure and test the pages' variant.
 */
int jano_concat_kv(const uint16_t *K_new, const uint16_t *V_new, int64_t n_act,
                   const uint16_t *Kc, const uint16_t *Vc, const int32_t *frozen_idx,
                   int64_t n_frozen, uint16_t *Kcat, uint16_t *Vcat, int64_t HD, void *stream);

/*
 * jano_qkv_proj -- project the active tokens' hidden states to Q, K, V and
 * apply a 3D rotary position encoding to Q and K.
 * Pages: only the active tokens are computed in an interleaved step (nl
 * methodology §2; zh §2.2 item 3) and cached keys keep the encoding they were
 * computed with, positions never restored (fr §2.B). The projection and the
 * encoding are model details the pages do not give; the form here:
 *   y = W x[idx[i]]                 W = Wqkv [3*H*d][Dm] bf16 (rows Q, K, V;
 *                                   head-major then dim), x = X [N][Dm] bf16,
 *                                   fp32 accumulation;
 *   Q, K rotated per token position (frame, row, column) of token idx[i] in
 *   the token grid of g: the head dim splits into d_f = d - 4*floor(d/6) and
 *   d_h = d_w = 2*floor(d/6) dims; pair k of a part of m dims turns dims
 *   (2k, 2k+1) of that part by pos * rope_base^(-2k/m).
 *   g NULL or rope_base <= 0: no rotation (g may then be NULL).
 *   Q, K_new, V_new (out) [n_act][H][d] bf16, 16-byte aligned.
 * Needs Dm a multiple of 32, d a multiple of 4 (and >= 6 with rotation),
 * N*Dm*2 < 2^32 bytes (JANO_E_UNSUPPORTED otherwise); idx entries in [0, N).
 */
int jano_qkv_proj(const uint16_t *X, int64_t N, int64_t Dm, const int32_t *idx, int64_t n_act,
                  const uint16_t *Wqkv, int H, int d, const jano_grid *g, float rope_base,
                  uint16_t *Q, uint16_t *K_new, uint16_t *V_new, void *stream);

/*
 * jano_attention -- non-causal softmax attention of n_q queries against all
 * N cached keys/values, per head: out[i,h] = softmax(Q[i,h] Kc[:,h]^T * scale) Vc[:,h].
 * Pages: full attention over all tokens, quadratic in sequence length
 * (nl problem statement; fr §1); order of keys/values is irrelevant
 * (nl methodology §2).
 *   Q [n_q][H][d], Kc, Vc [N][H][d], out (out) [n_q][H][d], all bf16;
 *   d in {64, 128}; scale <= 0 selects 1/sqrt(d); a non-finite scale is
 *   JANO_E_INVAL. Q, Kc, Vc must hold finite values (NaN/Inf inputs give
 *   unspecified outputs). bf16 MFMA products, fp32 accumulation and online
 *   softmax. n_q == 0 is a no-op; N >= 1.
 */
int jano_attention(const uint16_t *Q, int64_t n_q, const uint16_t *Kc, const uint16_t *Vc,
                   int64_t N, int H, int d, float scale, uint16_t *out, void *stream);

/*
 * jano_attention_plan -- host helper (no device access): how jano_attention
 * and jano_attn_step split the n_q queries of each of H heads into
 * workgroup tiles at head dim d.
 *   tiles_per_head (out) [3]: [0] tiles of 384 queries, [1] tiles of 256
 *   queries (d = 128), [2] tiles of 128 queries (d = 64). With d = 128 a head
 *   is covered by [0] tiles from its first query on, then [1] tiles (the
 *   last tile of the head may be ragged); the 256-query workgroups run last,
 *   to fill the launch's final round on the GPU's compute units (one
 *   workgroup per unit at a time).
 * Errors: JANO_E_INVAL (n_q or H below 1, null output), JANO_E_UNSUPPORTED (d).
 */
int jano_attention_plan(int64_t n_q, int H, int d, int32_t *tiles_per_head);

/*
 * jano_attn_step -- one interleaved-step attention: jano_scatter_kv of the
 * fresh rows into the cache, then jano_attention of the active queries against
 * the whole cache, on one stream (the scatter completes before attention reads).
 * Pages: nl methodology §2 (cached pairs of frozen tokens combined with the
 * active queries without restoring positions); zh §2.2 item 3; pt §2.B.
 *   Q_act, K_new, V_new [n_act][H][d]; idx [n_act] ascending distinct in [0,N);
 *   Kc, Vc [N][H][d] in/out; out (out) [n_act][H][d].
 */
int jano_attn_step(const uint16_t *Q_act, const uint16_t *K_new, const uint16_t *V_new,
                   const int32_t *idx, int64_t n_act, uint16_t *Kc, uint16_t *Vc,
                   int64_t N, int H, int d, float scale, uint16_t *out, void *stream);

/*
 * jano_attention_ws, jano_attn_step_ws -- jano_attention and jano_attn_step
 * with an optional workspace. With one, a launch may split each head's keys
 * into S key ranges handled by S workgroups each. It does so when its query
 * tiles alone would leave the GPU's compute units idle for much of the
 * launch (few queries, or a mostly empty last round). Each key range writes
 * its partial result to ws: the unnormalised fp32 output, the running max and
 * the row sum. A second launch merges the ranges in range order.
 * Pages: as jano_attention / jano_attn_step (nl problem statement; nl
 * methodology §2); the split is how this library fills the GPU.
 *   ws, ws_bytes   NULL: exactly jano_attention / jano_attn_step. Otherwise
 *                  a device buffer, 16-byte aligned, of at least
 *                  jano_attention_workspace_bytes(n_q or n_act, N, H, d) bytes;
 *                  contents need no initialisation. When that size is 0 the
 *                  plan does not split and ws is not touched.
 * Other arguments, layouts and results as there. A split launch sums over
 * the keys in another order than the unsplit one, so the two differ by
 * rounding; each is deterministic.
 * Errors: as there, and JANO_E_WORKSPACE (nothing launched) when the plan
 * splits and ws is too small or misaligned.
 */
int jano_attention_ws(const uint16_t *Q, int64_t n_q, const uint16_t *Kc, const uint16_t *Vc,
                      int64_t N, int H, int d, float scale, uint16_t *out, void *ws, size_t ws_bytes,
                      void *stream);
int jano_attn_step_ws(const uint16_t *Q_act, const uint16_t *K_new, const uint16_t *V_new,
                      const int32_t *idx, int64_t n_act, uint16_t *Kc, uint16_t *Vc, int64_t N, int H,
                      int d, float scale, uint16_t *out, void *ws, size_t ws_bytes, void *stream);

/* Host helper: bytes of workspace jano_attention_ws / jano_attn_step_ws need
 * for n_q queries against N keys (0: the plan does not split; always 0 for
 * d = 64 and for invalid sizes). */
size_t jano_attention_workspace_bytes(int64_t n_q, int64_t N, int H, int d);

/* Host helper: the plan of jano_attention_ws given a workspace.
 *   plan (out) [4]: [0..2] tiles per head as jano_attention_plan reports them
 *   (for a split plan, the one query-tile form it uses), [3] key ranges per
 *   query tile (1: no split).
 * Errors: JANO_E_INVAL (n_q, N or H below 1, null output), JANO_E_UNSUPPORTED (d). */
int jano_attention_plan_ws(int64_t n_q, int64_t N, int H, int d, int32_t *plan);

/*
 * jano_writeback_step -- write the active tokens' model output back and take
 * one sampler (Euler) step for every token.
 * Pages: nl "three groups" (the static group rests while its result is
 * remembered); zh three token classes (static regions skip intermediate steps
 * and use the cache instead); ko §2 (skipped parts keep the previous state
 * held in memory). Every token keeps its latest model output; frozen tokens
 * step with the output cached at their last update.
 *   out_act  [n_act][P] bf16: fresh model output of the tokens idx
 *   idx      [n_act] distinct indices in [0, N) (from jano_schedule)
 *   out_full [N][P] bf16, in/out: every token's latest output; rows idx are
 *            replaced by out_act
 *   x        [N][P] fp32, in/out: sampler state in token-major patch layout;
 *            x = fma(dt, out_full, x) elementwise after the write-back
 *   dt       finite step size (the sampler's signed time increment)
 * n_act == 0 only steps x. Duplicate indices race.
 */
int jano_writeback_step(const uint16_t *out_act, const int32_t *idx, int64_t n_act,
                        uint16_t *out_full, float *x, int64_t N, int64_t P, float dt,
                        void *stream);

/*
 * jano_check_idx -- validate an index list on the device: writes 0 to
 * *flag_dev when idx is strictly ascending within [0, N), else JANO_E_RANGE.
 * Debug aid for the precondition of jano_scatter_kv / jano_attn_step.
 */
int jano_check_idx(const int32_t *idx, int64_t n_act, int64_t N, int32_t *flag_dev,
                   void *stream);

#ifdef __cplusplus
}
#endif

#endif /* JANO_H */
