"""CPU oracle of the Jano per-step hot path -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct NumPy code. Only the tests, the smoke check and
the bench's CPU-baseline leg may import it; the product path (the HIP library
and its Python binding) never does, and shares no code with it.

Citations name the Jano summary pages on gist.science (one per language:
nl, fr, pt, zh, ko; all titled "Jano: Adaptive Diffusion Generation with
Early-stage Convergence Awareness") and the section of their technical summary.

Readings taken where the pages are silent (each is listed in the design notes):
  * the analyzer differences the gradient fields along the STEP axis (second
    order), using forward differences without padding; gradient pairs may cross
    into the neighbouring block (one-cell halo);
  * the block score is the mean absolute value over every valid
    (axis, step, channel, position) term that starts inside the block;
  * levels are rank quantiles: lowest static_permille of blocks -> 1 (Static),
    next moderate_permille -> 2 (Moderate), rest -> 3 (Active); ties by id;
  * a token is due at step s if s is a warm-up or cool-down step, else if
    (s - W) is a multiple of its level's period; index lists are ascending;
  * attention is non-causal softmax(Q K^T / sqrt(d)) V per head, over the
    whole full-sequence cache after the fresh rows were written into it.

Every function below is pinned by tests/test_oracle_pins.py against closed
forms, invariants and brute force; none is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

STATIC, MODERATE, ACTIVE = 1, 2, 3


# --------------------------------------------------------------------------
# Analyzer: block-wise complexity score.
# Jano pages: [zh] technical summary §2.1 (block-wise complexity analyzer:
# 3D frame x height x width blocks, temporal and spatial gradients, second
# order difference over the first K steps, a complexity score per block);
# [nl] methodology §1; [fr] §2.A; [pt] §2.A; [ko] §2.A.
# --------------------------------------------------------------------------

def block_grid(F: int, H: int, W: int, block) -> tuple:
    bF, bH, bW = block
    return (-(-F // bF), -(-H // bH), -(-W // bW))


def _block_ids(F, H, W, block, nB):
    bF, bH, bW = block
    _, nBH, nBW = nB
    f = np.arange(F) // bF
    h = np.arange(H) // bH
    w = np.arange(W) // bW
    return (f[:, None, None] * nBH + h[None, :, None]) * nBW + w[None, None, :]


def step_second_difference(lat: np.ndarray) -> np.ndarray:
    """D_k = L_{k+1} - 2 L_k + L_{k-1}, k = 1..K-2, in fp64 (exact for fp32 L)."""
    L = np.asarray(lat, dtype=np.float64)
    return L[2:] - 2.0 * L[1:-1] + L[:-2]


def analyze_scores(lat: np.ndarray, block) -> np.ndarray:
    """Per-block complexity score rounded to fp32 [B] (see analyze_scores_f64)."""
    return analyze_scores_f64(lat, block).astype(np.float32)


def analyze_scores_f64(lat: np.ndarray, block) -> np.ndarray:
    """Per-block complexity score, fp64 [B].

    lat: fp32 [K, C, F, H, W], the latents entering steps 0..K-1 (K >= 3).
    The gradient of x along axis a at p is x(p + e_a) - x(p); its second step
    difference equals D_k(p + e_a) - D_k(p) by linearity. The score of block b
    is the mean |.| of those terms over all axes a with extent >= 2, all
    k = 1..K-2, all channels and all p in b with p + e_a inside the latent."""
    K, C, F, H, W = lat.shape
    if K < 3:
        raise ValueError("need K >= 3 warm-up latents")
    D = step_second_difference(lat)               # [K-2, C, F, H, W]
    nB = block_grid(F, H, W, block)
    B = nB[0] * nB[1] * nB[2]
    bid = _block_ids(F, H, W, block, nB)
    total = np.zeros(B, dtype=np.float64)
    count = np.zeros(B, dtype=np.float64)
    for axis in (2, 3, 4):                        # F (temporal), H, W (spatial)
        ext = D.shape[axis]
        if ext < 2:
            continue
        E = np.abs(np.diff(D, axis=axis))         # D(p + e_a) - D(p)
        per_pos = E.sum(axis=(0, 1))              # sum over k and c -> [F', H', W']
        sl = [slice(None)] * 3
        sl[axis - 2] = slice(0, ext - 1)          # positions p with p + e_a valid
        ids = bid[tuple(sl)]
        total += np.bincount(ids.ravel(), weights=per_pos.ravel(), minlength=B)
        count += np.bincount(ids.ravel(), minlength=B) * float(D.shape[0] * C)
    return np.where(count > 0, total / np.where(count > 0, count, 1.0), 0.0)


def analyze_scores_bruteforce(lat: np.ndarray, block) -> np.ndarray:
    """The same definition as plain nested loops, fp64 [B] (tiny inputs only)."""
    K, C, F, H, W = lat.shape
    nB = block_grid(F, H, W, block)
    B = nB[0] * nB[1] * nB[2]
    tot = [0.0] * B
    cnt = [0] * B
    bF, bH, bW = block

    def x(k, c, f, h, w):
        return float(lat[k, c, f, h, w])

    for f in range(F):
        for h in range(H):
            for w in range(W):
                b = ((f // bF) * nB[1] + h // bH) * nB[2] + w // bW
                for (df, dh, dw) in ((1, 0, 0), (0, 1, 0), (0, 0, 1)):
                    f2, h2, w2 = f + df, h + dh, w + dw
                    if f2 >= F or h2 >= H or w2 >= W:
                        continue
                    for c in range(C):
                        for k in range(1, K - 1):
                            g_next = x(k + 1, c, f2, h2, w2) - x(k + 1, c, f, h, w)
                            g_cur = x(k, c, f2, h2, w2) - x(k, c, f, h, w)
                            g_prev = x(k - 1, c, f2, h2, w2) - x(k - 1, c, f, h, w)
                            tot[b] += abs(g_next - 2.0 * g_cur + g_prev)
                            cnt[b] += 1
    return np.array([t / n if n else 0.0 for t, n in zip(tot, cnt)], dtype=np.float64)


# --------------------------------------------------------------------------
# FFT complexity baseline: an alternative index source, not the method.
# Jano pages: [fr] §2.A (frequency measures such as the FFT, which the
# analyzer replaces because they are unreliable on noisy early latents);
# [zh] §2.1 (the comparison: an FFT computed directly on the early latents);
# [pt] results (the baseline's recognition accuracy beside the analyzer's).
# The pages give no formula. Reading taken: per block and channel, the energy
# of the block's 3D DFT outside the DC term, over the latest warm-up latent
# L[K-1], divided by n^2 (n = the block's pixels inside the latent), averaged
# over the channels.
# --------------------------------------------------------------------------

def fft_block_scores_f64(lat: np.ndarray, block) -> np.ndarray:
    """FFT-baseline score per block, fp64 [B]. lat: fp32 [K, C, F, H, W]."""
    K, C, F, H, W = lat.shape
    L = np.asarray(lat[K - 1], dtype=np.float64)          # [C, F, H, W]
    bF, bH, bW = block
    nB = block_grid(F, H, W, block)
    out = np.zeros(nB[0] * nB[1] * nB[2], dtype=np.float64)
    b = 0
    for bf in range(nB[0]):
        for bh in range(nB[1]):
            for bw in range(nB[2]):
                x = L[:, bf * bF:(bf + 1) * bF, bh * bH:(bh + 1) * bH, bw * bW:(bw + 1) * bW]
                n = x[0].size
                X = np.fft.fftn(x, axes=(1, 2, 3))
                energy = (np.abs(X) ** 2).reshape(C, -1)
                out[b] = energy[:, 1:].sum(axis=1).mean() / float(n) ** 2   # [:, 0] is DC
                b += 1
    return out


def fft_block_scores(lat: np.ndarray, block) -> np.ndarray:
    """fft_block_scores_f64 rounded to fp32 [B]."""
    return fft_block_scores_f64(lat, block).astype(np.float32)


# --------------------------------------------------------------------------
# Levels. Jano pages: [nl] methodology §1 (three convergence levels:
# Static, Moderate, Active); [zh] §2.2 item 1; [ko] §2.B.
# --------------------------------------------------------------------------

def level_split(B: int, static_permille: int, moderate_permille: int) -> tuple:
    """(nS, nSM): blocks of rank < nS are Static, rank < nSM Moderate."""
    nS = (static_permille * B + 500) // 1000
    nSM = ((static_permille + moderate_permille) * B + 500) // 1000
    return nS, nSM


def assign_levels(scores: np.ndarray, static_permille: int = 400,
                  moderate_permille: int = 300) -> np.ndarray:
    scores = np.asarray(scores, dtype=np.float32)
    B = scores.shape[0]
    order = np.lexsort((np.arange(B), scores))    # by score, then block id
    rank = np.empty(B, dtype=np.int64)
    rank[order] = np.arange(B)
    nS, nSM = level_split(B, static_permille, moderate_permille)
    lv = np.full(B, ACTIVE, dtype=np.uint8)
    lv[rank < nSM] = MODERATE
    lv[rank < nS] = STATIC
    return lv


def token_block_ids(latent_fhw, patch, block) -> np.ndarray:
    """Block id of every token in token-major order n = (f*Ht + h)*Wt + w.
    Token (f, h, w) starts at latent pixel (f*pF, h*pH, w*pW)."""
    F, H, W = latent_fhw
    pF, pH, pW = patch
    bF, bH, bW = block
    nB = block_grid(F, H, W, block)
    Ft, Ht, Wt = F // pF, H // pH, W // pW
    bf = (np.arange(Ft) * pF) // bF
    bh = (np.arange(Ht) * pH) // bH
    bw = (np.arange(Wt) * pW) // bW
    ids = (bf[:, None, None] * nB[1] + bh[None, :, None]) * nB[2] + bw[None, None, :]
    return ids.ravel()


def token_levels(levels: np.ndarray, latent_fhw, patch, block) -> np.ndarray:
    return np.asarray(levels, dtype=np.uint8)[token_block_ids(latent_fhw, patch, block)]


def level_token_counts(levels, latent_fhw, patch, block) -> np.ndarray:
    tl = token_levels(levels, latent_fhw, patch, block)
    return np.array([(tl == v).sum() for v in (STATIC, MODERATE, ACTIVE)], dtype=np.int64)


# --------------------------------------------------------------------------
# Schedule. Jano pages: [nl] methodology §2 (warm-up, interleaved generation
# with per-level update frequency, cool-down); [zh] §2.2 item 2; [pt] §2.B.
# --------------------------------------------------------------------------

def is_dense_step(step: int, T: int, W: int, Cd: int) -> bool:
    return step < W or step >= T - Cd


def active_mask(tok_levels: np.ndarray, step: int, T: int, W: int, Cd: int,
                periods=(4, 2, 1)) -> np.ndarray:
    tl = np.asarray(tok_levels)
    if is_dense_step(step, T, W, Cd):
        return np.ones(tl.shape[0], dtype=bool)
    due = np.zeros(tl.shape[0], dtype=bool)
    for lv, p in zip((STATIC, MODERATE, ACTIVE), periods):
        if (step - W) % p == 0:
            due |= tl == lv
    return due


def schedule(tok_levels, step, T, W, Cd, periods=(4, 2, 1)) -> np.ndarray:
    """Ascending int32 indices of the tokens computed at this step."""
    return np.flatnonzero(active_mask(tok_levels, step, T, W, Cd, periods)).astype(np.int32)


def schedule_frozen(tok_levels, step, T, W, Cd, periods=(4, 2, 1)) -> np.ndarray:
    """Ascending int32 indices of the tokens NOT computed at this step (their
    keys/values come from the cache)."""
    return np.flatnonzero(~active_mask(tok_levels, step, T, W, Cd, periods)).astype(np.int32)


# --------------------------------------------------------------------------
# Token activation and the full-sequence KV cache. Jano pages: [nl]
# methodology §2 (KV cache of frozen tokens; cached pairs combined with the
# active queries without restoring positions, correct because attention does
# not depend on key/value order); [zh] §2.2 item 3; [fr] §2.B.
# --------------------------------------------------------------------------

def gather_rows(X: np.ndarray, idx: np.ndarray) -> np.ndarray:
    return np.asarray(X)[np.asarray(idx, dtype=np.int64)]


def scatter_rows(cache: np.ndarray, idx: np.ndarray, rows: np.ndarray) -> np.ndarray:
    out = np.array(cache, copy=True)
    out[np.asarray(idx, dtype=np.int64)] = rows
    return out


def concat_kv(Knew_bits, Kc_bits, frozen_idx) -> np.ndarray:
    """The pages' layout of one interleaved step: the fresh rows of the active
    tokens first, then the cached rows of the frozen tokens, positions not
    restored ([nl] methodology §2; [fr] §2.B; [ko] KV-cache item)."""
    return np.concatenate([np.asarray(Knew_bits), np.asarray(Kc_bits)[np.asarray(frozen_idx, np.int64)]])


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) exactly."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float | None = None,
              dtype=np.float64, q_chunk: int = 2048) -> np.ndarray:
    """Non-causal softmax attention per head.

    Q [n, H, d], K and V [N, H, d] (float). Returns [n, H, d] in `dtype`.
    out[i, h] = sum_j softmax_j(Q[i,h] . K[j,h] * scale) V[j,h]; each query row
    is independent, so rows are evaluated in chunks to bound memory."""
    n, Hh, d = Q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    Q = np.asarray(Q, dtype=dtype)
    K = np.asarray(K, dtype=dtype)
    V = np.asarray(V, dtype=dtype)
    out = np.empty((n, Hh, d), dtype=dtype)
    for h in range(Hh):
        Kh = np.ascontiguousarray(K[:, h, :])
        Vh = np.ascontiguousarray(V[:, h, :])
        for i0 in range(0, n, q_chunk):
            S = (Q[i0:i0 + q_chunk, h, :] @ Kh.T) * dtype(scale)
            S -= S.max(axis=1, keepdims=True)
            P = np.exp(S)
            out[i0:i0 + q_chunk, h, :] = (P @ Vh) / P.sum(axis=1, keepdims=True)
    return out


def attention_bruteforce(Q, K, V, scale=None) -> np.ndarray:
    """Scalar-loop fp64 attention for tiny inputs (no max shift needed there)."""
    n, Hh, d = Q.shape
    N = K.shape[0]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((n, Hh, d))
    for h in range(Hh):
        for i in range(n):
            logits = [sum(float(Q[i, h, e]) * float(K[j, h, e]) for e in range(d)) * scale
                      for j in range(N)]
            m = max(logits)
            wts = [np.exp(t - m) for t in logits]
            z = sum(wts)
            for e in range(d):
                out[i, h, e] = sum(wts[j] * float(V[j, h, e]) for j in range(N)) / z
    return out


def attn_step(Q_act_bits, Knew_bits, Vnew_bits, idx, Kc_bits, Vc_bits, scale=None,
              dtype=np.float64, queries=None):
    """One interleaved attention step on bf16 bit-pattern inputs.

    Writes the fresh K/V rows of the active tokens into the caches, then runs
    the active queries against the whole cache. Returns (out, Kc', Vc') with
    out in `dtype`; `queries` optionally restricts which active rows are
    evaluated (sampled checks at large sizes)."""
    Kc2 = scatter_rows(Kc_bits, idx, Knew_bits)
    Vc2 = scatter_rows(Vc_bits, idx, Vnew_bits)
    Q = bf16_to_f64(Q_act_bits)
    if queries is not None:
        Q = Q[np.asarray(queries)]
    out = attention(Q, bf16_to_f64(Kc2), bf16_to_f64(Vc2), scale, dtype=dtype)
    return out, Kc2, Vc2


# --------------------------------------------------------------------------
# Write-back of the active tokens' model output and the sampler step.
# Jano pages: [nl] "three groups" (the static group rests and its result is
# remembered); [zh] three classes (static regions skip intermediate steps and
# use the cache instead); [ko] §2 (skipped parts keep using the previous state
# held in memory). Reading taken: every token keeps its latest model output in
# a full-sequence buffer; active tokens overwrite theirs, frozen tokens reuse
# theirs, and every token takes the sampler step with that output.
# --------------------------------------------------------------------------

def f32_round_once(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """fp32 value nearest to the exact sum a + b (ties to even), for fp64
    arrays a and b whose exact sum fits fp64's exponent range.

    The fp64 sum s = fl(a + b) can itself be rounded, and rounding s again to
    fp32 may then land on the other side of an fp32 midpoint. So the exact
    error e = (a + b) - s is recovered with Knuth's TwoSum, and an inexact s
    is moved to its odd neighbour on the side of the exact sum (rounding to
    odd); rounding a round-to-odd value with p >= 24 + 2 bits to fp32 gives
    the correctly rounded fp32 result (Boldo and Melquiond, "When double
    rounding is odd", 2005)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    s = a + b
    bv = s - a
    e = (a - (s - bv)) + (b - bv)                 # exact: a + b = s + e
    even = (s.view(np.int64) & 1) == 0
    fix = (e != 0) & even
    toward = np.where(e > 0, np.inf, -np.inf)
    s = np.where(fix, np.nextafter(s, toward), s)
    return s.astype(np.float32)


def writeback_step(out_act_bits, idx, out_full_bits, x, dt):
    """Returns (out_full', x').

    out_act_bits [n_act, P] bf16 bits: the fresh model output of the active
    tokens idx; out_full_bits [N, P] bf16 bits: every token's latest output;
    x [N, P] fp32 sampler state (token-major latent patches). The active rows
    of out_full are replaced, then x' = x + dt * out_full' elementwise (one
    Euler step) rounded once to fp32: the bf16 x fp32 product has at most
    8 + 24 significant bits and is exact in fp64, and the sum with x is
    rounded to fp32 exactly once (f32_round_once)."""
    of = scatter_rows(out_full_bits, idx, out_act_bits)
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    prod = np.float64(np.float32(dt)) * bf16_to_f64(of)
    return of, f32_round_once(x64, prod)


# --------------------------------------------------------------------------
# Projection of the active tokens' hidden states to Q, K, V with a 3D rotary
# position encoding. The pages place only the active tokens' computation in
# the interleaved step ([nl] methodology §2; [zh] §2.2 item 3) and cache keys
# without restoring positions ([fr] §2.B), so the cached keys already carry
# their position encoding. The projection itself and the encoding are model
# details the pages do not give; reading taken: y = W x with W [3*H*d, Dm]
# (rows Q, then K, then V; head-major, then dim), and a rotary encoding of Q
# and K over the token's (frame, row, column): the head dim splits into three
# even parts d_f = d - 4*floor(d/6), d_h = d_w = 2*floor(d/6); pair i of a
# part of size m rotates dims (2i, 2i+1) of that part by pos * base**(-2i/m).
# --------------------------------------------------------------------------

def rope_parts(d: int) -> tuple:
    dh = 2 * (d // 6)
    return d - 2 * dh, dh, dh


def rope_apply(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """x [n, H, d] (float), pos [n, 3] integer (frame, row, column)."""
    x = np.asarray(x, dtype=np.float64)
    n, Hh, d = x.shape
    out = np.empty_like(x)
    j0 = 0
    for axis, m in enumerate(rope_parts(d)):
        for i in range(m // 2):
            ang = pos[:, axis].astype(np.float64) * base ** (-2.0 * i / m)
            c, s = np.cos(ang)[:, None], np.sin(ang)[:, None]
            a, b = x[:, :, j0 + 2 * i], x[:, :, j0 + 2 * i + 1]
            out[:, :, j0 + 2 * i] = a * c - b * s
            out[:, :, j0 + 2 * i + 1] = a * s + b * c
        j0 += m
    return out


def token_positions(idx: np.ndarray, token_grid) -> np.ndarray:
    """(frame, row, column) of token-major indices n = (f * Ht + h) * Wt + w."""
    Ft, Ht, Wt = token_grid
    idx = np.asarray(idx, dtype=np.int64)
    return np.stack([idx // (Ht * Wt), (idx // Wt) % Ht, idx % Wt], axis=1)


def qkv_proj(X_bits, idx, W_bits, H: int, d: int, token_grid=None, base: float = 10000.0):
    """Q, K, V [n_act, H, d] in fp64 for the active tokens idx.

    X_bits [N, Dm] bf16 hidden states, W_bits [3*H*d, Dm] bf16 weights.
    Y = X[idx] W^T exactly in fp64; Q and K are rotated when token_grid is
    given (base > 0), V never."""
    Xa = bf16_to_f64(np.asarray(X_bits)[np.asarray(idx, dtype=np.int64)])
    Y = Xa @ bf16_to_f64(W_bits).T
    n = Y.shape[0]
    Q, K, V = (Y[:, p * H * d:(p + 1) * H * d].reshape(n, H, d) for p in range(3))
    if token_grid is not None and base > 0:
        pos = token_positions(idx, token_grid)
        Q, K = rope_apply(Q, pos, base), rope_apply(K, pos, base)
    return Q, K, V
