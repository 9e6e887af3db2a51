"""Pins of the CPU oracle against what the Jano pages and the mathematics fix.

Each test is chosen so that a plausible slip in the oracle (a dropped axis, a
first instead of a second step difference, a term booked to the wrong block,
an off-by-one in the level split, softmax over the wrong axis, a missing
scale, a scatter that touches other rows) fails at least one of them.
"""
import itertools

from fractions import Fraction

import numpy as np
import pytest

from oracle import jano_oracle as O
from token_sparse_attention_block_amd import configs, synth


# ---------------------------------------------------------------- analyzer --

def _int_latents(rng, K, C, F, H, W, lo=-100, hi=100):
    return rng.integers(lo, hi, size=(K, C, F, H, W)).astype(np.float32)


def test_constant_latents_score_zero():
    lat = np.full((5, 3, 2, 8, 8), 0.37, dtype=np.float32)
    s = O.analyze_scores(lat, (1, 4, 4))
    assert s.shape == (2 * 2 * 2,)
    assert np.all(s == 0.0)


def test_affine_in_step_scores_zero():
    # L_k = A + k*B with integer fields: exact in fp32, so D_k == 0 exactly,
    # whatever the spatial pattern.
    rng = np.random.default_rng(1)
    A = rng.integers(-1000, 1000, size=(4, 3, 9, 10)).astype(np.float64)
    Bf = rng.integers(-1000, 1000, size=(4, 3, 9, 10)).astype(np.float64)
    lat = np.stack([A + k * Bf for k in range(6)]).astype(np.float32)
    assert np.all(O.analyze_scores(lat, (1, 4, 4)) == 0.0)
    assert np.all(O.analyze_scores(lat, (2, 3, 5)) == 0.0)


def test_spatial_ramp_with_affine_slope_zero():
    # a spatially linear ramp whose slope changes linearly over the steps
    K, C, F, H, W = 5, 2, 3, 8, 8
    k = np.arange(K, dtype=np.float64)[:, None, None, None, None]
    f = np.arange(F)[None, None, :, None, None]
    h = np.arange(H)[None, None, None, :, None]
    w = np.arange(W)[None, None, None, None, :]
    lat = ((3 + 2 * k) * (f + 2 * h - 3 * w)).astype(np.float32)
    lat = np.broadcast_to(lat, (K, C, F, H, W)).copy()
    assert np.all(O.analyze_scores(lat, (1, 4, 4)) == 0.0)


def test_quadratic_in_step_linear_in_space_closed_form():
    # L_k = k^2 * (sF f + sH h + sW w): D_k = 2 (sF f + sH h + sW w), so the
    # term along axis a is 2|s_a| everywhere it is defined. A block's score is
    # 2 * sum_a n_a |s_a| / sum_a n_a with n_a its positions having a +a
    # neighbour (counted here by enumeration).
    K, C, F, H, W = 6, 3, 3, 10, 7
    block = (2, 4, 3)
    s = {0: 1, 1: -2, 2: 3}
    kk = np.arange(K, dtype=np.float64)[:, None, None, None, None] ** 2
    f = np.arange(F)[None, None, :, None, None]
    h = np.arange(H)[None, None, None, :, None]
    w = np.arange(W)[None, None, None, None, :]
    lat = np.broadcast_to(kk * (s[0] * f + s[1] * h + s[2] * w), (K, C, F, H, W)).astype(np.float32)
    nB = O.block_grid(F, H, W, block)
    B = nB[0] * nB[1] * nB[2]
    num = np.zeros(B)
    den = np.zeros(B)
    ext = (F, H, W)
    for p in itertools.product(range(F), range(H), range(W)):
        b = ((p[0] // block[0]) * nB[1] + p[1] // block[1]) * nB[2] + p[2] // block[2]
        for a in range(3):
            if p[a] + 1 < ext[a]:
                num[b] += 2 * abs(s[a])
                den[b] += 1
    expect = (num / den).astype(np.float32)
    np.testing.assert_array_equal(O.analyze_scores(lat, block), expect)


def test_impulse_golden(golden):
    g = golden("analyzer_impulse.json")
    lat = np.zeros(g["shape"], dtype=np.float32)
    i = g["impulse"]
    lat[i["k"], i["c"], i["f"], i["h"], i["w"]] = 1.0
    s = O.analyze_scores_f64(lat, tuple(g["block"]))
    expect = np.zeros(g["num_blocks"])
    for b, (num, den) in g["expected_scores"].items():
        expect[int(b)] = num / den
    np.testing.assert_allclose(s, expect, rtol=1e-15, atol=0)


def test_homogeneity_affine_shift_and_channel_permutation():
    rng = np.random.default_rng(7)
    lat = _int_latents(rng, 5, 4, 3, 12, 10)
    base = O.analyze_scores_f64(lat, (1, 4, 4))
    assert np.any(base > 0)
    np.testing.assert_array_equal(O.analyze_scores_f64(-2.0 * lat, (1, 4, 4)), 2.0 * base)
    A = rng.integers(-50, 50, size=lat.shape[1:]).astype(np.float32)
    Bf = rng.integers(-50, 50, size=lat.shape[1:]).astype(np.float32)
    shifted = lat + np.stack([A + k * Bf for k in range(5)])
    np.testing.assert_array_equal(O.analyze_scores_f64(shifted, (1, 4, 4)), base)
    perm = rng.permutation(4)
    np.testing.assert_array_equal(O.analyze_scores_f64(lat[:, perm], (1, 4, 4)), base)


@pytest.mark.parametrize("shape,block", [
    ((4, 2, 3, 6, 5), (1, 2, 2)),
    ((5, 3, 2, 7, 9), (2, 4, 3)),
    ((3, 1, 1, 5, 8), (1, 4, 4)),      # one frame: spatial terms only
    ((6, 2, 4, 1, 6), (3, 1, 4)),      # H == 1: no height term
])
def test_bruteforce_agrees(shape, block):
    rng = np.random.default_rng(11)
    lat = rng.standard_normal(shape).astype(np.float32)
    np.testing.assert_allclose(O.analyze_scores_f64(lat, block),
                               O.analyze_scores_bruteforce(lat, block), rtol=1e-12, atol=0)


def test_bruteforce_agrees_tiny_config():
    cfg = configs.TINY
    lat = synth.latents(cfg, signal=True)[:, :4]   # 4 channels keep the loops short
    np.testing.assert_allclose(O.analyze_scores_f64(lat, cfg.block),
                               O.analyze_scores_bruteforce(lat, cfg.block), rtol=1e-12, atol=0)


def test_signal_variant_ranks_textured_blocks_on_top():
    # The signal variant puts a quadratic-in-step term on the textured blocks;
    # their scores must dominate, and the top-30% must be exactly those blocks.
    cfg = configs.TINY
    lat = synth.latents(cfg, signal=True)
    s = O.analyze_scores(lat, cfg.block)
    tex = synth.texture_blocks(cfg).ravel()
    lv = O.assign_levels(s, 400, 300)
    assert set(np.flatnonzero(lv == 3)) == set(np.flatnonzero(tex))


# ----------------------------------------------- FFT complexity baseline --

def _block_variance_direct(lat, block):
    """Mean over channels of each block's population variance of the last
    latent, by plain loops (no DFT)."""
    K, C, F, H, W = lat.shape
    L = lat[K - 1].astype(np.float64)
    bF, bH, bW = block
    out = []
    for bf in range(-(-F // bF)):
        for bh in range(-(-H // bH)):
            for bw in range(-(-W // bW)):
                v = []
                for c in range(C):
                    x = L[c, bf * bF:(bf + 1) * bF, bh * bH:(bh + 1) * bH, bw * bW:(bw + 1) * bW].ravel()
                    m = sum(x) / len(x)
                    v.append(sum((xi - m) ** 2 for xi in x) / len(x))
                out.append(sum(v) / C)
    return np.array(out)


def test_fft_scores_equal_block_variance():
    # Parseval: the DFT energy outside the DC term over n^2 is the population
    # variance; ragged edge blocks use the pixels present
    rng = np.random.default_rng(7)
    for shape, block in [((3, 2, 3, 10, 13), (2, 4, 5)), ((4, 3, 1, 9, 9), (1, 4, 4)),
                         ((3, 1, 5, 6, 7), (3, 3, 3))]:
        lat = (3.0 * rng.standard_normal(shape) + 1.0).astype(np.float32)
        np.testing.assert_allclose(O.fft_block_scores_f64(lat, block),
                                   _block_variance_direct(lat, block), rtol=1e-12, atol=1e-14)


def test_fft_scores_closed_forms():
    h = np.arange(8.0)[:, None]
    w = np.arange(8.0)[None, :]
    lat = np.zeros((3, 3, 1, 8, 8))
    lat[2, 0, 0] = 3.0 * np.cos(2 * np.pi * (h / 8 + 2 * w / 8)) + 5.0   # variance 9/2, DC ignored
    lat[2, 1, 0] = 2.0 * np.cos(2 * np.pi * 3 * w / 8)                   # variance 4/2
    lat[2, 2, 0] = 0.5 * np.cos(np.pi * h)                               # Nyquist: variance 1/4
    lat[0] = 100.0                                                       # earlier latents ignored
    s = O.fft_block_scores_f64(lat.astype(np.float32), (1, 8, 8))
    assert s.shape == (1,)
    assert abs(s[0] - (4.5 + 2.0 + 0.25) / 3) <= 1e-6
    const = np.full((3, 2, 2, 8, 8), 0.37, dtype=np.float32)
    assert np.all(np.abs(O.fft_block_scores_f64(const, (1, 4, 4))) <= 1e-20)


def test_fft_scores_last_latent_scale_and_offset():
    rng = np.random.default_rng(11)
    lat = rng.standard_normal((4, 2, 2, 8, 12)).astype(np.float32)
    block = (1, 4, 4)
    base = O.fft_block_scores_f64(lat, block)
    other = lat.copy()
    other[:-1] = rng.standard_normal(other[:-1].shape)
    np.testing.assert_array_equal(O.fft_block_scores_f64(other, block), base)
    np.testing.assert_allclose(O.fft_block_scores_f64(lat * np.float32(4.0), block), 16.0 * base,
                               rtol=1e-12)
    shifted = lat.astype(np.float64)                                     # exact offsets
    offs = rng.integers(-8, 8, size=(2, 2, 2, 3)).astype(np.float64)     # one constant per block
    shifted[-1] += np.repeat(np.repeat(offs, 4, axis=2), 4, axis=3)
    np.testing.assert_allclose(O.fft_block_scores_f64(shifted, block), base, rtol=1e-9, atol=1e-12)


def test_fft_baseline_misses_textured_blocks_on_noisy_latents():
    # On the signal variant (textured blocks quadratic in the step) the
    # analyzer's Active set is exactly the textured blocks, while the FFT
    # baseline on the latest, still noise-dominated latent recovers only about
    # half of them -- the behaviour the pages' comparison describes.
    cfg = configs.IMAGE
    lat = synth.latents(cfg, signal=True)
    tex = set(np.flatnonzero(synth.texture_blocks(cfg).ravel()))
    act_an = set(np.flatnonzero(O.assign_levels(O.analyze_scores(lat, cfg.block)) == 3))
    act_fft = set(np.flatnonzero(O.assign_levels(O.fft_block_scores(lat, cfg.block)) == 3))
    assert act_an == tex
    assert len(act_fft & tex) < 0.75 * len(tex)


# ------------------------------------------------------------------ levels --

def test_level_split_counts():
    for B, expect in [(48, (19, 15, 14)), (256, (102, 77, 77)),
                      (2184, (874, 655, 655)), (5040, (2016, 1512, 1512))]:
        nS, nSM = O.level_split(B, 400, 300)
        assert (nS, nSM - nS, B - nSM) == expect
        rng = np.random.default_rng(B)
        lv = O.assign_levels(rng.random(B).astype(np.float32))
        assert tuple(np.bincount(lv, minlength=4)[1:]) == expect


def test_levels_golden(golden):
    g = golden("levels_and_schedule.json")["levels_case"]
    lv = O.assign_levels(np.array(g["scores"], dtype=np.float32),
                         g["static_permille"], g["moderate_permille"])
    assert lv.tolist() == g["expected_levels"]


def test_levels_monotone_and_ties_by_id():
    rng = np.random.default_rng(3)
    s = rng.integers(0, 5, size=200).astype(np.float32)   # many ties
    lv = O.assign_levels(s)
    for i in range(200):
        for j in range(200):
            if s[i] < s[j] or (s[i] == s[j] and i < j):
                assert lv[i] <= lv[j]
    flat = O.assign_levels(np.zeros(10, dtype=np.float32))
    assert flat.tolist() == [1, 1, 1, 1, 2, 2, 2, 3, 3, 3]


def test_token_block_map_matches_enumeration():
    # 720p-shaped grid: 90 latent rows / blocks of 8 -> ragged last block row
    F, H, W, patch, block = 2, 90, 24, (1, 2, 2), (1, 8, 8)
    ids = O.token_block_ids((F, H, W), patch, block)
    nB = O.block_grid(F, H, W, block)
    n = 0
    for f in range(F):
        for h in range(H // 2):
            for w in range(W // 2):
                # token (f,h,w) covers latent pixels [2h, 2h+2) x [2w, 2w+2)
                b = set()
                for hh in range(2 * h, 2 * h + 2):
                    for ww in range(2 * w, 2 * w + 2):
                        b.add((f * nB[1] + hh // 8) * nB[2] + ww // 8)
                assert len(b) == 1 and ids[n] == b.pop()
                n += 1
    counts = O.level_token_counts(np.array([1, 2, 3] * 40, dtype=np.uint8)[:nB[0] * nB[1] * nB[2]],
                                  (F, H, W), patch, block)
    assert counts.sum() == F * (H // 2) * (W // 2)


# ---------------------------------------------------------------- schedule --

@pytest.mark.parametrize("case", ["schedule_case", "schedule_case_short"])
def test_schedule_golden(golden, case):
    g = golden("levels_and_schedule.json")[case]
    tl = np.array(g["token_levels"], dtype=np.uint8)
    for s, expect in g["expected"].items():
        idx = O.schedule(tl, int(s), g["T"], g["W"], g["Cd"], tuple(g["periods"]))
        assert idx.tolist() == expect, s


def test_schedule_properties():
    cfg = configs.SCHED480
    rng = np.random.default_rng(5)
    lv = rng.integers(1, 4, size=cfg.B).astype(np.uint8)
    tl = O.token_levels(lv, (cfg.F, cfg.H, cfg.W), cfg.patch, cfg.block)
    cnt = O.level_token_counts(lv, (cfg.F, cfg.H, cfg.W), cfg.patch, cfg.block)
    sc = cfg.schedule
    for s in range(sc.T):
        idx = O.schedule(tl, s, sc.T, sc.W, sc.Cd, sc.periods)
        assert idx.dtype == np.int32
        assert np.all(np.diff(idx) > 0)
        if s < sc.W or s >= sc.T - sc.Cd:
            assert np.array_equal(idx, np.arange(cfg.N))
        else:
            due = [(s - sc.W) % p == 0 for p in sc.periods]
            assert len(idx) == sum(c for c, d in zip(cnt, due) if d)
            if s + 4 < sc.T - sc.Cd:
                assert np.array_equal(idx, O.schedule(tl, s + 4, sc.T, sc.W, sc.Cd, sc.periods))
    # mean active share over the interleaved phase with a 40/30/30 split is
    # 100/30/60/30% -> the 50-step total is 32 dense equivalents
    lv2 = O.assign_levels(rng.random(cfg.B).astype(np.float32))
    tl2 = O.token_levels(lv2, (cfg.F, cfg.H, cfg.W), cfg.patch, cfg.block)
    tot = sum(len(O.schedule(tl2, s, sc.T, sc.W, sc.Cd, sc.periods)) for s in range(sc.T))
    assert abs(tot / cfg.N - 32.0) < 0.5


# -------------------------------------------------------- gather / scatter --

def test_gather_scatter_rows():
    rng = np.random.default_rng(9)
    X = rng.integers(0, 65535, size=(50, 7), dtype=np.uint16)
    idx = np.array([0, 3, 4, 17, 49], dtype=np.int32)
    g = O.gather_rows(X, idx)
    for i, r in enumerate(idx):
        assert np.array_equal(g[i], X[r])
    new = rng.integers(0, 65535, size=(5, 7), dtype=np.uint16)
    c2 = O.scatter_rows(X, idx, new)
    for r in range(50):
        if r in idx:
            assert np.array_equal(c2[r], new[list(idx).index(r)])
        else:
            assert np.array_equal(c2[r], X[r])
    assert np.array_equal(X, O.gather_rows(X, np.arange(50)))  # input untouched


# --------------------------------------------------------------- attention --

def _bf(x):
    return synth.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_attention_bruteforce_tiny():
    rng = np.random.default_rng(2)
    Q = rng.standard_normal((5, 2, 8))
    K = rng.standard_normal((9, 2, 8))
    V = rng.standard_normal((9, 2, 8))
    np.testing.assert_allclose(O.attention(Q, K, V), O.attention_bruteforce(Q, K, V),
                               rtol=1e-12, atol=1e-13)


def test_attention_two_key_closed_form():
    d = 4
    q = np.array([[[1.0, 2.0, 0.0, -1.0]]])
    k = np.array([[[0.5, 0.0, 1.0, 0.0]], [[0.0, 1.0, 0.0, 1.0]]])
    v = np.array([[[1.0, 0.0, 0.0, 0.0]], [[0.0, 0.0, 3.0, 0.0]]])
    s1, s2 = 0.5 / np.sqrt(d), 1.0 / np.sqrt(d)
    w1 = np.exp(s1) / (np.exp(s1) + np.exp(s2))
    expect = w1 * v[0, 0] + (1 - w1) * v[1, 0]
    np.testing.assert_allclose(O.attention(q, k, v)[0, 0], expect, rtol=1e-14)
    # an explicit scale replaces 1/sqrt(d)
    w1b = np.exp(0.5 * 3) / (np.exp(0.5 * 3) + np.exp(1.0 * 3))
    np.testing.assert_allclose(O.attention(q, k, v, scale=3.0)[0, 0],
                               w1b * v[0, 0] + (1 - w1b) * v[1, 0], rtol=1e-14)


def test_attention_closed_forms():
    rng = np.random.default_rng(4)
    n, N, Hh, d = 6, 11, 3, 16
    V = rng.standard_normal((N, Hh, d))
    Q = rng.standard_normal((n, Hh, d))
    # all keys equal -> uniform weights -> mean of V
    Keq = np.broadcast_to(rng.standard_normal((1, Hh, d)), (N, Hh, d))
    np.testing.assert_allclose(O.attention(Q, Keq, V), np.broadcast_to(V.mean(0), (n, Hh, d)), rtol=1e-12)
    # Q = 0 -> mean of V
    K = rng.standard_normal((N, Hh, d))
    np.testing.assert_allclose(O.attention(np.zeros_like(Q), K, V),
                               np.broadcast_to(V.mean(0), (n, Hh, d)), rtol=1e-12)
    # one key -> that value
    np.testing.assert_allclose(O.attention(Q, K[:1], V[:1]), np.broadcast_to(V[0], (n, Hh, d)), rtol=1e-12)
    # a dominant logit -> that value row
    Kd = K.copy()
    Kd[7] = 50.0 * Q[2]
    out = O.attention(Q[2:3], Kd, V)
    np.testing.assert_allclose(out[0], V[7], atol=1e-9)


def test_full_activation_equals_dense():
    cfg = configs.TINY
    Qb, Kb, Vb = synth.qkv_bits(cfg)
    idx = np.arange(cfg.N, dtype=np.int32)
    stale = np.zeros_like(Kb)
    out, Kc, Vc = O.attn_step(Qb, Kb, Vb, idx, stale, stale)
    assert np.array_equal(Kc, Kb) and np.array_equal(Vc, Vb)
    dense = O.attention(O.bf16_to_f64(Qb), O.bf16_to_f64(Kb), O.bf16_to_f64(Vb))
    np.testing.assert_array_equal(out, dense)


def test_cached_equals_recompute_and_permutation_invariance():
    cfg = configs.TINY
    Qb, Kb, Vb = synth.qkv_bits(cfg)
    rng = np.random.default_rng(8)
    idx = np.sort(rng.choice(cfg.N, size=230, replace=False)).astype(np.int32)
    # frozen rows are current, active rows are stale in the cache
    Kst, Vst = Kb.copy(), Vb.copy()
    Kst[idx] = _bf(rng.standard_normal((230, cfg.heads, cfg.d)))
    Vst[idx] = _bf(rng.standard_normal((230, cfg.heads, cfg.d)))
    out, Kc, Vc = O.attn_step(Qb[idx], Kb[idx], Vb[idx], idx, Kst, Vst)
    dense = O.attention(O.bf16_to_f64(Qb), O.bf16_to_f64(Kb), O.bf16_to_f64(Vb))
    np.testing.assert_allclose(out, dense[idx], rtol=1e-12, atol=1e-14)
    # the pages' order: fresh K/V of the active tokens first, then the frozen
    # tokens' cached K/V, positions never restored
    frozen = np.setdiff1d(np.arange(cfg.N), idx)
    Kcat = np.concatenate([Kb[idx], Kst[frozen]])
    Vcat = np.concatenate([Vb[idx], Vst[frozen]])
    cat = O.attention(O.bf16_to_f64(Qb[idx]), O.bf16_to_f64(Kcat), O.bf16_to_f64(Vcat))
    np.testing.assert_allclose(cat, out, rtol=1e-12, atol=1e-14)
    perm = rng.permutation(cfg.N)
    outp = O.attention(O.bf16_to_f64(Qb[idx]), O.bf16_to_f64(Kc[perm]), O.bf16_to_f64(Vc[perm]))
    np.testing.assert_allclose(outp, out, rtol=1e-12, atol=1e-14)


def test_bf16_decode():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x7F80, 0x4049, 0x0001], dtype=np.uint16)
    v = O.bf16_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -1.0 and v[2] == 0.0 and np.isinf(v[3])
    assert v[4] == 3.140625
    assert v[5] == 2.0 ** -133


# ---------------------------------------------------------------- write-back

def _wb_inputs(N=12, P=5, seed=3):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((N, P)).astype(np.float32)
    full = rng.integers(0x3C00, 0x4100, size=(N, P), dtype=np.uint16)
    return rng, x, full


def test_writeback_closed_forms():
    # x = 1, out = 2 (bf16 0x4000), dt = 0.25 -> x' = 1.5 exactly; frozen rows
    # keep their cached output and step with it (out = -0.5, bf16 0xBF00)
    x = np.ones((3, 2), np.float32)
    full = np.full((3, 2), 0xBF00, np.uint16)
    act = np.full((1, 2), 0x4000, np.uint16)
    of, x2 = O.writeback_step(act, np.array([1]), full, x, 0.25)
    assert of[1].tolist() == [0x4000, 0x4000] and of[0].tolist() == [0xBF00, 0xBF00]
    assert x2[1].tolist() == [1.5, 1.5]
    assert x2[0].tolist() == [0.875, 0.875] and x2[2].tolist() == [0.875, 0.875]


def test_writeback_dt_zero_and_empty():
    rng, x, full = _wb_inputs()
    act = rng.integers(0, 0x7F00, size=(4, 5), dtype=np.uint16)
    idx = np.array([0, 3, 4, 11])
    of, x2 = O.writeback_step(act, idx, full, x, 0.0)
    np.testing.assert_array_equal(x2.view(np.uint32), x.view(np.uint32))
    np.testing.assert_array_equal(of[idx], act)
    keep = np.setdiff1d(np.arange(12), idx)
    np.testing.assert_array_equal(of[keep], full[keep])
    of, x3 = O.writeback_step(np.zeros((0, 5), np.uint16), np.zeros(0, np.int64), full, x, -0.1)
    np.testing.assert_array_equal(of, full)


def _rn32_exact(q: Fraction) -> np.float32:
    """fp32 nearest to the rational q, ties to the even significand: the
    candidates are the fp32 values around float(q), compared exactly."""
    c = np.float32(float(q))
    cands = {float(c), float(np.nextafter(c, np.float32(np.inf))),
             float(np.nextafter(c, np.float32(-np.inf)))}
    best = min(cands, key=lambda v: (abs(Fraction(v) - q),
                                     int(np.array(v, np.float32).view(np.uint32)) & 1))
    return np.float32(best)


def _bf16_fraction(bits) -> Fraction:
    return Fraction(float(np.array([int(bits) << 16], np.uint32).view(np.float32)[0]))


def test_writeback_rounds_once_counterexample():
    # x + dt*v = 1 + 2^-23 + 2^-24 - 2^-54: just below the fp32 midpoint
    # between 1 + 2^-23 and 1 + 2^-22, so the nearest fp32 is 1 + 2^-23. The
    # nearest fp64 of that sum is the midpoint itself, and a second rounding
    # of it to fp32 (ties to even) would give 1 + 2^-22.
    x = np.array([[1.0 + 2.0 ** -23]], np.float32)
    dt = np.float32(13944699 * 2.0 ** -48)
    exact = Fraction(float(x[0, 0])) + Fraction(float(dt)) * _bf16_fraction(0x3F9A)
    assert exact == 1 + Fraction(1, 2 ** 23) + Fraction(1, 2 ** 24) - Fraction(1, 2 ** 54)
    _, x2 = O.writeback_step(np.array([[0x3F9A]], np.uint16), np.array([0]),
                             np.zeros((1, 1), np.uint16), x, dt)
    assert float(x2[0, 0]) == 1.0 + 2.0 ** -23
    assert float(np.float32(float(exact))) == 1.0 + 2.0 ** -22   # the twice-rounded value


def test_f32_round_once_against_exact_rationals():
    # random sums and sums placed near fp32 midpoints, against the exact
    # rational sum rounded to the nearest fp32 value
    rng = np.random.default_rng(23)
    a = rng.standard_normal(400).astype(np.float32).astype(np.float64)
    b = (rng.standard_normal(400) * 2.0 ** rng.integers(-40, 2, 400)).astype(np.float32).astype(np.float64)
    # b = half an fp32 ulp of a, plus or minus a few 2^-35 ulp: a + b lies
    # within 2^-58 |a| of an fp32 midpoint, below fp64's own resolution there
    ulp = np.spacing(np.abs(a).astype(np.float32)).astype(np.float64) * np.sign(a)
    off = rng.integers(-3, 4, 400) * 2.0 ** -35
    b = np.concatenate([b, ulp * (0.5 + off)])
    a = np.concatenate([a, a])
    naive = (a + b).astype(np.float32)        # fp64 sum, then fp32: twice rounded
    assert (naive != O.f32_round_once(a, b)).sum() > 50
    got = O.f32_round_once(a, b)
    for i in range(a.size):
        want = _rn32_exact(Fraction(float(a[i])) + Fraction(float(b[i])))
        assert got[i].view(np.uint32) == want.view(np.uint32), i


def test_writeback_bruteforce_all_active():
    # every token active: scalar loops over exact rationals, rounded once
    rng, x, full = _wb_inputs(N=4, P=3, seed=9)
    act = rng.integers(0x3000, 0x4400, size=(4, 3), dtype=np.uint16)
    perm = np.array([2, 0, 3, 1])
    dt = np.float32(-0.0625)
    of, x2 = O.writeback_step(act, perm, full, x, dt)
    for i in range(4):
        for p in range(3):
            want = _rn32_exact(Fraction(float(x[perm[i], p])) + Fraction(float(dt)) * _bf16_fraction(act[i, p]))
            assert of[perm[i], p] == act[i, p]
            assert x2[perm[i], p] == want, (i, p)


def test_writeback_two_steps_compose():
    # stepping twice with the same active set = writing once, stepping twice
    rng, x, full = _wb_inputs(seed=5)
    act = rng.integers(0x3400, 0x4200, size=(5, 5), dtype=np.uint16)
    idx = np.array([1, 2, 6, 7, 9])
    of1, x1 = O.writeback_step(act, idx, full, x, 0.5)
    of2, x2 = O.writeback_step(act, idx, of1, x1, 0.5)
    np.testing.assert_array_equal(of2, of1)
    for n in range(x.shape[0]):
        for p in range(x.shape[1]):
            v = Fraction(1, 2) * _bf16_fraction(of1[n, p])
            once = _rn32_exact(Fraction(float(x[n, p])) + v)
            assert x1[n, p] == once
            assert x2[n, p] == _rn32_exact(Fraction(float(once)) + v)


# ------------------------------------------------------- concatenated layout

def test_schedule_frozen_is_the_complement():
    cfg = configs.TINY
    lv = synth.active_level_map(cfg, 0.3)
    tl = O.token_levels(lv, (cfg.F, cfg.H, cfg.W), cfg.patch, cfg.block)
    sc = cfg.schedule
    for step in range(sc.T):
        act = O.schedule(tl, step, sc.T, sc.W, sc.Cd, sc.periods)
        frz = O.schedule_frozen(tl, step, sc.T, sc.W, sc.Cd, sc.periods)
        assert len(np.intersect1d(act, frz)) == 0
        np.testing.assert_array_equal(np.union1d(act, frz), np.arange(cfg.N))
        assert np.all(np.diff(frz) > 0)
        if step < sc.W or step >= sc.T - sc.Cd:
            assert len(frz) == 0


def test_concat_layout_rows():
    # row i < n_act is the fresh row i; row n_act + j is the cached row frozen[j]
    rng = np.random.default_rng(4)
    Kc = rng.integers(0, 65535, size=(9, 3), dtype=np.uint16)
    Kn = rng.integers(0, 65535, size=(2, 3), dtype=np.uint16)
    frozen = np.array([0, 3, 4, 8])
    cat = O.concat_kv(Kn, Kc, frozen)
    assert cat.shape == (6, 3)
    for i in range(2):
        assert cat[i].tolist() == Kn[i].tolist()
    for j, r in enumerate(frozen):
        assert cat[2 + j].tolist() == Kc[r].tolist()


# ------------------------------------------------------- projection + RoPE

def test_rope_parts_and_identity_at_origin():
    assert O.rope_parts(128) == (44, 42, 42) and O.rope_parts(64) == (24, 20, 20)
    assert O.rope_parts(6) == (2, 2, 2)
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 2, 128))
    np.testing.assert_array_equal(O.rope_apply(x, np.zeros((3, 3), np.int64), 10000.0), x)


def test_rope_closed_form_d6():
    # d = 6: one pair per axis, frequency base**0 = 1, so the angle is the position
    x = np.array([[[1.0, 0.0, 1.0, 0.0, 0.0, 2.0]]])
    pos = np.array([[1, 2, 3]])
    y = O.rope_apply(x, pos, 10000.0)[0, 0]
    np.testing.assert_allclose(y[:2], [np.cos(1), np.sin(1)], atol=1e-15)
    np.testing.assert_allclose(y[2:4], [np.cos(2), np.sin(2)], atol=1e-15)
    np.testing.assert_allclose(y[4:], [-2 * np.sin(3), 2 * np.cos(3)], atol=1e-15)


def test_rope_relative_position_property():
    # <rope(q, p1), rope(k, p2)> depends only on p1 - p2, per axis, and pair
    # norms are kept
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 1, 64))
    k = rng.standard_normal((1, 1, 64))
    def dot(p1, p2):
        return float(np.sum(O.rope_apply(q, np.array([p1]), 500.0) * O.rope_apply(k, np.array([p2]), 500.0)))
    assert abs(dot([3, 5, 7], [1, 2, 4]) - dot([12, 9, 10], [10, 6, 7])) < 1e-9
    assert abs(dot([3, 5, 7], [1, 2, 4]) - dot([3, 5, 7], [1, 2, 5])) > 1e-6
    r = O.rope_apply(q, np.array([[4, 1, 9]]), 10000.0)
    np.testing.assert_allclose(r[0, 0, ::2] ** 2 + r[0, 0, 1::2] ** 2, q[0, 0, ::2] ** 2 + q[0, 0, 1::2] ** 2)


def test_token_positions():
    pos = O.token_positions(np.array([0, 1, 5, 6, 13]), (2, 2, 3))
    assert pos.tolist() == [[0, 0, 0], [0, 0, 1], [0, 1, 2], [1, 0, 0], [2, 0, 1]]


def test_qkv_proj_identity_weights_and_bruteforce():
    rng = np.random.default_rng(5)
    H, d, N = 2, 6, 7
    X = synth.f32_to_bf16_bits(rng.standard_normal((N, H * d)).astype(np.float32))
    eye = np.eye(H * d, dtype=np.float32)
    W = synth.f32_to_bf16_bits(np.concatenate([eye, 2 * eye, -eye]))
    idx = np.array([1, 4, 6])
    Q, K, V = O.qkv_proj(X, idx, W, H, d)
    xa = O.bf16_to_f64(X[idx]).reshape(3, H, d)
    np.testing.assert_array_equal(Q, xa)
    np.testing.assert_array_equal(K, 2 * xa)
    np.testing.assert_array_equal(V, -xa)
    # brute force with Python loops on random weights, with the rotation
    W = synth.f32_to_bf16_bits(rng.standard_normal((3 * H * d, H * d)).astype(np.float32))
    Q, K, V = O.qkv_proj(X, idx, W, H, d, token_grid=(1, 1, N), base=100.0)
    Wf, Xf = O.bf16_to_f64(W), O.bf16_to_f64(X)
    for a, n in enumerate(idx):
        y = [sum(Wf[o, e] * Xf[n, e] for e in range(H * d)) for o in range(3 * H * d)]
        v = np.array(y[2 * H * d:]).reshape(H, d)
        np.testing.assert_allclose(V[a], v, rtol=1e-12, atol=1e-12)
        q = np.array(y[:H * d]).reshape(1, H, d)
        pos = np.array([[0, 0, n]])
        np.testing.assert_allclose(Q[a], O.rope_apply(q, pos, 100.0)[0], rtol=1e-12, atol=1e-12)
        # the column axis is the last part (dims 4, 5 for d = 6): angle n * 1
        qq = q[0, :, 4:6]
        want = np.stack([qq[:, 0] * np.cos(n) - qq[:, 1] * np.sin(n), qq[:, 0] * np.sin(n) + qq[:, 1] * np.cos(n)], 1)
        np.testing.assert_allclose(Q[a][:, 4:6], want, rtol=1e-12, atol=1e-12)


def test_rope_second_pair_frequency():
    # d = 12: parts of 4; pair 1 of a part turns by pos * base**(-2/4), which
    # at base 100 and position 10 is exactly 1 radian (frame part, dims 2, 3)
    x = np.zeros((1, 1, 12))
    x[0, 0, 2] = 1.0
    y = O.rope_apply(x, np.array([[10, 0, 0]]), 100.0)[0, 0]
    np.testing.assert_allclose(y[2:4], [np.cos(1.0), np.sin(1.0)], atol=1e-14)
    # the row part starts at dim 4: its pair 0 turns by the row position
    x = np.zeros((1, 1, 12))
    x[0, 0, 4] = 1.0
    y = O.rope_apply(x, np.array([[10, 3, 0]]), 100.0)[0, 0]
    np.testing.assert_allclose(y[4:6], [np.cos(3.0), np.sin(3.0)], atol=1e-14)


# ------------------------------------------------- random-masking index source

def test_random_masking_levels_have_exact_shares():
    # ranking blocks by seeded random draws keeps the level shares exact and
    # makes the split independent of the latents (the pages' ablation)
    for cfg in (configs.TINY, configs.V480):
        sc = synth.random_block_scores(cfg)
        assert sc.dtype == np.float32 and np.all((sc >= 0) & (sc < 1))
        lv = O.assign_levels(sc, cfg.static_permille, cfg.moderate_permille)
        nS, nSM = O.level_split(cfg.B, cfg.static_permille, cfg.moderate_permille)
        assert (lv == 1).sum() == nS and (lv == 2).sum() == nSM - nS and (lv == 3).sum() == cfg.B - nSM
        order = np.argsort(sc, kind="stable")
        assert np.all(lv[order[:nS]] == 1) and np.all(lv[order[nSM:]] == 3)
        other = synth.random_block_scores(cfg, extra=1)
        assert not np.array_equal(O.assign_levels(other, cfg.static_permille, cfg.moderate_permille), lv)
