"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Every kernel is fed the oracle's own inputs (e.g. the oracle's levels for the
schedule, the oracle's index list for attention) so a mismatch is pinned to
one kernel. Sizes span several tiles with ragged tails; the 720p cases run at
the full size the bench times and are checked on sampled outputs.
"""
import numpy as np
import pytest

from oracle import jano_oracle as O
from token_sparse_attention_block_amd import configs, jano, synth

from gpu_helpers import (SCORE_RTOL, assert_attn_close, dev, dev_bf16, host_bf16_f64, host_bits,
                         threshold_band)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    jano.lib()  # fail loudly if the library is missing
    return t


def _idx_for(cfg, frac):
    """Oracle index list of an Active-only interleaved step on a seeded map."""
    lv = synth.active_level_map(cfg, frac)
    tl = O.token_levels(lv, (cfg.F, cfg.H, cfg.W), cfg.patch, cfg.block)
    sc = cfg.schedule
    return O.schedule(tl, sc.W + 1, sc.T, sc.W, sc.Cd, sc.periods)


# ------------------------------------------------------------- gather/scatter

@pytest.mark.parametrize("cfg", [configs.TINY, configs.IMAGE, configs.V720], ids=lambda c: c.name)
def test_gather_rows_bit_exact(torch, cfg):
    frac = cfg.active_fracs[0] if cfg.active_fracs else 0.25
    print("gather", cfg.name, flush=True)
    (Qb,) = synth.qkv_bits(cfg, which="q")
    idx = _idx_for(cfg, 0.25 if cfg is configs.V720 else frac)
    X = dev_bf16(Qb)
    out = jano.gather_rows(X, dev(idx))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_bits(out), O.gather_rows(Qb, idx))


def test_gather_scalar_path_and_edges(torch):
    rng = np.random.default_rng(3)
    X = rng.integers(0, 65535, size=(37, 7), dtype=np.uint16)   # 14-byte rows -> scalar path
    Xd = dev_bf16(X)
    for idx in (np.array([36], np.int32), np.array([0, 5, 6, 36], np.int32),
                np.arange(37, dtype=np.int32)):
        out = jano.gather_rows(Xd, dev(idx))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host_bits(out), X[idx])
    empty = jano.gather_rows(Xd, dev(np.zeros(0, np.int32)))
    assert empty.shape[0] == 0


@pytest.mark.parametrize("cfg,frac", [(configs.TINY, 0.3), (configs.IMAGE, 0.3),
                                      (configs.V720, 0.25), (configs.V720, 1.0)],
                         ids=["tiny", "image", "720p-25", "720p-100"])
def test_scatter_kv_bit_exact(torch, cfg, frac):
    print("scatter", cfg.name, frac, flush=True)
    Qb, Kb, Vb = synth.qkv_bits(cfg)
    idx = _idx_for(cfg, frac)
    rng = np.random.default_rng(5)
    Kn = rng.integers(0, 65535, size=(len(idx), cfg.heads, cfg.d), dtype=np.uint16)
    Vn = rng.integers(0, 65535, size=(len(idx), cfg.heads, cfg.d), dtype=np.uint16)
    Kc, Vc = dev_bf16(Kb), dev_bf16(Vb)
    jano.scatter_kv(dev_bf16(Kn), dev_bf16(Vn), dev(idx), Kc, Vc)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_bits(Kc), O.scatter_rows(Kb, idx, Kn))
    np.testing.assert_array_equal(host_bits(Vc), O.scatter_rows(Vb, idx, Vn))


def test_scatter_scalar_path(torch):
    rng = np.random.default_rng(6)
    K = rng.integers(0, 65535, size=(20, 3, 3), dtype=np.uint16)   # 18-byte rows
    V = rng.integers(0, 65535, size=(20, 3, 3), dtype=np.uint16)
    idx = np.array([1, 2, 19], np.int32)
    Kn = rng.integers(0, 65535, size=(3, 3, 3), dtype=np.uint16)
    Kc, Vc = dev_bf16(K), dev_bf16(V)
    jano.scatter_kv(dev_bf16(Kn), dev_bf16(Kn), dev(idx), Kc, Vc)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_bits(Kc), O.scatter_rows(K, idx, Kn))
    np.testing.assert_array_equal(host_bits(Vc), O.scatter_rows(V, idx, Kn))


# ------------------------------------------------------------------ analyzer

def _analyze_gpu(torch, lat, spec, spm=400, mpm=300):
    scores, levels, counts = jano.analyze(dev(lat), spec, spm, mpm)
    torch.cuda.synchronize()
    return scores.cpu().numpy(), levels.cpu().numpy(), counts.cpu().numpy()


def _check_analyzer(lat, spec, s_gpu, l_gpu, c_gpu, spm=400, mpm=300):
    ref64 = O.analyze_scores_f64(lat, spec.block)
    err = np.abs(s_gpu.astype(np.float64) - ref64)
    bad = err > SCORE_RTOL * np.abs(ref64)
    assert not bad.any(), ("scores", int(bad.sum()), float(err[bad].max()))
    ref32 = ref64.astype(np.float32)
    lv_ref = O.assign_levels(ref32, spm, mpm)
    band = threshold_band(ref32, spm, mpm)
    mism = (l_gpu != lv_ref) & ~band
    assert not mism.any(), ("levels", np.flatnonzero(mism)[:10])
    cnt = O.level_token_counts(l_gpu, (spec.F, spec.H, spec.W), spec.patch, spec.block)
    np.testing.assert_array_equal(c_gpu, cnt)
    return int(band.sum())


@pytest.mark.parametrize("cfg", [configs.TINY, configs.IMAGE, configs.V480, configs.V720],
                         ids=lambda c: c.name)
@pytest.mark.parametrize("signal", [False, True], ids=["literal", "signal"])
def test_analyzer_configs(torch, cfg, signal):
    print("analyze", cfg.name, signal, flush=True)
    lat = synth.latents(cfg, signal=signal)
    spec = jano.GridSpec.of(cfg)
    s, l, c = _analyze_gpu(torch, lat, spec, cfg.static_permille, cfg.moderate_permille)
    nb = _check_analyzer(lat, spec, s, l, c, cfg.static_permille, cfg.moderate_permille)
    print("  blocks in threshold band:", nb, flush=True)


@pytest.mark.parametrize("shape,block,patch", [
    ((5, 3, 4, 24, 40), (2, 8, 8), (1, 2, 2)),     # bF=2: frame pairs, F chunks
    ((6, 2, 3, 18, 36), (1, 6, 12), (1, 2, 2)),    # R=2 strips (G=3), 12-lane segments
    ((4, 2, 5, 30, 70), (1, 4, 4), (1, 1, 1)),     # several W chunks, ragged tail
    ((3, 1, 1, 16, 16), (1, 4, 4), (1, 1, 1)),     # K=3, one frame
    ((9, 2, 2, 8, 8), (1, 4, 4), (1, 1, 1)),       # K=9 -> generic kernel
    ((5, 2, 2, 12, 140), (1, 4, 70), (1, 2, 2)),   # block wider than a wave -> generic
    ((5, 2, 3, 9, 10), (1, 3, 5), (1, 1, 1)),      # odd block height -> generic
    ((3, 2, 5, 20, 232), (1, 8, 16), (1, 2, 2)),   # 16-wide blocks, ragged last block column and row
    ((8, 3, 6, 12, 64), (3, 8, 32), (1, 1, 1)),    # K=8, 32-wide blocks, 3-frame blocks
    ((4, 2, 7, 13, 196), (1, 4, 4), (1, 1, 1)),    # one-row last block row, many W chunks
])
def test_analyzer_shapes(torch, shape, block, patch):
    print("analyze shape", shape, block, flush=True)
    rng = np.random.default_rng(sum(shape))
    lat = rng.standard_normal(shape).astype(np.float32)
    spec = jano.GridSpec(*shape, block=block, patch=patch)
    s, l, c = _analyze_gpu(torch, lat, spec)
    _check_analyzer(lat, spec, s, l, c)


@pytest.mark.parametrize("cfg", [configs.V720, configs.TINY], ids=lambda c: c.name)
def test_analyzer_unaligned_latents(torch, cfg):
    # latents that start 4 bytes past a 16-byte boundary (a view into a larger
    # buffer) score the same as aligned ones
    lat = synth.latents(cfg, signal=True)
    spec = jano.GridSpec.of(cfg)
    buf = torch.empty(lat.size + 1, dtype=torch.float32, device="cuda")
    view = buf[1:].view(lat.shape)
    view.copy_(torch.from_numpy(lat))
    assert view.data_ptr() % 16 == 4
    scores, levels, counts = jano.analyze(view, spec, cfg.static_permille, cfg.moderate_permille)
    torch.cuda.synchronize()
    _check_analyzer(lat, spec, scores.cpu().numpy(), levels.cpu().numpy(), counts.cpu().numpy(),
                    cfg.static_permille, cfg.moderate_permille)


def test_analyzer_closed_forms(torch, golden):
    # constant and step-affine latents score exactly zero
    spec = jano.GridSpec(5, 3, 2, 8, 8, (1, 4, 4), (1, 1, 1))
    s, l, c = _analyze_gpu(torch, np.full((5, 3, 2, 8, 8), 0.37, np.float32), spec)
    assert np.all(s == 0.0)
    assert l.tolist() == [1, 1, 1, 2, 2, 2, 3, 3]   # all ties -> by block id (nS=3, nSM=6)
    rng = np.random.default_rng(1)
    A = rng.integers(-1000, 1000, size=(3, 2, 8, 8)).astype(np.float64)
    Bf = rng.integers(-1000, 1000, size=(3, 2, 8, 8)).astype(np.float64)
    lat = np.stack([A + k * Bf for k in range(5)]).astype(np.float32)
    s, _, _ = _analyze_gpu(torch, lat, spec)
    assert np.all(s == 0.0)
    # hand-derived impulse scores
    g = golden("analyzer_impulse.json")
    lat = np.zeros(g["shape"], dtype=np.float32)
    i = g["impulse"]
    lat[i["k"], i["c"], i["f"], i["h"], i["w"]] = 1.0
    spec = jano.GridSpec(*g["shape"], block=tuple(g["block"]), patch=(1, 1, 1))
    s, _, _ = _analyze_gpu(torch, lat, spec)
    expect = np.zeros(g["num_blocks"], np.float32)
    for b, (num, den) in g["expected_scores"].items():
        expect[int(b)] = np.float32(num / den)
    np.testing.assert_array_equal(s, expect)


@pytest.mark.parametrize("cfg", [configs.TINY, configs.IMAGE, configs.V480, configs.V720],
                         ids=lambda c: c.name)
@pytest.mark.parametrize("signal", [False, True], ids=["literal", "signal"])
def test_fft_scores_configs(torch, cfg, signal):
    # the FFT-baseline index source: scores against the oracle's DFT energies,
    # then its levels through jano_levels, and one interleaved step's index list
    print("fft scores", cfg.name, signal, flush=True)
    lat = synth.latents(cfg, signal=signal)
    spec = jano.GridSpec.of(cfg)
    s = jano.fft_scores(dev(lat), spec)
    lv, cnt = jano.levels(s, spec, cfg.static_permille, cfg.moderate_permille)
    torch.cuda.synchronize()
    ref64 = O.fft_block_scores_f64(lat, spec.block)
    got = s.cpu().numpy().astype(np.float64)
    err = np.abs(got - ref64)
    bad = err > SCORE_RTOL * np.abs(ref64)
    assert not bad.any(), ("scores", int(bad.sum()), float(err[bad].max()))
    ref32 = ref64.astype(np.float32)
    lv_ref = O.assign_levels(ref32, cfg.static_permille, cfg.moderate_permille)
    band = threshold_band(ref32, cfg.static_permille, cfg.moderate_permille)
    l_gpu = lv.cpu().numpy()
    assert not ((l_gpu != lv_ref) & ~band).any()
    fhw = (spec.F, spec.H, spec.W)
    np.testing.assert_array_equal(cnt.cpu().numpy(), O.level_token_counts(l_gpu, fhw, spec.patch, spec.block))
    sc = cfg.schedule
    step = sc.W + 1
    idx, n_dev = jano.schedule(lv, spec, step, sc.T, sc.W, sc.Cd, sc.periods)
    torch.cuda.synchronize()
    ref_idx = O.schedule(O.token_levels(l_gpu, fhw, spec.patch, spec.block), step, sc.T, sc.W, sc.Cd,
                         sc.periods)
    n = int(n_dev.item())
    assert n == len(ref_idx)
    np.testing.assert_array_equal(idx[:n].cpu().numpy(), ref_idx)
    print("  blocks in threshold band:", int(band.sum()), " n_act at step", step, ":", n, flush=True)


@pytest.mark.parametrize("shape,block", [
    ((3, 2, 3, 10, 13), (2, 4, 5)),        # ragged edges along every axis
    ((4, 3, 1, 9, 9), (1, 4, 4)),
    ((3, 5, 2, 8, 2100), (1, 8, 1)),       # 2100 block columns: two column passes
    ((3, 1, 1, 4, 4), (1, 4, 4)),          # one block
    ((3, 2, 2, 9, 20), (1, 4, 8)),         # 16-byte loads, ragged last block column and row
    ((3, 1, 3, 700, 2), (3, 700, 1)),      # 2100 rows per block, two blocks
    ((3, 2, 3, 700, 8), (3, 700, 4)),      # the same with 16-byte loads and two channels
])
def test_fft_scores_shapes(torch, shape, block):
    print("fft scores shape", shape, block, flush=True)
    rng = np.random.default_rng(sum(shape))
    lat = (2.0 * rng.standard_normal(shape) + 3.0).astype(np.float32)
    spec = jano.GridSpec(*shape, block=block, patch=(1, 1, 1))
    s = jano.fft_scores(dev(lat), spec)
    torch.cuda.synchronize()
    ref64 = O.fft_block_scores_f64(lat, block)
    np.testing.assert_allclose(s.cpu().numpy().astype(np.float64), ref64, rtol=SCORE_RTOL, atol=0)


@pytest.mark.parametrize("spm,mpm", [(0, 0), (1000, 0), (0, 1000), (400, 600), (333, 333)])
def test_analyzer_level_mixes(torch, spm, mpm):
    cfg = configs.TINY
    lat = synth.latents(cfg, signal=True)
    spec = jano.GridSpec.of(cfg)
    s, l, c = _analyze_gpu(torch, lat, spec, spm, mpm)
    _check_analyzer(lat, spec, s, l, c, spm, mpm)


@pytest.mark.parametrize("cfg", [configs.TINY, configs.IMAGE, configs.V480, configs.V720],
                         ids=lambda c: c.name)
def test_levels_from_oracle_scores(torch, cfg):
    # jano_levels on the oracle's own fp32 scores: levels and counts bit-exact
    print("levels", cfg.name, flush=True)
    spec = jano.GridSpec.of(cfg)
    lat = synth.latents(cfg, signal=True)
    ref32 = O.analyze_scores(lat, spec.block)
    lv, cnt = jano.levels(dev(ref32), spec, cfg.static_permille, cfg.moderate_permille)
    torch.cuda.synchronize()
    lv_ref = O.assign_levels(ref32, cfg.static_permille, cfg.moderate_permille)
    np.testing.assert_array_equal(lv.cpu().numpy(), lv_ref)
    np.testing.assert_array_equal(
        cnt.cpu().numpy(), O.level_token_counts(lv_ref, (spec.F, spec.H, spec.W), spec.patch, spec.block))


@pytest.mark.parametrize("B_side,nvals", [(4, 3), (37, 5), (128, 1), (128, 1000), (128, 1 << 20)])
def test_levels_ties_and_max_size(torch, B_side, nvals):
    # scores with many ties (ordered by block id), one value only, and the
    # largest block count (128 x 128 = 16384 blocks)
    print("levels ties", B_side, nvals, flush=True)
    spec = jano.GridSpec(3, 1, 1, 4 * B_side, 4 * B_side, (1, 4, 4), (1, 1, 1))
    B = B_side * B_side
    rng = np.random.default_rng(B_side + nvals)
    sc = (rng.integers(0, nvals, B) * np.float32(0.125)).astype(np.float32)
    for spm, mpm in [(400, 300), (0, 1000), (1000, 0), (333, 333)]:
        lv, cnt = jano.levels(dev(sc), spec, spm, mpm)
        torch.cuda.synchronize()
        lv_ref = O.assign_levels(sc, spm, mpm)
        np.testing.assert_array_equal(lv.cpu().numpy(), lv_ref)
        np.testing.assert_array_equal(
            cnt.cpu().numpy(), O.level_token_counts(lv_ref, (spec.F, spec.H, spec.W), spec.patch, spec.block))


@pytest.mark.parametrize("cfg", [configs.TINY, configs.V720], ids=lambda c: c.name)
def test_random_masking_index_source(torch, cfg):
    # the pages' random-masking ablation as an index source: seeded random
    # block scores through jano_levels and jano_schedule, bit-exact
    spec = jano.GridSpec.of(cfg)
    sc = synth.random_block_scores(cfg)
    lv, cnt = jano.levels(dev(sc), spec, cfg.static_permille, cfg.moderate_permille)
    lv_ref = O.assign_levels(sc, cfg.static_permille, cfg.moderate_permille)
    np.testing.assert_array_equal(lv.cpu().numpy(), lv_ref)
    tl = O.token_levels(lv_ref, (cfg.F, cfg.H, cfg.W), cfg.patch, cfg.block)
    s_ = cfg.schedule
    for step in (s_.W, s_.W + 1, s_.W + 2):
        idx, n = jano.schedule(lv, spec, step, s_.T, s_.W, s_.Cd, s_.periods)
        torch.cuda.synchronize()
        ref = O.schedule(tl, step, s_.T, s_.W, s_.Cd, s_.periods)
        assert int(n.item()) == len(ref)
        np.testing.assert_array_equal(idx.cpu().numpy()[:len(ref)], ref)


def test_analyze_scores_entry_point(torch):
    # the scores-only call equals jano_analyze's scores, bit for bit, every call
    cfg = configs.V480
    spec = jano.GridSpec.of(cfg)
    lat = dev(synth.latents(cfg, signal=True))
    s_all, _, _ = jano.analyze(lat, spec)
    s1 = jano.analyze_scores(lat, spec)
    s2 = jano.analyze_scores(lat, spec)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(s1.cpu().numpy(), s_all.cpu().numpy())
    np.testing.assert_array_equal(s2.cpu().numpy(), s1.cpu().numpy())


# ------------------------------------------------------------------ write-back

def _wb_case(rng, N, P, n_act):
    x = rng.standard_normal((N, P)).astype(np.float32)
    full = synth.f32_to_bf16_bits(rng.standard_normal((N, P)).astype(np.float32))
    act = synth.f32_to_bf16_bits(rng.standard_normal((n_act, P)).astype(np.float32))
    idx = np.sort(rng.choice(N, size=n_act, replace=False)).astype(np.int32)
    return x, full, act, idx


def _wb_check(torch, x, full, act, idx, dt, x_off=0):
    N, P = full.shape
    ref_full, ref_x = O.writeback_step(act, idx, full, x, dt)
    of = dev_bf16(full)
    # x_off > 0 places x at an element offset, so the vector path is not aligned
    xbuf = torch.zeros(N * P + x_off, dtype=torch.float32, device="cuda")
    xd = xbuf[x_off:].view(N, P)
    xd.copy_(torch.from_numpy(x).cuda())
    jano.writeback_step(dev_bf16(act) if len(idx) else dev_bf16(np.zeros((1, P), np.uint16)),
                        dev(idx) if len(idx) else dev(np.zeros(1, np.int32)), of, xd, dt,
                        n_act=len(idx))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_bits(of), ref_full)
    np.testing.assert_array_equal(xd.cpu().numpy().view(np.uint32), ref_x.view(np.uint32))


@pytest.mark.parametrize("cfg,frac", [(configs.TINY, 0.3), (configs.IMAGE, 0.3), (configs.V720, 0.25)],
                         ids=lambda v: getattr(v, "name", str(v)))
def test_writeback_bit_exact(torch, cfg, frac):
    print("writeback", cfg.name, frac, flush=True)
    rng = np.random.default_rng(cfg.cfg_id)
    P = cfg.C * cfg.patch[0] * cfg.patch[1] * cfg.patch[2]
    idx = _idx_for(cfg, frac)
    x, full, act, _ = _wb_case(rng, cfg.N, P, len(idx))
    _wb_check(torch, x, full, act, idx, -0.02)


def test_writeback_edges(torch):
    rng = np.random.default_rng(11)
    x, full, act, idx = _wb_case(rng, 37, 5, 9)        # 185 elements: vector body + tail
    _wb_check(torch, x, full, act, idx, 0.125)
    _wb_check(torch, x, full, act, idx, 0.125, x_off=1)  # unaligned: scalar path
    x, full, act, idx = _wb_case(rng, 16, 8, 0)         # nothing active: x still steps
    _wb_check(torch, x, full, act, idx, -1.0)
    x, full, act, idx = _wb_case(rng, 16, 8, 16)        # everything active
    _wb_check(torch, x, full, act, idx, 0.0)


def test_writeback_rounds_once(torch):
    # x + dt*v = 1 + 2^-23 + 2^-24 - 2^-54 just below an fp32 midpoint: the
    # correctly rounded step is 1 + 2^-23 (a sum formed in fp64 and then
    # rounded to fp32 would give 1 + 2^-22). Placed in the 16-byte vector body
    # and in the scalar tail, and through the unaligned path.
    print("writeback rounds once", flush=True)
    N, P = 37, 5
    rng = np.random.default_rng(29)
    x = rng.standard_normal((N, P)).astype(np.float32)
    full = synth.f32_to_bf16_bits(rng.standard_normal((N, P)).astype(np.float32))
    for (n, p) in ((0, 0), (3, 2), (N - 1, P - 1)):
        x[n, p] = np.float32(1.0 + 2.0 ** -23)
        full[n, p] = 0x3F9A
    act = full[[5, 9]].copy()
    idx = np.array([5, 9], np.int32)
    dt = np.float32(13944699 * 2.0 ** -48)
    _, ref_x = O.writeback_step(act, idx, full, x, dt)
    assert float(ref_x[0, 0]) == 1.0 + 2.0 ** -23 and float(ref_x[N - 1, P - 1]) == 1.0 + 2.0 ** -23
    _wb_check(torch, x, full, act, idx, dt)
    _wb_check(torch, x, full, act, idx, dt, x_off=1)


# ------------------------------------------------------------------ schedule

def test_schedule_all_steps_480p(torch):
    cfg = configs.SCHED480
    lat = synth.latents(cfg)
    lv = O.assign_levels(O.analyze_scores(lat, cfg.block))
    tl = O.token_levels(lv, (cfg.F, cfg.H, cfg.W), cfg.patch, cfg.block)
    counts = O.level_token_counts(lv, (cfg.F, cfg.H, cfg.W), cfg.patch, cfg.block)
    spec = jano.GridSpec.of(cfg)
    sc = cfg.schedule
    lvd = dev(lv)
    idx_d = torch.full((cfg.N,), -7, dtype=torch.int32, device="cuda")
    for s in range(sc.T):
        idx, n = jano.schedule(lvd, spec, s, sc.T, sc.W, sc.Cd, sc.periods, idx=idx_d)
        torch.cuda.synchronize()
        ref = O.schedule(tl, s, sc.T, sc.W, sc.Cd, sc.periods)
        n = int(n.item())
        assert n == len(ref) == jano.schedule_count(counts, sc.T, sc.W, sc.Cd, sc.periods, s)
        np.testing.assert_array_equal(idx.cpu().numpy()[:n], ref)
        # the complement list of the concatenated layout
        fidx, nf = jano.schedule(lvd, spec, s, sc.T, sc.W, sc.Cd, sc.periods, frozen=True)
        torch.cuda.synchronize()
        fref = O.schedule_frozen(tl, s, sc.T, sc.W, sc.Cd, sc.periods)
        nf = int(nf.item())
        assert nf == len(fref) == cfg.N - n
        np.testing.assert_array_equal(fidx.cpu().numpy()[:nf], fref)


@pytest.mark.parametrize("cfg", [configs.TINY, configs.IMAGE, configs.V720], ids=lambda c: c.name)
def test_schedule_random_levels(torch, cfg):
    rng = np.random.default_rng(cfg.cfg_id)
    lv = rng.integers(1, 4, size=cfg.B).astype(np.uint8)
    tl = O.token_levels(lv, (cfg.F, cfg.H, cfg.W), cfg.patch, cfg.block)
    spec = jano.GridSpec.of(cfg)
    for s, periods in ((6, (4, 2, 1)), (7, (4, 2, 1)), (9, (4, 2, 1)), (11, (3, 5, 2)), (0, (4, 2, 1))):
        idx, n = jano.schedule(dev(lv), spec, s, 50, 5, 5, periods)
        torch.cuda.synchronize()
        ref = O.schedule(tl, s, 50, 5, 5, periods)
        assert int(n.item()) == len(ref)
        np.testing.assert_array_equal(idx.cpu().numpy()[:len(ref)], ref)


@pytest.mark.parametrize("shape,block,patch", [
    ((5, 4, 6, 36, 44), (2, 8, 6), (1, 2, 2)),      # blocks of 2 frames, ragged H and W edges
    ((5, 2, 14, 42, 46), (4, 4, 4), (2, 2, 2)),     # 2x2x2 patches, 2 token frames per block, ragged
    ((5, 2, 3, 64, 704), (1, 8, 8), (1, 2, 2)),     # 33792 tokens: 33 chunks, last one partial
    ((5, 2, 1, 8, 8), (1, 4, 4), (1, 1, 1)),        # one chunk of 64 tokens
], ids=["bF2-ragged", "patch222", "33-chunks", "tiny"])
def test_schedule_grids(torch, shape, block, patch):
    """Index lists on grids whose blocks span several token frames, with
    ragged block edges and chunk counts that do not divide the tokens: every
    workgroup's start offset comes out of the closed form over the blocks
    before its chunk."""
    K, C, F, H, W = shape
    spec = jano.GridSpec(K, C, F, H, W, block, patch)
    B, N = jano.grid_sizes(spec)
    rng = np.random.default_rng(B + N)
    lv = rng.integers(1, 4, size=B).astype(np.uint8)
    tl = O.token_levels(lv, (F, H, W), patch, block)
    assert tl.shape[0] == N
    for s, periods in ((6, (4, 2, 1)), (7, (4, 2, 1)), (9, (4, 2, 1)), (2, (4, 2, 1)), (8, (3, 5, 2))):
        for frozen in (False, True):
            idx, n = jano.schedule(dev(lv), spec, s, 50, 5, 5, periods, frozen=frozen)
            torch.cuda.synchronize()
            ref = (O.schedule_frozen if frozen else O.schedule)(tl, s, 50, 5, 5, periods)
            assert int(n.item()) == len(ref), (s, frozen)
            np.testing.assert_array_equal(idx.cpu().numpy()[:len(ref)], ref)


def test_check_idx(torch):
    good = dev(np.array([0, 3, 9], np.int32))
    assert int(jano.check_idx(good, 10).item()) == 0
    for bad in ([0, 3, 3], [0, 10], [-1, 2], [5, 2]):
        assert int(jano.check_idx(dev(np.array(bad, np.int32)), 10).item()) == jano.JANO_E_RANGE


# ----------------------------------------------------------------- attention

_QKV_MEMO = {}


def _qkv(cfg, extra=0):
    """synth.qkv_bits, kept for the next test of the same workload (drawing
    the 720p tensors takes longer than the parity check itself)."""
    key = (cfg.name, extra)
    if key not in _QKV_MEMO:
        _QKV_MEMO.clear()
        _QKV_MEMO[key] = synth.qkv_bits(cfg, extra=extra)
    return _QKV_MEMO[key]


def _attn_case(torch, cfg, idx, sample=None, extra=0, q_mult=1.0, ws=False):
    Qb, Kb, Vb = _qkv(cfg, extra)
    if q_mult != 1.0:
        Qb = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(Qb) * np.float32(q_mult))
    rng = np.random.default_rng(11 + extra)
    # the cache holds stale rows where the active tokens are; attn_step
    # refreshes them from K_new / V_new = the current K / V rows
    Kst, Vst = Kb.copy(), Vb.copy()
    Kst[idx] = rng.integers(0, 65535, size=(len(idx), cfg.heads, cfg.d), dtype=np.uint16) & 0x3FFF
    Vst[idx] = rng.integers(0, 65535, size=(len(idx), cfg.heads, cfg.d), dtype=np.uint16) & 0x3FFF
    Kc, Vc = dev_bf16(Kst), dev_bf16(Vst)
    workspace = None
    if ws:
        # with a workspace, these shapes' launches split the keys
        assert jano.attention_plan_ws(len(idx), cfg.N, cfg.heads, cfg.d)[3] > 1
        workspace = jano.attention_workspace(len(idx), cfg.N, cfg.heads, cfg.d, "cuda")
    out = jano.attn_step(dev_bf16(Qb[idx]), dev_bf16(Kb[idx]), dev_bf16(Vb[idx]), dev(idx), Kc, Vc,
                         workspace=workspace)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_bits(Kc), Kb)
    np.testing.assert_array_equal(host_bits(Vc), Vb)
    got = host_bf16_f64(out)
    rows = np.arange(len(idx)) if sample is None else sample
    ref, _, _ = O.attn_step(Qb[idx], Kb[idx], Vb[idx], idx, Kst, Vst, queries=rows)
    return got[rows], ref


# rows checked at full size: the first and last query (first and last
# workgroup tile, ragged tail) and 512 seeded others, every head of each
SAMPLE_ROWS = 512


def _sample_rows(n, seed=17):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], rng.choice(n, size=min(n, SAMPLE_ROWS), replace=False)]))


@pytest.mark.parametrize("cfg,frac", [(configs.TINY, 0.3), (configs.IMAGE, 0.3), (configs.IMAGE, 1.0)],
                         ids=["tiny-30", "image-30", "image-100"])
def test_attention_full_compare(torch, cfg, frac):
    print("attention", cfg.name, frac, flush=True)
    idx = _idx_for(cfg, frac)
    got, ref = _attn_case(torch, cfg, idx)
    assert_attn_close(got, ref, "%s %.0f%%" % (cfg.name, 100 * frac))


@pytest.mark.parametrize("cfg,frac", [(configs.V480, 0.25), (configs.V720, 0.10), (configs.V720, 0.25),
                                      (configs.V720, 0.50)],
                         ids=["480p-25", "720p-10", "720p-25", "720p-50"])
def test_attention_full_size_sampled(torch, cfg, frac):
    # the interleaved steps the bench times (scatter + active-query attention)
    print("attention sampled", cfg.name, frac, flush=True)
    idx = _idx_for(cfg, frac)
    sample = _sample_rows(len(idx))
    got, ref = _attn_case(torch, cfg, idx, sample=sample)
    assert_attn_close(got, ref, "%s %.0f%% sampled" % (cfg.name, 100 * frac))


@pytest.mark.parametrize("cfg,frac,sampled", [(configs.IMAGE, 0.3, False), (configs.IMAGE, 1.0, False),
                                              (configs.V480, 0.25, True)],
                         ids=["image-30", "image-100", "480p-25-sampled"])
def test_attention_split_keys_configs(torch, cfg, frac, sampled):
    # the steps whose launches split the keys when given a workspace
    print("attention split", cfg.name, frac, flush=True)
    idx = _idx_for(cfg, frac)
    sample = _sample_rows(len(idx)) if sampled else None
    got, ref = _attn_case(torch, cfg, idx, sample=sample, ws=True)
    assert_attn_close(got, ref, "%s %.0f%% split" % (cfg.name, 100 * frac))


# Given a workspace, a launch may split each head's keys into S ranges
# (jano_attention_plan_ws): both query-tile forms with 2, 3 and 4 ranges,
# ragged query tails, and the ragged key tile always in the last range.
@pytest.mark.parametrize("n,N,H,plan", [
    (50, 200, 1, (0, 1, 0, 2)), (3000, 500, 6, (0, 12, 0, 3)), (50, 500, 1, (0, 1, 0, 4)),
    (3000, 200, 12, (8, 0, 0, 2)), (2000, 500, 12, (6, 0, 0, 3)), (3000, 500, 8, (8, 0, 0, 4))])
def test_attention_split_keys(torch, n, N, H, plan):
    print("attention split keys", n, N, H, flush=True)
    d = 128
    assert jano.attention_plan_ws(n, N, H, d) == plan
    rng = np.random.default_rng(n + 3 * N + H)
    Q = synth.f32_to_bf16_bits(rng.standard_normal((n, H, d)).astype(np.float32))
    K = synth.f32_to_bf16_bits(rng.standard_normal((N, H, d)).astype(np.float32))
    V = synth.f32_to_bf16_bits(rng.standard_normal((N, H, d)).astype(np.float32))
    ws = jano.attention_workspace(n, N, H, d, "cuda")
    assert ws.numel() == plan[3] * n * H * 130 * 4
    Qd, Kd, Vd = dev_bf16(Q), dev_bf16(K), dev_bf16(V)
    out = jano.attention(Qd, Kd, Vd, workspace=ws)
    again = jano.attention(Qd, Kd, Vd, workspace=ws)
    torch.cuda.synchronize()
    ref = O.attention(O.bf16_to_f64(Q), O.bf16_to_f64(K), O.bf16_to_f64(V))
    assert_attn_close(host_bf16_f64(out), ref, "split n=%d N=%d H=%d" % (n, N, H))
    np.testing.assert_array_equal(host_bits(again), host_bits(out))   # deterministic


@pytest.mark.parametrize("case", ["mid-tile", "ragged-tail", "double"])
def test_attention_split_keys_late_max(torch, case):
    # the late-max inputs below (N = 1000: 15 tiles + 40 keys) in four key
    # ranges of 4 tiles: the jumps land in ranges 1 and 3, so the ranges merge
    # with different maxima
    rng = np.random.default_rng(77)
    n, N, H, d = 100, 1000, 2, 128
    assert jano.attention_plan_ws(n, N, H, d)[3] == 4
    c = 1.4426950408889634 / np.sqrt(d)
    Q = 0.1 * rng.standard_normal((n, H, d)).astype(np.float32)
    K = 0.1 * rng.standard_normal((N, H, d)).astype(np.float32)
    V = rng.standard_normal((N, H, d)).astype(np.float32)
    Q[:, :, 0] = 4.0
    K[:, :, 0] = 0.0
    up = np.float32(8.5 / (4.0 * c))
    if case == "mid-tile":
        K[448:512, :, 0] = up
    elif case == "ragged-tail":
        K[960:1000, :, 0] = up
    else:
        K[500, :, 0] = 40.0
        K[990, :, 0] = 80.0
    Qb, Kb, Vb = (synth.f32_to_bf16_bits(x) for x in (Q, K, V))
    ws = jano.attention_workspace(n, N, H, d, "cuda")
    out = jano.attention(dev_bf16(Qb), dev_bf16(Kb), dev_bf16(Vb), workspace=ws)
    torch.cuda.synchronize()
    ref = O.attention(O.bf16_to_f64(Qb), O.bf16_to_f64(Kb), O.bf16_to_f64(Vb))
    assert_attn_close(host_bf16_f64(out), ref, "split late max %s" % case)


@pytest.mark.parametrize("cfg", [configs.V480, configs.V720], ids=["480p-dense", "720p-dense"])
def test_dense_full_size_sampled(torch, cfg):
    # the dense reference step (every token a query), the denominator of the
    # step speedups and of the 50-step run's total
    print("attention dense sampled", cfg.name, flush=True)
    Qb, Kb, Vb = _qkv(cfg)
    out = jano.attention(dev_bf16(Qb), dev_bf16(Kb), dev_bf16(Vb))
    torch.cuda.synchronize()
    rows = _sample_rows(cfg.N, seed=19)
    got = host_bf16_f64(out)[rows]
    del out
    ref = O.attention(O.bf16_to_f64(Qb[rows]), O.bf16_to_f64(Kb), O.bf16_to_f64(Vb))
    assert_attn_close(got, ref, "%s dense sampled" % cfg.name)


def test_full_activation_equals_dense(torch):
    cfg = configs.IMAGE
    Qb, Kb, Vb = synth.qkv_bits(cfg)
    Q, K, V = dev_bf16(Qb), dev_bf16(Kb), dev_bf16(Vb)
    dense = jano.attention(Q, K, V)
    idx = np.arange(cfg.N, dtype=np.int32)
    Kc, Vc = torch.zeros_like(K), torch.zeros_like(V)
    step = jano.attn_step(Q, K, V, dev(idx), Kc, Vc)
    torch.cuda.synchronize()
    # same kernel, same inputs after the scatter: identical bits
    np.testing.assert_array_equal(host_bits(step), host_bits(dense))


def test_cached_equals_recompute(torch):
    # frozen rows current in the cache, active rows refreshed -> the active
    # queries' outputs equal dense attention's rows
    cfg = configs.IMAGE
    Qb, Kb, Vb = synth.qkv_bits(cfg)
    idx = _idx_for(cfg, 0.3)
    dense = host_bits(jano.attention(dev_bf16(Qb), dev_bf16(Kb), dev_bf16(Vb)))
    Kst, Vst = Kb.copy(), Vb.copy()
    Kst[idx] = 0
    Vst[idx] = 0
    Kc, Vc = dev_bf16(Kst), dev_bf16(Vst)
    step = jano.attn_step(dev_bf16(Qb[idx]), dev_bf16(Kb[idx]), dev_bf16(Vb[idx]), dev(idx), Kc, Vc)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_bits(step), dense[idx])


# d = 128 cases cover a cache shorter than one 64-key tile (1, 63), whole
# tiles only (64, 128), one extra key (65, 129, 4097) and a mid-tile tail
# (1000); query counts straddle the 384-query workgroup tile.
# d = 128 launches cover each head with 384-query tiles, 256-query tiles, or
# full 384-query tiles followed by 256-query ones (jano_attention_plan); the
# cases below run each form with ragged query and key tails: 256 only for
# launches that fit one round of the GPU (H = 3), 384 only where those take
# fewer rounds (H = 256), and the mixed form (H = 96 and 128).
@pytest.mark.parametrize("n,N,d,H,tiles", [
    (1, 1, 64, 3, (0, 0, 1)), (31, 100, 64, 3, (0, 0, 1)), (64, 129, 64, 3, (0, 0, 1)),
    (129, 65, 128, 3, (0, 1, 0)), (200, 1000, 128, 3, (0, 1, 0)), (257, 4097, 128, 3, (0, 2, 0)),
    (5, 1, 128, 3, (0, 1, 0)), (48, 63, 128, 3, (0, 1, 0)), (100, 64, 128, 3, (0, 1, 0)),
    (384, 128, 128, 3, (0, 2, 0)), (385, 129, 128, 3, (0, 2, 0)), (300, 1000, 128, 256, (1, 0, 0)),
    (384, 128, 128, 256, (1, 0, 0)), (257, 65, 128, 256, (1, 0, 0)), (300, 1, 128, 256, (1, 0, 0)),
    (1151, 300, 128, 128, (2, 2, 0)), (1299, 1000, 128, 96, (2, 3, 0)), (1151, 64, 128, 128, (2, 2, 0))])
def test_attention_ragged(torch, n, N, d, H, tiles):
    print("attention ragged", n, N, d, H, flush=True)
    assert jano.attention_plan(n, H, d) == tiles
    rng = np.random.default_rng(n * 7 + N)
    Q = synth.f32_to_bf16_bits(rng.standard_normal((n, H, d)).astype(np.float32))
    K = synth.f32_to_bf16_bits(rng.standard_normal((N, H, d)).astype(np.float32))
    V = synth.f32_to_bf16_bits(rng.standard_normal((N, H, d)).astype(np.float32))
    out = jano.attention(dev_bf16(Q), dev_bf16(K), dev_bf16(V))
    torch.cuda.synchronize()
    ref = O.attention(O.bf16_to_f64(Q), O.bf16_to_f64(K), O.bf16_to_f64(V))
    assert_attn_close(host_bf16_f64(out), ref, "ragged n=%d N=%d d=%d" % (n, N, d))


def test_empty_step_is_a_no_op(torch):
    # a step with no due token: attention of zero queries and a scatter of
    # zero rows write nothing and leave both caches as they were
    rng = np.random.default_rng(3)
    N, H = 300, 2
    for d in (64, 128):
        Kb = synth.f32_to_bf16_bits(rng.standard_normal((N, H, d)).astype(np.float32))
        Vb = synth.f32_to_bf16_bits(rng.standard_normal((N, H, d)).astype(np.float32))
        Kc, Vc = dev_bf16(Kb), dev_bf16(Vb)
        empty = torch.empty((0, H, d), dtype=torch.bfloat16, device="cuda")
        idx = torch.empty(0, dtype=torch.int32, device="cuda")
        out = jano.attn_step(empty, empty, empty, idx, Kc, Vc)
        out2 = jano.attention(empty, Kc, Vc)
        torch.cuda.synchronize()
        assert out.shape[0] == 0 and out2.shape[0] == 0
        np.testing.assert_array_equal(host_bits(Kc), Kb)
        np.testing.assert_array_equal(host_bits(Vc), Vb)


def test_attention_peaked_and_scale(torch):
    # large logits exercise the running-max rescale; an explicit scale is used
    cfg = configs.IMAGE
    idx = _idx_for(cfg, 0.3)
    got, ref = _attn_case(torch, cfg, idx, q_mult=8.0, extra=1)
    assert_attn_close(got, ref, "peaked")
    rng = np.random.default_rng(2)
    Q = synth.f32_to_bf16_bits(rng.standard_normal((70, 2, 64)).astype(np.float32))
    K = synth.f32_to_bf16_bits(rng.standard_normal((300, 2, 64)).astype(np.float32))
    V = synth.f32_to_bf16_bits(rng.standard_normal((300, 2, 64)).astype(np.float32))
    out = jano.attention(dev_bf16(Q), dev_bf16(K), dev_bf16(V), scale=0.3)
    torch.cuda.synchronize()
    ref = O.attention(O.bf16_to_f64(Q), O.bf16_to_f64(K), O.bf16_to_f64(V), scale=0.3)
    assert_attn_close(host_bf16_f64(out), ref, "scale=0.3")


@pytest.mark.parametrize("case", ["mid-tile", "ragged-tail", "double"])
@pytest.mark.parametrize("d,H,n,tiles", [(128, 2, 100, (0, 1, 0)), (128, 256, 300, (1, 0, 0)),
                                         (128, 128, 1151, (2, 2, 0)), (64, 2, 100, (0, 0, 1))])
def test_attention_late_max_jumps(torch, d, H, n, tiles, case):
    """The running max jumps past the rescale slack (2^8) after many tiles,
    with N = 1000 = 15 tiles of 64 + a ragged tile of 40. Every query shares
    a component of 4 that meets chosen keys with a large value; the other
    components are small, so the jump is the same for every query.
      mid-tile:    keys 448..511 (one whole tile) 8.5 log2 units up;
      ragged-tail: keys 960..999 (the ragged tile) 8.5 log2 units up;
      double:      key 500 up by ~20 and key 990 by ~40.
    In the first two the keys before the jump keep a few percent of the
    softmax weight, so a wrong rescale of what was accumulated before it
    shows in the output."""
    rng = np.random.default_rng(31 + d)
    N = 1000
    assert jano.attention_plan(n, H, d) == tiles
    c = 1.4426950408889634 / np.sqrt(d)          # log2 units per unit of q . k
    Q = 0.1 * rng.standard_normal((n, H, d)).astype(np.float32)
    K = 0.1 * rng.standard_normal((N, H, d)).astype(np.float32)
    V = rng.standard_normal((N, H, d)).astype(np.float32)
    Q[:, :, 0] = 4.0
    K[:, :, 0] = 0.0
    up = np.float32(8.5 / (4.0 * c))
    if case == "mid-tile":
        K[448:512, :, 0] = up
    elif case == "ragged-tail":
        K[960:1000, :, 0] = up
    else:
        K[500, :, 0] = 40.0
        K[990, :, 0] = 80.0
    Qb, Kb, Vb = (synth.f32_to_bf16_bits(x) for x in (Q, K, V))
    out = jano.attention(dev_bf16(Qb), dev_bf16(Kb), dev_bf16(Vb))
    torch.cuda.synchronize()
    ref = O.attention(O.bf16_to_f64(Qb), O.bf16_to_f64(Kb), O.bf16_to_f64(Vb))
    assert_attn_close(host_bf16_f64(out), ref, "late max jump %s d=%d H=%d" % (case, d, H))


def test_attention_closed_forms(torch):
    rng = np.random.default_rng(4)
    n, N, H, d = 40, 300, 2, 128
    V = synth.f32_to_bf16_bits(rng.standard_normal((N, H, d)).astype(np.float32))
    K = synth.f32_to_bf16_bits(rng.standard_normal((N, H, d)).astype(np.float32))
    Qz = np.zeros((n, H, d), np.uint16)
    out = host_bf16_f64(jano.attention(dev_bf16(Qz), dev_bf16(K), dev_bf16(V)))
    mean = O.bf16_to_f64(V).mean(axis=0)
    assert np.abs(out - mean[None]).max() <= 2e-2 * max(1.0, np.abs(mean).max())
    one = host_bf16_f64(jano.attention(dev_bf16(Qz), dev_bf16(K[:1]), dev_bf16(V[:1])))
    np.testing.assert_array_equal(one, np.broadcast_to(O.bf16_to_f64(V[:1]), one.shape))


# ------------------------------------------------- concatenated K/V layout

def _concat_case(torch, cfg, frac):
    idx = _idx_for(cfg, frac)
    lv = synth.active_level_map(cfg, frac)
    tl = O.token_levels(lv, (cfg.F, cfg.H, cfg.W), cfg.patch, cfg.block)
    sc = cfg.schedule
    frozen = O.schedule_frozen(tl, sc.W + 1, sc.T, sc.W, sc.Cd, sc.periods)
    Qb, Kb, Vb = synth.qkv_bits(cfg)
    rng = np.random.default_rng(21)
    Kst, Vst = Kb.copy(), Vb.copy()       # stale rows where the active tokens are
    Kst[idx] = rng.integers(0, 65535, size=(len(idx), cfg.heads, cfg.d), dtype=np.uint16) & 0x3FFF
    Vst[idx] = rng.integers(0, 65535, size=(len(idx), cfg.heads, cfg.d), dtype=np.uint16) & 0x3FFF
    Kcat, Vcat = jano.concat_kv(dev_bf16(Kb[idx]), dev_bf16(Vb[idx]), dev_bf16(Kst), dev_bf16(Vst),
                                dev(frozen))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_bits(Kcat), O.concat_kv(Kb[idx], Kst, frozen))
    np.testing.assert_array_equal(host_bits(Vcat), O.concat_kv(Vb[idx], Vst, frozen))
    return idx, Qb, Kb, Vb, Kst, Vst, Kcat, Vcat


@pytest.mark.parametrize("cfg,frac", [(configs.TINY, 0.3), (configs.IMAGE, 0.3), (configs.V720, 0.25)],
                         ids=["tiny-30", "image-30", "720p-25"])
def test_concat_kv_bit_exact(torch, cfg, frac):
    print("concat", cfg.name, frac, flush=True)
    _concat_case(torch, cfg, frac)


def test_concat_attention_equals_scatter_path(torch):
    # the pages' layout and the scatter cache give the same attention output
    # (to the kernel's rounding; key order differs), both within tolerance of
    # the oracle
    cfg = configs.IMAGE
    idx, Qb, Kb, Vb, Kst, Vst, Kcat, Vcat = _concat_case(torch, cfg, 0.3)
    Qd = dev_bf16(Qb[idx])
    out_cat = jano.attention(Qd, Kcat, Vcat)
    Kc, Vc = dev_bf16(Kst), dev_bf16(Vst)
    out_sc = jano.attn_step(Qd, dev_bf16(Kb[idx]), dev_bf16(Vb[idx]), dev(idx), Kc, Vc)
    torch.cuda.synchronize()
    ref = O.attention(O.bf16_to_f64(Qb[idx]), O.bf16_to_f64(O.concat_kv(Kb[idx], Kst, np.setdiff1d(
        np.arange(cfg.N), idx))), O.bf16_to_f64(O.concat_kv(Vb[idx], Vst, np.setdiff1d(np.arange(cfg.N), idx))))
    assert_attn_close(host_bf16_f64(out_cat), ref, "concat layout")
    assert_attn_close(host_bf16_f64(out_sc), ref, "scatter layout")
    assert_attn_close(host_bf16_f64(out_cat), host_bf16_f64(out_sc), "concat vs scatter")


# ------------------------------------------------ gathered QKV projection

def _proj_close(got, ref, label):
    got = np.asarray(got, np.float64)
    tol = 2.0 ** -8 * np.abs(ref) + 1e-4 * np.max(np.abs(ref))
    bad = np.abs(got - ref) > tol
    assert not bad.any(), (label, int(bad.sum()), float(np.abs(got - ref)[bad].max()))


def _proj_run(torch, X_bits, idx, W_bits, H, d, spec, base):
    Xd = dev_bf16(X_bits)
    Q, K, V = jano.qkv_proj(Xd, dev(idx), dev_bf16(W_bits), H, d, spec, base)
    torch.cuda.synchronize()
    return [host_bf16_f64(t) for t in (Q, K, V)]


@pytest.mark.parametrize("rotate,Dm", [(False, 96), (True, 96), (True, 32), (False, 64), (True, 160)],
                         ids=["plain-k3", "rotary-k3", "rotary-k1", "plain-k2", "rotary-k5"])
def test_qkv_proj_small_ragged(torch, rotate, Dm):
    # 77 tokens (ragged token tile), 3*H*d = 384 columns (ragged column tile),
    # Dm / 32 k tiles (1, 2, 3 and 5 exercise the pipeline's start and tail)
    rng = np.random.default_rng(3 + Dm)
    spec = jano.GridSpec(3, 1, 3, 10, 10, (1, 5, 5), (1, 1, 1))     # token grid 3 x 10 x 10
    N, H, d = 300, 2, 64
    X = synth.f32_to_bf16_bits(rng.standard_normal((N, Dm)).astype(np.float32))
    W = synth.f32_to_bf16_bits((rng.standard_normal((3 * H * d, Dm)) / 8).astype(np.float32))
    idx = np.sort(rng.choice(N, 77, replace=False)).astype(np.int32)
    got = _proj_run(torch, X, idx, W, H, d, spec if rotate else None, 500.0)
    ref = O.qkv_proj(X, idx, W, H, d, (3, 10, 10) if rotate else None, 500.0)
    for name, g_, r_ in zip("QKV", got, ref):
        _proj_close(g_, r_, name)


def test_qkv_proj_full_size_sampled(torch):
    # 720p token grid, hidden size 5120 = 40 heads x 128, 25% active; rows of
    # X that are not active are never read, so only the active rows are set
    cfg = configs.V720
    spec = jano.GridSpec.of(cfg)
    H, d, Dm = cfg.heads, cfg.d, cfg.heads * cfg.d
    idx = _idx_for(cfg, 0.25)
    rng = np.random.default_rng(5)
    Xa = synth.f32_to_bf16_bits(rng.standard_normal((len(idx), Dm)).astype(np.float32))
    W = synth.f32_to_bf16_bits((rng.standard_normal((3 * H * d, Dm)) / 64).astype(np.float32))
    Xd = torch.zeros((cfg.N, Dm), dtype=torch.bfloat16, device="cuda")
    Xd[torch.from_numpy(idx.astype(np.int64)).cuda()] = dev_bf16(Xa)
    Q, K, V = jano.qkv_proj(Xd, dev(idx), dev_bf16(W), H, d, spec, 10000.0)
    torch.cuda.synchronize()
    sample = np.unique(np.concatenate([rng.choice(len(idx), 200, replace=False), [0, len(idx) - 1]]))
    Xs = np.zeros((cfg.N, Dm), np.uint16)
    Xs[idx[sample]] = Xa[sample]
    ref = O.qkv_proj(Xs, idx[sample], W, H, d, (cfg.F // cfg.patch[0], cfg.H // cfg.patch[1],
                                                cfg.W // cfg.patch[2]), 10000.0)
    for name, t, r_ in zip("QKV", (Q, K, V), ref):
        _proj_close(host_bf16_f64(t)[sample], r_, name)
