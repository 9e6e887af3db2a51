"""The 50-step interleaved run on the 480p grid (32760 tokens, 12 heads,
d = 128), end to end through the C ABI, against the oracle replaying the same
steps.

The fresh Q/K/V of step s are bf16(cos(0.05 s) base + sin(0.05 s) dir) from
seeded fp32 base and direction tensors (each element stays N(0, 1)), so the
rows a step leaves in the caches really differ from the current ones. The GPU runs the analyzer once (its levels must match
the oracle's), then per step: schedule -> scatter of the fresh K/V rows into
the caches + attention of the active queries (the fresh rows are built on the
host for the active tokens, as a projection would produce them). Checked at
every step: the index list (bit-exact), both caches (bit-exact against the
oracle's scatter) and attention on a seeded sample of active queries (fp32
oracle); at the first interleaved step where only the Active tokens are due,
every active query is checked.
"""
import numpy as np
import pytest

from oracle import jano_oracle as O
from token_sparse_attention_block_amd import configs, jano, synth

from gpu_helpers import assert_attn_close, dev, dev_bf16, host_bf16_f64, host_bits, threshold_band

pytestmark = pytest.mark.gpu

FULL_CHECK_STEPS = (6,)     # (s - W) odd: only Active tokens are due
SAMPLE = 96                 # sampled active queries per step (all heads)


def test_interleaved_run_480p():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    jano.lib()  # fail loudly if the library is missing
    cfg = configs.SCHED480
    sc = cfg.schedule
    spec = jano.GridSpec.of(cfg)
    fhw = (cfg.F, cfg.H, cfg.W)
    N, H, d = cfg.N, cfg.heads, cfg.d

    # levels from the GPU analyzer, checked against the oracle's
    lat = synth.latents(cfg)
    scores_ref = O.analyze_scores(lat, cfg.block)
    lv_ref = O.assign_levels(scores_ref)
    _, lv_dev, _ = jano.analyze(dev(lat), spec)
    torch.cuda.synchronize()
    lv = lv_dev.cpu().numpy()
    band = threshold_band(scores_ref, 400, 300)
    np.testing.assert_array_equal(lv[~band], lv_ref[~band])
    tl = O.token_levels(lv, fhw, cfg.patch, cfg.block)

    base, dirs = synth.drift_qkv_f32(cfg)
    Kc_ref = np.zeros((N, H, d), np.uint16)
    Vc_ref = np.zeros((N, H, d), np.uint16)
    Kc_f32 = np.zeros((N, H, d), np.float32)    # fp32 values of the oracle caches
    Vc_f32 = np.zeros((N, H, d), np.float32)
    Kc = torch.zeros((N, H, d), dtype=torch.bfloat16, device="cuda")
    Vc = torch.zeros_like(Kc)
    idx_dev = torch.empty(N, dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(5)
    # the per-step fresh rows of synth.step_qkv_bits, with torch's threaded
    # CPU ops (the same fp32 multiplies and add, bf16 rounding to nearest even)
    base_t = [torch.from_numpy(b) for b in base]
    dirs_t = [torch.from_numpy(dr) for dr in dirs]

    def fresh(i, rows, s):
        c, sn = synth.step_coeffs(s)
        x = c * base_t[i][rows] + sn * dirs_t[i][rows]
        return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)

    probe = np.arange(0, N, 97)
    ref_probe = synth.step_qkv_bits([b[probe] for b in base], [dr[probe] for dr in dirs], 23)
    for i in range(3):
        np.testing.assert_array_equal(fresh(i, torch.from_numpy(probe), 23), ref_probe[i])
    n_full = 0
    for s in range(sc.T):
        ref_idx = O.schedule(tl, s, sc.T, sc.W, sc.Cd, sc.periods)
        n = len(ref_idx)
        rows_t = torch.from_numpy(ref_idx.astype(np.int64))
        Qa, Kn, Vn = (fresh(i, rows_t, s) for i in range(3))

        idx, n_dev = jano.schedule(lv_dev, spec, s, sc.T, sc.W, sc.Cd, sc.periods, idx=idx_dev)
        out = jano.attn_step(dev_bf16(Qa), dev_bf16(Kn), dev_bf16(Vn), idx, Kc, Vc, n_act=n)
        torch.cuda.synchronize()

        assert int(n_dev.item()) == n, s
        np.testing.assert_array_equal(idx[:n].cpu().numpy(), ref_idx)
        Kc_ref = O.scatter_rows(Kc_ref, ref_idx, Kn)
        Vc_ref = O.scatter_rows(Vc_ref, ref_idx, Vn)
        np.testing.assert_array_equal(host_bits(Kc), Kc_ref)
        np.testing.assert_array_equal(host_bits(Vc), Vc_ref)
        Kc_f32[ref_idx] = synth.bf16_bits_to_f32(Kn)
        Vc_f32[ref_idx] = synth.bf16_bits_to_f32(Vn)

        if s in FULL_CHECK_STEPS:
            rows = np.arange(n)
            n_full += 1
        else:
            rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, size=min(n, SAMPLE),
                                                                     replace=False)]))
        ref = O.attention(synth.bf16_bits_to_f32(Qa[rows]), Kc_f32, Vc_f32, dtype=np.float32)
        got = host_bf16_f64(out)[rows]
        assert_attn_close(got, ref.astype(np.float64), "step %d n_act=%d rows=%d" % (s, n, len(rows)))
    assert n_full == len(FULL_CHECK_STEPS)
