"""A whole interleaved run captured as one HIP graph.

The entry points allocate nothing, keep no state between calls and never
synchronise, so a run (analyzer once, then per step schedule -> gather ->
scatter + attention) can be captured once and replayed. Replays are checked
bit for bit against the same run done eagerly, several times in a row with
eager work and synchronisations between them (the caches are reset from a
snapshot by an eager copy before each replay).
"""
import numpy as np
import pytest

from token_sparse_attention_block_amd import configs, jano, synth

from gpu_helpers import host_bits

pytestmark = pytest.mark.gpu

T, W, CD, PERIODS = 12, 2, 2, (4, 2, 1)


def test_interleaved_run_replays_as_a_graph():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    jano.lib()  # fail loudly if the library is missing
    cfg = configs.IMAGE
    spec = jano.GridSpec.of(cfg)
    B, N = jano.grid_sizes(spec)
    H, d = cfg.heads, cfg.d
    dev = "cuda"

    lat = torch.from_numpy(synth.latents(cfg)).to(dev)
    scores = torch.empty(B, dtype=torch.float32, device=dev)
    levels = torch.empty(B, dtype=torch.uint8, device=dev)
    counts = torch.empty(3, dtype=torch.int32, device=dev)
    ws = torch.empty(jano.analyze_workspace_bytes(spec), dtype=torch.uint8, device=dev)
    jano.analyze(lat, spec, 400, 300, scores, levels, counts, workspace=ws)
    torch.cuda.synchronize()
    cnt = counts.cpu().tolist()
    n_per = [jano.schedule_count(cnt, T, W, CD, PERIODS, s) for s in range(T)]
    assert min(n_per) < N  # some steps are interleaved

    base, dirs = synth.drift_qkv_f32(cfg)

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    steps = [tuple(bf(x) for x in synth.step_qkv_bits(base, dirs, s)) for s in range(T)]
    idx = torch.empty(N, dtype=torch.int32, device=dev)
    n_dev = torch.empty(1, dtype=torch.int32, device=dev)
    q_act = torch.empty((N, H, d), dtype=torch.bfloat16, device=dev)
    k_new = torch.empty_like(q_act)
    v_new = torch.empty_like(q_act)
    outs = [torch.empty((n, H, d), dtype=torch.bfloat16, device=dev) for n in n_per]
    Kc0 = torch.zeros((N, H, d), dtype=torch.bfloat16, device=dev)
    Vc0 = torch.zeros_like(Kc0)
    Kc, Vc = Kc0.clone(), Vc0.clone()

    def run():
        jano.analyze(lat, spec, 400, 300, scores, levels, counts, workspace=ws)
        for s in range(T):
            n = n_per[s]
            Qs, Ks, Vs = steps[s]
            jano.schedule(levels, spec, s, T, W, CD, PERIODS, idx, n_dev)
            ii = idx[:n]
            jano.gather_rows(Qs, ii, n, out=q_act[:n])
            jano.gather_rows(Ks, ii, n, out=k_new[:n])
            jano.gather_rows(Vs, ii, n, out=v_new[:n])
            jano.attn_step(q_act[:n], k_new[:n], v_new[:n], ii, Kc, Vc, out=outs[s], n_act=n)

    run()
    torch.cuda.synchronize()
    ref_out = [host_bits(o) for o in outs]
    ref_k, ref_v = host_bits(Kc), host_bits(Vc)

    g = torch.cuda.CUDAGraph()
    Kc.copy_(Kc0)
    Vc.copy_(Vc0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        Kc.copy_(Kc0)
        Vc.copy_(Vc0)
        for o in outs:
            o.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for s in range(T):
            np.testing.assert_array_equal(host_bits(outs[s]), ref_out[s], err_msg="replay %d step %d" % (rep, s))
        np.testing.assert_array_equal(host_bits(Kc), ref_k)
        np.testing.assert_array_equal(host_bits(Vc), ref_v)
        # eager work between replays
        jano.attention(q_act[:64], Kc, Vc)
        torch.cuda.synchronize()
        print("graph replay", rep, "matches the eager run", flush=True)
