"""jano_analyze_noalloc (the analyzer with the library's fixed scratch array
instead of a caller workspace) against jano_analyze, bit for bit, on two calls
in a row whose second input is smaller than the first."""
import numpy as np
import pytest

from token_sparse_attention_block_amd import configs, jano, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    jano.lib()
    return t


def _outputs(torch, spec):
    B, _ = jano.grid_sizes(spec)
    return (torch.full((B,), -1.0, dtype=torch.float32, device="cuda"),
            torch.zeros(B, dtype=torch.uint8, device="cuda"),
            torch.full((3,), -1, dtype=torch.int32, device="cuda"))


def test_noalloc_matches_workspace_entry_point(torch):
    runs = []
    # 720p grid first (645 KB of partial sums), then the smaller image grid
    for cfg, signal, mix in ((configs.V720, True, (450, 300)), (configs.IMAGE, False, (400, 300))):
        print("noalloc", cfg.name, signal, mix, flush=True)
        spec = jano.GridSpec.of(cfg)
        assert jano.analyze_workspace_bytes(spec) <= jano.NOALLOC_SCRATCH_BYTES
        lat = torch.from_numpy(synth.latents(cfg, signal=signal)).cuda()
        out = _outputs(torch, spec)
        jano.analyze_noalloc(lat, spec, *out, static_permille=mix[0], moderate_permille=mix[1])
        torch.cuda.synchronize()
        runs.append((lat, spec, mix, [t.cpu().numpy() for t in out]))
    for lat, spec, mix, got in runs:
        ref = jano.analyze(lat, spec, mix[0], mix[1])
        torch.cuda.synchronize()
        for g, r, name in zip(got, ref, ("scores", "levels", "counts")):
            np.testing.assert_array_equal(g, r.cpu().numpy(), err_msg=name)
        assert int(got[2].sum()) == spec.F // spec.patch[0] * (spec.H // spec.patch[1]) * (spec.W // spec.patch[2])


def test_noalloc_repeated_calls_are_identical(torch):
    cfg = configs.V480
    spec = jano.GridSpec.of(cfg)
    lat = torch.from_numpy(synth.latents(cfg, signal=True)).cuda()
    a = _outputs(torch, spec)
    b = _outputs(torch, spec)
    jano.analyze_noalloc(lat, spec, *a)
    jano.analyze_noalloc(lat, spec, *b)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x.cpu().numpy(), y.cpu().numpy())
