"""Host-side checks of the C ABI: the library loads, exports every function
include/jano.h declares, and rejects bad arguments before touching a GPU; the
calibration library exports what include/jano_calib.h declares and rejects
bad arguments. No kernel is launched here (runs on machines without a GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

from token_sparse_attention_block_amd import configs, jano

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "jano.h")

pytestmark = pytest.mark.skipif(not os.path.exists(jano.LIB_PATH),
                                reason="libjano.so not built (run __graft_entry__.build())")


def declared_functions(header=HEADER):
    src = open(header).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(jano_[a-z_0-9]+)\s*\(",
                                 src, flags=re.M)))


def test_header_declares_binding_exports():
    assert declared_functions() == sorted(jano.EXPORTS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", jano.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    syms = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for name in declared_functions():
        assert name in syms, name
    L = jano.lib()
    for name in declared_functions():
        assert hasattr(L, name)


def test_calib_library_exports_and_rejects():
    from token_sparse_attention_block_amd import build as B
    names = declared_functions(os.path.join(ROOT, "include", "jano_calib.h"))
    assert names == ["jano_calib_mfma_loop", "jano_calib_stream"]
    out = subprocess.run(["nm", "-D", "--defined-only", B.CALIB_LIB], capture_output=True,
                         text=True, check=True).stdout
    syms = {l.split()[-1] for l in out.splitlines() if l.strip()}
    assert set(names) <= syms
    f = ctypes.CDLL(B.CALIB_LIB).jano_calib_mfma_loop
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p]
    f.restype = ctypes.c_int
    sink = ctypes.c_void_p(0x1000)   # never dereferenced: every call below is rejected first
    assert f(2, 1, 1, sink, None, None) == 1
    assert f(-1, 1, 1, sink, None, None) == 1
    assert f(0, 0, 1, sink, None, None) == 1
    assert f(0, 1, 0, sink, None, None) == 1
    assert f(1, 1, 1, None, None, None) == 1
    g = ctypes.CDLL(B.CALIB_LIB).jano_calib_stream
    g.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_void_p]
    g.restype = ctypes.c_int
    buf = ctypes.c_void_p(0x1000)    # 16-byte aligned, never dereferenced
    assert g(2, buf, buf, 16, 1, sink, None) == 1          # mode
    assert g(0, None, buf, 16, 1, sink, None) == 1         # src NULL
    assert g(0, ctypes.c_void_p(0x1004), buf, 16, 1, sink, None) == 1   # src misaligned
    assert g(0, buf, buf, 0, 1, sink, None) == 1           # no bytes
    assert g(0, buf, buf, 24, 1, sink, None) == 1          # not a multiple of 16
    assert g(0, buf, buf, 16, 0, sink, None) == 1          # no workgroups
    assert g(0, buf, None, 16, 1, sink, None) == 1         # copy without dst
    assert g(1, buf, None, 16, 1, None, None) == 1         # read without sink


def test_version_and_status_strings():
    assert jano.abi_version() == 1
    L = jano.lib()
    assert L.jano_status_string(0) == b"ok"
    for code in (-1, -2, -3, -4, -5, -6):
        assert L.jano_status_string(code) not in (b"ok", b"unknown status")


@pytest.mark.parametrize("cfg", list(configs.CONFIGS.values()), ids=lambda c: c.name)
def test_grid_sizes_match_configs(cfg):
    B, N = jano.grid_sizes(jano.GridSpec.of(cfg))
    assert (B, N) == (cfg.B, cfg.N)
    # one fp64 partial per (channel, strip, block)
    ws = jano.analyze_workspace_bytes(jano.GridSpec.of(cfg))
    assert ws >= cfg.C * cfg.B * 8


def test_known_block_and_token_counts():
    assert jano.grid_sizes(jano.GridSpec.of(configs.V720)) == (5040, 75600)
    assert jano.grid_sizes(jano.GridSpec.of(configs.V480)) == (2184, 32760)
    assert jano.grid_sizes(jano.GridSpec.of(configs.IMAGE)) == (256, 4096)
    assert jano.grid_sizes(jano.GridSpec.of(configs.TINY)) == (48, 768)


def test_schedule_count_closed_form():
    counts = (40, 30, 30)
    got = [jano.schedule_count(counts, 50, 5, 5, (4, 2, 1), s) for s in range(50)]
    assert got[:5] == [100] * 5 and got[45:] == [100] * 5
    assert got[5:9] == [100, 30, 60, 30]
    assert sum(got) == 10 * 100 + 10 * 100 + 10 * 30 + 10 * 60 + 10 * 30


def _grid(**kw):
    base = dict(K=5, C=16, F=21, H=90, W=160, bF=1, bH=8, bW=8, pF=1, pH=2, pW=2)
    base.update(kw)
    return jano.Grid(*[base[n] for n in ("K", "C", "F", "H", "W", "bF", "bH", "bW", "pF", "pH", "pW")])


@pytest.mark.parametrize("kw", [dict(K=2), dict(C=0), dict(H=91), dict(bH=7), dict(pW=3),
                                dict(bW=0), dict(F=-1),
                                # 4 x 64 x 65 = 16640 blocks: above the 16384-block limit
                                dict(F=4, H=512, W=520, bF=1, bH=8, bW=8)])
def test_bad_geometry_rejected(kw):
    L = jano.lib()
    g = _grid(**kw)
    B, N = ctypes.c_int64(), ctypes.c_int64()
    assert L.jano_grid_sizes(ctypes.byref(g), ctypes.byref(B), ctypes.byref(N)) == jano.JANO_E_INVAL
    assert L.jano_analyze_workspace_bytes(ctypes.byref(g)) == 0
    fake = ctypes.c_void_p(0x1000)
    assert L.jano_analyze(fake, ctypes.byref(g), 400, 300, fake, fake, fake, fake, 1 << 30,
                          None) == jano.JANO_E_INVAL


def test_block_limit_accepted():
    # 128 x 128 = 16384 blocks: the largest geometry accepted
    L = jano.lib()
    g = _grid(F=1, H=1024, W=1024, bF=1, bH=8, bW=8)
    B, N = ctypes.c_int64(), ctypes.c_int64()
    assert L.jano_grid_sizes(ctypes.byref(g), ctypes.byref(B), ctypes.byref(N)) == jano.JANO_OK
    assert B.value == 16384


def test_analyze_noalloc_rejects_before_touching_the_gpu():
    # every case below returns before the scratch lookup or any launch
    L = jano.lib()
    fake = ctypes.c_void_p(0x1000)
    null = ctypes.c_void_p(0)
    g = _grid()
    assert L.jano_analyze_workspace_bytes(ctypes.byref(g)) <= jano.NOALLOC_SCRATCH_BYTES
    assert L.jano_analyze_noalloc(null, ctypes.byref(g), 400, 300, fake, fake, fake, None) == -1
    assert L.jano_analyze_noalloc(fake, ctypes.byref(g), 400, 300, fake, null, fake, None) == -1
    assert L.jano_analyze_noalloc(fake, ctypes.byref(g), 700, 400, fake, fake, fake, None) == -1
    assert L.jano_analyze_noalloc(fake, None, 400, 300, fake, fake, fake, None) == -1
    bad = _grid(K=2)
    assert L.jano_analyze_noalloc(fake, ctypes.byref(bad), 400, 300, fake, fake, fake, None) == -1
    # 64 channels x 16384 blocks of fp64 partial sums = 8 MiB > the 4 MiB array
    big = _grid(K=3, C=64, F=1, H=1024, W=1024, bF=1, bH=8, bW=8)
    need = L.jano_analyze_workspace_bytes(ctypes.byref(big))
    assert need > jano.NOALLOC_SCRATCH_BYTES
    assert L.jano_analyze_noalloc(fake, ctypes.byref(big), 400, 300, fake, fake, fake,
                                  None) == jano.JANO_E_SCRATCH
    assert b"scratch" in L.jano_status_string(jano.JANO_E_SCRATCH)


def test_analyze_argument_errors():
    L = jano.lib()
    g = _grid()
    fake = ctypes.c_void_p(0x1000)
    null = ctypes.c_void_p(0)
    ws = L.jano_analyze_workspace_bytes(ctypes.byref(g))
    assert ws > 0
    assert L.jano_analyze(null, ctypes.byref(g), 400, 300, fake, fake, fake, fake, ws, None) == -1
    assert L.jano_analyze(fake, ctypes.byref(g), 700, 400, fake, fake, fake, fake, ws, None) == -1
    assert L.jano_analyze(fake, ctypes.byref(g), -1, 300, fake, fake, fake, fake, ws, None) == -1
    assert L.jano_analyze(fake, ctypes.byref(g), 400, 300, fake, fake, fake, fake, ws - 1, None) == -4
    assert L.jano_analyze(fake, ctypes.byref(g), 400, 300, fake, fake, fake, null, ws, None) == -4
    # the two halves reject the same things
    assert L.jano_analyze_scores(null, ctypes.byref(g), fake, fake, ws, None) == -1
    assert L.jano_analyze_scores(fake, ctypes.byref(g), null, fake, ws, None) == -1
    assert L.jano_analyze_scores(fake, ctypes.byref(g), fake, fake, ws - 1, None) == -4
    assert L.jano_analyze_scores(fake, ctypes.byref(g), fake, null, ws, None) == -4
    assert L.jano_levels(null, ctypes.byref(g), 400, 300, fake, fake, None) == -1
    assert L.jano_levels(fake, ctypes.byref(g), 400, 300, null, fake, None) == -1
    assert L.jano_levels(fake, ctypes.byref(g), 400, 300, fake, null, None) == -1
    assert L.jano_levels(fake, ctypes.byref(g), 700, 400, fake, fake, None) == -1
    assert L.jano_levels(fake, ctypes.byref(g), 400, -1, fake, fake, None) == -1
    bad = _grid(K=2)
    assert L.jano_levels(fake, ctypes.byref(bad), 400, 300, fake, fake, None) == -1
    # the FFT-baseline index source
    assert L.jano_fft_scores(null, ctypes.byref(g), fake, None) == -1
    assert L.jano_fft_scores(fake, ctypes.byref(g), null, None) == -1
    assert L.jano_fft_scores(fake, ctypes.byref(bad), fake, None) == -1
    assert L.jano_fft_scores(fake, None, fake, None) == -1


def test_schedule_argument_errors():
    L = jano.lib()
    g = _grid()
    fake = ctypes.c_void_p(0x1000)
    sc = jano.Sched(50, 5, 5, (ctypes.c_int32 * 3)(4, 2, 1))
    assert L.jano_schedule(fake, ctypes.byref(g), ctypes.byref(sc), 50, fake, fake, None) == -1
    assert L.jano_schedule(fake, ctypes.byref(g), ctypes.byref(sc), -1, fake, fake, None) == -1
    bad = jano.Sched(50, 5, 5, (ctypes.c_int32 * 3)(0, 2, 1))
    assert L.jano_schedule(fake, ctypes.byref(g), ctypes.byref(bad), 7, fake, fake, None) == -1
    bad2 = jano.Sched(8, 5, 5, (ctypes.c_int32 * 3)(4, 2, 1))
    assert L.jano_schedule(fake, ctypes.byref(g), ctypes.byref(bad2), 1, fake, fake, None) == -1
    assert L.jano_schedule(fake, ctypes.byref(g), ctypes.byref(sc), 7, ctypes.c_void_p(0), fake, None) == -1


def test_rows_and_attention_argument_errors():
    L = jano.lib()
    f = ctypes.c_void_p(0x1000)
    n = ctypes.c_void_p(0)
    # gather
    assert L.jano_gather_rows(f, 0, 8, f, 1, f, None) == -1
    assert L.jano_gather_rows(f, 10, 8, n, 1, f, None) == -1
    assert L.jano_gather_rows(n, 10, 8, n, 0, n, None) == 0          # empty is a no-op
    # scatter: n_act > N, null cache
    assert L.jano_scatter_kv(f, f, f, 11, f, f, 10, 8, None) == -1
    assert L.jano_scatter_kv(f, f, f, 5, n, f, 10, 8, None) == -1
    assert L.jano_scatter_kv(n, n, n, 0, f, f, 10, 8, None) == 0
    # attention: unsupported head dim, misaligned pointer, bad sizes
    assert L.jano_attention(f, 4, f, f, 10, 2, 96, 0.0, f, None) == -2
    assert L.jano_attention(ctypes.c_void_p(0x1002), 4, f, f, 10, 2, 64, 0.0, f, None) == -1
    assert L.jano_attention(f, 4, f, f, 0, 2, 64, 0.0, f, None) == -1
    assert L.jano_attention(f, 4, f, f, 10, 0, 64, 0.0, f, None) == -1
    assert L.jano_attention(f, 4, f, f, 10, 2, 64, float("nan"), f, None) == -1
    assert L.jano_attention(f, 4, f, f, 10, 2, 64, float("inf"), f, None) == -1
    assert L.jano_attention(n, 0, f, f, 10, 2, 64, 0.0, n, None) == 0
    assert L.jano_attn_step(f, f, f, f, 11, f, f, 10, 2, 64, 0.0, f, None) == -1
    assert L.jano_attn_step(f, f, f, f, 4, f, f, 10, 2, 80, 0.0, f, None) == -2
    assert L.jano_attn_step(f, n, f, f, 4, f, f, 10, 2, 64, 0.0, f, None) == -1
    assert L.jano_check_idx(f, 4, 10, n, None) == -1
    # projection: unsupported Dm / d, bad token grid for the rotation, nulls
    qp = L.jano_qkv_proj
    g = _grid()    # token grid 3 x 16 x 16 = 768 tokens
    c = ctypes.c_float
    assert qp(f, 768, 100, f, 4, f, 2, 64, None, c(0.0), f, f, f, None) == -2     # Dm % 32
    assert qp(f, 768, 128, f, 4, f, 2, 62, None, c(0.0), f, f, f, None) == -2     # d % 4
    assert qp(f, 767, 128, f, 4, f, 2, 64, ctypes.byref(g), c(1e4), f, f, f, None) == -1  # N != grid
    assert qp(f, 768, 128, f, 4, f, 2, 4, ctypes.byref(g), c(1e4), f, f, f, None) == -1   # d < 6 rotated
    assert qp(f, 768, 128, f, 4, f, 2, 64, None, c(float("nan")), f, f, f, None) == -1
    assert qp(f, 768, 128, n, 4, f, 2, 64, None, c(0.0), f, f, f, None) == -1
    assert qp(f, 768, 128, f, 4, f, 2, 64, None, c(0.0), f, n, f, None) == -1
    assert qp(n, 768, 128, n, 0, n, 2, 64, None, c(0.0), n, n, n, None) == 0       # nothing active
    # concatenated layout: negative counts, null outputs, null sources
    cc = L.jano_concat_kv
    assert cc(f, f, -1, f, f, f, 3, f, f, 8, None) == -1
    assert cc(f, f, 2, f, f, f, 3, n, f, 8, None) == -1
    assert cc(n, f, 2, f, f, f, 3, f, f, 8, None) == -1
    assert cc(f, f, 2, n, f, f, 3, f, f, 8, None) == -1
    assert cc(f, f, 2, f, f, n, 3, f, f, 8, None) == -1
    assert cc(f, f, 2, f, f, f, 3, f, f, 0, None) == -1
    assert cc(n, n, 0, n, n, n, 0, n, n, 8, None) == 0           # empty is a no-op
    # write-back: n_act > N, null state, non-finite dt, null rows with n_act > 0
    wb = L.jano_writeback_step
    assert wb(f, f, 11, f, f, 10, 4, ctypes.c_float(0.1), None) == -1
    assert wb(f, f, 2, n, f, 10, 4, ctypes.c_float(0.1), None) == -1
    assert wb(f, f, 2, f, n, 10, 4, ctypes.c_float(0.1), None) == -1
    assert wb(f, f, 2, f, f, 10, 0, ctypes.c_float(0.1), None) == -1
    assert wb(f, f, 2, f, f, 10, 4, ctypes.c_float(float("inf")), None) == -1
    assert wb(n, f, 2, f, f, 10, 4, ctypes.c_float(0.1), None) == -1
    assert wb(f, n, 2, f, f, 10, 4, ctypes.c_float(0.1), None) == -1


def test_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(4, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        jano.attention(x, x, x)
    with pytest.raises(ValueError):
        jano.analyze(torch.zeros(5, 16, 1, 16, 16), jano.GridSpec.of(configs.TINY))


def test_attention_plan_tiles():
    # per head: (384-query tiles, 256-query tiles, 128-query tiles)
    assert jano.attention_plan(75600, 40, 128) == (197, 0, 0)     # 30.8 rounds: all 384
    assert jano.attention_plan(18468, 40, 128) == (44, 7, 0)      # 7.66 rounds -> 44 full + 7 of 256
    assert jano.attention_plan(37848, 40, 128) == (96, 4, 0)
    assert jano.attention_plan(32760, 12, 128) == (0, 128, 0)     # 4.03 rounds of 384 -> 6 of 256
    assert jano.attention_plan(200, 3, 128) == (0, 1, 0)          # one round either way
    assert jano.attention_plan(300, 256, 128) == (1, 0, 0)        # one round against two
    assert jano.attention_plan(10, 1, 64) == (0, 0, 1)
    for n, H in ((18468, 40), (37848, 40), (19640, 12), (1151, 128), (1299, 96), (7, 1)):
        k3, m2, _ = jano.attention_plan(n, H, 128)
        if k3 and m2:
            # mixed: full 384-query tiles, then 256-query tiles covering the rest
            assert 384 * k3 < n <= 384 * k3 + 256 * m2 < n + 256
        else:
            assert 384 * k3 + 256 * m2 >= n
    L = jano.lib()
    t = (ctypes.c_int32 * 3)()
    assert L.jano_attention_plan(0, 1, 128, t) == jano.JANO_E_INVAL
    assert L.jano_attention_plan(10, 0, 128, t) == jano.JANO_E_INVAL
    assert L.jano_attention_plan(10, 1, 96, t) == jano.JANO_E_UNSUPPORTED
    assert L.jano_attention_plan(10, 1, 128, None) == jano.JANO_E_INVAL


def test_attention_split_plan_and_workspace():
    # with a workspace: (384-query tiles, 256-query tiles, 128-query tiles, key ranges)
    assert jano.attention_plan_ws(18468, 75600, 40, 128) == (44, 7, 0, 1)    # 7.7 rounds: no split
    assert jano.attention_plan_ws(75600, 75600, 40, 128) == (197, 0, 0, 1)
    assert jano.attention_plan_ws(8190, 32760, 12, 128) == (0, 32, 0, 2)     # 1.4 rounds -> 2 ranges
    assert jano.attention_plan_ws(4096, 4096, 24, 128) == (0, 16, 0, 2)
    assert jano.attention_plan_ws(100, 1000, 2, 128) == (0, 1, 0, 4)
    assert jano.attention_plan_ws(10, 100, 1, 64) == (0, 0, 1, 1)            # d = 64 never splits
    assert jano.attention_plan_ws(50, 100, 1, 128)[3] == 1                  # 2 tiles: too few to split
    for n, N, H in ((8190, 32760, 12), (4096, 4096, 24), (100, 1000, 2), (3000, 500, 8)):
        S = jano.attention_plan_ws(n, N, H, 128)[3]
        assert S > 1 and -(-N // 64) >= 2 * S
        assert jano.attention_workspace_bytes(n, N, H, 128) == S * n * H * 130 * 4
    assert jano.attention_workspace_bytes(18468, 75600, 40, 128) == 0
    assert jano.attention_workspace_bytes(10, 100, 1, 64) == 0
    assert jano.attention_workspace_bytes(0, 100, 1, 128) == 0
    L = jano.lib()
    t = (ctypes.c_int32 * 4)()
    assert L.jano_attention_plan_ws(10, 0, 1, 128, t) == jano.JANO_E_INVAL
    assert L.jano_attention_plan_ws(10, 100, 1, 96, t) == jano.JANO_E_UNSUPPORTED
    assert L.jano_attention_plan_ws(10, 100, 1, 128, None) == jano.JANO_E_INVAL
    # workspace errors are reported before anything is enqueued (fake,
    # never-dereferenced device pointers)
    f = ctypes.c_void_p(0x1000)
    n, N, H, d = 8190, 32760, 12, 128
    need = jano.attention_workspace_bytes(n, N, H, d)
    assert L.jano_attention_ws(f, n, f, f, N, H, d, 0.0, f, f, need - 16, None) == jano.JANO_E_WORKSPACE
    assert L.jano_attention_ws(f, n, f, f, N, H, d, 0.0, f, ctypes.c_void_p(0x1008), need, None) == \
        jano.JANO_E_WORKSPACE
    assert L.jano_attn_step_ws(f, f, f, f, n, f, f, N, H, d, 0.0, f, f, 16, None) == jano.JANO_E_WORKSPACE
    # the usual argument checks come first
    assert L.jano_attention_ws(f, n, f, f, N, H, 96, 0.0, f, f, 0, None) == jano.JANO_E_UNSUPPORTED
    assert L.jano_attention_ws(f, n, f, f, 0, H, d, 0.0, f, f, need, None) == jano.JANO_E_INVAL
