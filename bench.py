"""Bench of the Jano hot path on one MI355X.

Workload (default): the 720p video-shaped grid, 21x45x80 = 75600 tokens,
40 heads, d = 128, bf16; warm-up latents 5 x [16, 21, 90, 160] fp32.
One step = one pass of the whole path on resident inputs:
    jano_analyze_scores (block scores) -> jano_levels (40/30/30 mix shifted
    so that the Active level holds the configured share) -> jano_schedule at an
    Active-only interleaved step -> jano_gather_rows (active rows of Q) ->
    jano_scatter_kv (fresh K/V rows into the full-sequence cache) ->
    jano_attention (active queries against the whole cache).
`value` = active-query attention FLOPs per step (4 * n_act * N * H * d) divided
by the measured wall time of the whole step. The dense reference (all N
queries), the 10/25/50% step speedups and the 50-step interleaved run on the
480p grid are reported beside it, as are per-kernel times from HIP events and
the CPU oracle timed on a bounded sample. Per-kernel times are medians: over
the timed steps for gather, scatter and attention, over 200 back-to-back calls
for the µs-scale analyzer, levels, schedule and FFT-baseline score entry
points.

    python bench.py [--steps K] [--warmup W] [--frac 0.25] [--no-cpu]

HBM traffic (`roofline.traffic`) comes from profiles/traffic.json, written by
    python bench.py --ingest-counters FETCH WRITE
from two rocprofv3 --pmc passes (FETCH_SIZE, then WRITE_SIZE; each output a
CSV or rocprofv3's SQLite .db) over
`bench.py --steps 2 --warmup 0 --no-cpu --no-extra --calibrate-copy`; it is
used only while the kernel sources still hash to what was profiled.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
ACTIVE_ONLY_OFFSET = 1         # (step - W) odd: only Active tokens are due
MIX_FOR_ACTIVE = {0.10: (600, 300), 0.25: (450, 300), 0.50: (300, 200), 1.0: (0, 0)}


def _ev(torch):
    return torch.cuda.Event(enable_timing=True)


def kernel_source_hash(name):
    p = os.path.join(ROOT, "token_sparse_attention_block_amd", "csrc", name)
    with open(p, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


TRAFFIC_KERNELS = {            # kernel name prefix -> (source file, key)
    "attn_fwd_d128_kernel": ("attention.hip", "attention"),
    "gather_rows_v16": ("rows.hip", "gather"),
    "scatter_kv_v16": ("rows.hip", "scatter"),
    "analyze_stream_kernel": ("analyze.hip", "analyze_stream"),
}


def _short_kernel_name(name):
    name = name.replace("void ", "").replace("jano::(anonymous namespace)::", "")
    return name.split("(")[0].split("<")[0]


def ingest_counters(fetch_path, write_path, workload, out_path=None):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) -> HBM bytes per launch.

    Each counter is scaled by what it reads for the 1 GiB device copy that
    --calibrate-copy issues first (the largest __amd_rocclr_copyBuffer
    dispatch: 1 GiB read, 1 GiB written). In a --no-extra run the attention
    kernel appears with two grids: the active-query step (smaller) and the
    dense reference (larger); they are stored as `attention` and
    `attention_dense`."""
    import csv
    import statistics

    def rows(path):
        # rocprofv3 writes either a CSV (--output-format csv) or its SQLite
        # database (the default): the same four fields from either
        if path.endswith(".db"):
            import sqlite3
            con = sqlite3.connect(path)
            try:
                yield from con.execute("select counter_name, kernel_name, grid_size, dispatch_id, value "
                                       "from counters_collection")
            finally:
                con.close()
        else:
            with open(path) as f:
                for r in csv.DictReader(f):
                    yield (r["Counter_Name"], r["Kernel_Name"], r["Grid_Size"], r["Dispatch_Id"],
                           r["Counter_Value"])

    def per_group(path, counter):
        groups = {}
        for name, kernel, grid, dispatch, value in rows(path):
            if name != counter:
                continue
            k = (_short_kernel_name(kernel), int(grid))
            groups.setdefault(k, {}).setdefault(str(dispatch), 0.0)
            groups[k][str(dispatch)] += float(value)
        return groups

    fg, wg = per_group(fetch_path, "FETCH_SIZE"), per_group(write_path, "WRITE_SIZE")
    gib_kib = float(1 << 20)
    # the calibration copy is the largest copy dispatch (the cache clones are smaller)
    copy_f = max(max(v.values()) for (n, _), v in fg.items() if n == "__amd_rocclr_copyBuffer")
    copy_w = max(max(v.values()) for (n, _), v in wg.items() if n == "__amd_rocclr_copyBuffer")
    fetch = {k: statistics.median(v.values()) for k, v in fg.items()}
    write = {k: statistics.median(v.values()) for k, v in wg.items()}
    f_fac, w_fac = gib_kib / copy_f, gib_kib / copy_w
    out = {"calibration": {"copy_bytes": 1 << 30, "fetch_kib": copy_f, "write_kib": copy_w,
                           "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4)}}
    for prefix, (src, key) in TRAFFIC_KERNELS.items():
        grids = sorted(g for (n, g) in fetch if n == prefix)
        if not grids:
            continue
        if key == "attention":
            if len(grids) != 2:
                raise SystemExit("expected the active and the dense attention grid, got %s" % grids)
            named = [("attention", grids[0]), ("attention_dense", grids[1])]
        else:
            named = [(key, grids[0])]
        for name, g in named:
            fb, wb = fetch[(prefix, g)] * 1024 * f_fac, write[(prefix, g)] * 1024 * w_fac
            out[name] = {"source": src, "source_sha256_16": kernel_source_hash(src),
                         "grid_threads": g, "fetch_bytes": round(fb), "write_bytes": round(wb),
                         "hbm_bytes_per_launch": round(fb + wb)}
    p = out_path or os.path.join(ROOT, "profiles", "traffic.json")
    allw = {}
    if os.path.exists(p):
        with open(p) as f:
            allw = json.load(f)
    allw[workload] = out
    with open(p, "w") as f:
        json.dump(allw, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(out, indent=1))
    return out


def summarize_trace(trace_csv, bench_log, out_md, command):
    """Markdown summary of a rocprofv3 kernel trace (--output-format csv) taken
    over a bench.py run, next to the bench line that run printed: per kernel
    and grid the dispatch count and durations, and the headline attention
    launch's average without its first (cold) dispatch set against the line's
    roofline.achieved."""
    import csv
    rows = list(csv.DictReader(open(trace_csv)))
    line = None
    for l in open(bench_log):
        l = l.strip()
        if l.startswith("{") and '"metric"' in l:
            line = json.loads(l)
    if line is None:
        raise SystemExit("no bench line in %s" % bench_log)

    def grid(r):
        gx = r.get("Grid_Size_X", r.get("Grid_Size", "0"))
        return "%s,%s" % (gx, r.get("Grid_Size_Y", "1"))

    groups = {}
    for r in rows:
        name = r["Kernel_Name"]
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3    # us
        key = (name, grid(r), r.get("Workgroup_Size_X", r.get("Workgroup_Size", "")))
        groups.setdefault(key, []).append((int(r["Start_Timestamp"]), dur))
    table = []
    for (name, g, wg), v in groups.items():
        v.sort()
        d = [x[1] for x in v]
        table.append((sum(d), name, g, wg, d))
    table.sort(reverse=True)
    cfg = line["config"]
    flops = 4.0 * cfg["n_act"] * cfg["tokens"] * cfg["heads"] * cfg["head_dim"]
    k3, m2 = line["roofline"]["tiles_per_head_384_256"]
    want_grid = "%d,1" % ((k3 + m2) * cfg["heads"] * 512)      # one workgroup of 512 per tile
    att = [t for t in table if t[1].startswith("void attn_fwd_d128_kernel") or "attn_fwd_d128_kernel" in t[1]]
    att = [t for t in att if t[2] == want_grid]
    out = ["# Kernel trace of the bench run, %s" % cfg["workload"], "",
           "Command (repository root, one MI355X, `export TMPDIR=/tmp` first):", "", "```", command, "```", "",
           "Bench line printed by the same run (excerpt): value %.2f TFLOP/s, ms_per_step %.4f, "
           "roofline.achieved %.2f TFLOP/s, frac %.5f." % (line["value"], line["ms_per_step"],
                                                           line["roofline"]["achieved"], line["roofline"]["frac"]),
           "", "Durations in microseconds (end - start per dispatch).", "",
           "| kernel | grid (threads) x,y | block | calls | avg us | avg us w/o first | min us | max us | total ms |",
           "|---|---|---|---|---|---|---|---|---|"]
    for tot, name, g, wg, d in table[:24]:
        nm = name if len(name) <= 90 else name[:87] + "..."
        rest = d[1:] if len(d) > 1 else d
        out.append("| `%s` | %s | %s | %d | %.2f | %.2f | %.2f | %.2f | %.3f |" % (
            nm, g, wg, len(d), sum(d) / len(d), sum(rest) / len(rest), min(d), max(d), tot / 1e3))
    if att:
        d = att[0][4][1:] if len(att[0][4]) > 1 else att[0][4]
        avg_ms = sum(d) / len(d) / 1e3
        tf = flops / (avg_ms * 1e-3) / 1e12
        out += ["", "Headline attention launch (grid %s): %d dispatches after the first, average %.3f ms, "
                    "max %.3f ms -> %.4g FLOP / %.3f ms = %.1f TFLOP/s = %.4f of 2.5 PFLOP/s; the bench line's "
                    "roofline.frac is %.4f (ratio %.4f). The run's ms_per_step is %.4f ms." % (
                        att[0][2], len(d), avg_ms, max(d) / 1e3, flops, avg_ms, tf, tf / 2500.0,
                        line["roofline"]["frac"], (tf / 2500.0) / line["roofline"]["frac"], line["ms_per_step"])]
    with open(out_md, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


def load_traffic(key, workload, path=None):
    """HBM bytes per launch from a committed rocprofv3 counter summary, only
    if it was taken on the current kernel source; else None."""
    p = path or os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    e = t.get(workload, {}).get(key)
    if not e or e.get("source_sha256_16") != kernel_source_hash(e["source"]):
        return None
    return e.get("hbm_bytes_per_launch")


class Path:
    """Device-resident inputs and outputs of one workload."""

    def __init__(self, torch, jano, synth, cfg, frac, n_lat_copies=5):
        self.torch, self.jano, self.cfg, self.frac = torch, jano, cfg, frac
        dev = "cuda"
        self.spec = jano.GridSpec.of(cfg)
        lat = synth.latents(cfg)
        # rotate several latent copies so the analyzer streams from HBM rather
        # than from the 256 MB last-level cache
        self.lats = [torch.from_numpy(lat).to(dev) for _ in range(n_lat_copies)]
        self.spm, self.mpm = MIX_FOR_ACTIVE[frac]
        B, N = jano.grid_sizes(self.spec)
        self.B, self.N = B, N
        self.scores = torch.empty(B, dtype=torch.float32, device=dev)
        self.fft = torch.empty(B, dtype=torch.float32, device=dev)
        self.levels = torch.empty(B, dtype=torch.uint8, device=dev)
        self.counts = torch.empty(3, dtype=torch.int32, device=dev)
        self.ws = torch.empty(jano.analyze_workspace_bytes(self.spec), dtype=torch.uint8, device=dev)
        self.idx = torch.empty(N, dtype=torch.int32, device=dev)
        self.n_dev = torch.empty(1, dtype=torch.int32, device=dev)
        sc = cfg.schedule
        self.sched = (sc.T, sc.W, sc.Cd, sc.periods)
        self.step_id = sc.W + ACTIVE_ONLY_OFFSET if frac < 1.0 else 0
        # the one host sync of a generation: level token counts -> n_act
        self.analyze(0)
        torch.cuda.synchronize()
        self.n_act = jano.schedule_count(self.counts.cpu().tolist(), sc.T, sc.W, sc.Cd,
                                         sc.periods, self.step_id)

    def analyze(self, i):
        self.analyze_scores(i)
        self.levels_()

    def analyze_scores(self, i):
        self.jano.analyze_scores(self.lats[i % len(self.lats)], self.spec, self.scores, self.ws)

    def fft_scores(self, i):
        # the copy the analyzer read longest ago, so it streams from HBM too
        self.jano.fft_scores(self.lats[(i + 1) % len(self.lats)], self.spec, self.fft)

    def levels_(self):
        self.jano.levels(self.scores, self.spec, self.spm, self.mpm, self.levels, self.counts)

    def schedule(self):
        T, W, Cd, per = self.sched
        self.jano.schedule(self.levels, self.spec, self.step_id, T, W, Cd, per, self.idx, self.n_dev)


def upload_bf16(torch, bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to("cuda")


def make_qkv(torch, synth, cfg):
    return [upload_bf16(torch, b) for b in synth.qkv_bits(cfg)]


STEP_CALLS = ("analyze_scores", "levels", "schedule", "gather", "scatter", "attention")
LAYERS = 3      # per-layer buffers the timed steps rotate through


def make_layers(torch, jano, Q, K, V, n_layers=LAYERS):
    """Per-layer device buffers, as a DiT holds one set per transformer layer:
    the hidden rows the queries are gathered from and the full-sequence K/V
    cache. Consecutive steps use consecutive layers, so the gather and the
    scatter stream from HBM: the buffers they touch total several GB, far
    above the 256 MB last-level cache."""
    layers = []
    for l in range(n_layers):
        layers.append({"Q": Q.clone() if l else Q, "Kc": K.clone(), "Vc": V.clone()})
    return layers


def run_step(p, i, lay, ev=None):
    """One whole pass on layer buffers `lay`; `ev` (len(STEP_CALLS) + 1
    events) brackets each call."""
    jano = p.jano
    idx = p.idx[:p.n_act]
    calls = (lambda: p.analyze_scores(i), p.levels_, p.schedule,
             lambda: jano.gather_rows(lay["Q"], idx, p.n_act, out=lay["q_act"]),
             lambda: jano.scatter_kv(lay["Kn"], lay["Vn"], idx, lay["Kc"], lay["Vc"], n_act=p.n_act),
             lambda: jano.attention(lay["q_act"], lay["Kc"], lay["Vc"], out=lay["out"], n_q=p.n_act))
    if ev:
        ev[0].record()
    for j, call in enumerate(calls):
        call()
        if ev:
            ev[j + 1].record()


def time_fraction(torch, jano, synth, cfg, frac, K, V, layers, steps, warmup):
    p = Path(torch, jano, synth, cfg, frac)
    n = p.n_act
    H, d = cfg.heads, cfg.d
    idx = p.idx[:n]
    p.schedule()
    for lay in layers:
        # fresh rows of each layer, as its projection would emit them
        lay["Kn"] = jano.gather_rows(K, idx, n)
        lay["Vn"] = jano.gather_rows(V, idx, n)
        lay["q_act"] = torch.empty((n, H, d), dtype=torch.bfloat16, device="cuda")
        lay["out"] = torch.empty((n, H, d), dtype=torch.bfloat16, device="cuda")
    L = len(layers)
    for i in range(warmup):
        run_step(p, i, layers[i % L])
    torch.cuda.synchronize()
    evs = [[_ev(torch) for _ in range(len(STEP_CALLS) + 1)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        run_step(p, i, layers[i % L], evs[i])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    per = {k: float(np.median([e[j].elapsed_time(e[j + 1]) for e in evs])) for j, k in enumerate(STEP_CALLS)}
    per["analyze"] = per["analyze_scores"] + per["levels"]
    per["attention_mean"] = float(np.mean([e[-2].elapsed_time(e[-1]) for e in evs]))
    for lay in layers:
        for k in ("Kn", "Vn", "q_act", "out"):
            lay.pop(k)
    return p, n, wall * 1e3, per


def time_small_calls(torch, p, reps=200):
    """Median per-call time of the µs-scale entry points over `reps` calls
    each. A spin kernel keeps the GPU busy while every call is enqueued with
    its own event pair, so the calls then run back to back on the GPU and the
    host's launch latency stays out of the intervals."""
    calls = {"analyze_scores": lambda i: p.analyze_scores(i), "levels": lambda i: p.levels_(),
             "schedule": lambda i: p.schedule(), "fft_scores": lambda i: p.fft_scores(i)}
    evs = {k: [(_ev(torch), _ev(torch)) for _ in range(reps)] for k in calls}
    torch.cuda.synchronize()
    torch.cuda._sleep(100_000_000)       # tens of ms of spinning on the stream
    for i in range(reps):
        for k, call in calls.items():
            a, b = evs[k][i]
            a.record()
            call(i)
            b.record()
    torch.cuda.synchronize()
    return {k: float(np.median([a.elapsed_time(b) for a, b in v])) for k, v in evs.items()}


def time_writeback(torch, jano, cfg, idx, reps=20):
    """jano_writeback_step on the token outputs of the workload: P = C * patch
    values per token, fresh rows for the active tokens, fp32 sampler state."""
    P = cfg.C * cfg.patch[0] * cfg.patch[1] * cfg.patch[2]
    N, n = cfg.N, idx.numel()
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    out_full = torch.randn((N, P), generator=g, device="cuda").to(torch.bfloat16)
    out_act = torch.randn((n, P), generator=g, device="cuda").to(torch.bfloat16)
    x = torch.randn((N, P), generator=g, device="cuda")
    for _ in range(3):
        jano.writeback_step(out_act, idx, out_full, x, -0.02)
    a, b = _ev(torch), _ev(torch)
    a.record()
    for _ in range(reps):
        jano.writeback_step(out_act, idx, out_full, x, -0.02)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    nbytes = 2 * n * P * 2 + N * P * (2 + 4 + 4)
    return {"ms": round(ms, 5), "tokens": N, "values_per_token": P, "n_act": n, "bytes": nbytes,
            "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 3),
            "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 5)}


def time_concat_layout(torch, jano, p, Q, K, V, reps=3):
    """The pages' own layout of an interleaved step, [fresh K/V of the active
    tokens ; cached K/V of the frozen tokens], timed beside the scatter cache:
    frozen-token list, concatenation, attention over the concatenated K/V."""
    n = p.n_act
    T, W, Cd, per = p.sched
    idx = p.idx[:n]
    fidx, nf_dev = jano.schedule(p.levels, p.spec, p.step_id, T, W, Cd, per, frozen=True)
    torch.cuda.synchronize()
    nf = int(nf_dev.item())
    Kn, Vn = jano.gather_rows(K, idx, n), jano.gather_rows(V, idx, n)
    q_act = jano.gather_rows(Q, idx, n)
    Kcat = torch.empty((n + nf,) + tuple(K.shape[1:]), dtype=torch.bfloat16, device="cuda")
    Vcat = torch.empty_like(Kcat)
    out = torch.empty_like(q_act)
    calls = (lambda: jano.schedule(p.levels, p.spec, p.step_id, T, W, Cd, per, idx=fidx, n_act=nf_dev,
                                   frozen=True),
             lambda: jano.concat_kv(Kn, Vn, K, V, fidx, n_act=n, n_frozen=nf, Kcat=Kcat, Vcat=Vcat),
             lambda: jano.attention(q_act, Kcat, Vcat, out=out, n_q=n))
    for c in calls:
        c()
    torch.cuda.synchronize()
    ev = [[_ev(torch) for _ in range(len(calls) + 1)] for _ in range(reps)]
    for e in ev:
        e[0].record()
        for j, c in enumerate(calls):
            c()
            e[j + 1].record()
    torch.cuda.synchronize()
    ms = [float(np.mean([e[j].elapsed_time(e[j + 1]) for e in ev])) for j in range(len(calls))]
    row_bytes = K.shape[1] * K.shape[2] * 2
    cat_bytes = 2 * 2 * (n + nf) * row_bytes
    return {"n_act": n, "n_frozen": nf, "schedule_frozen_ms": round(ms[0], 5), "concat_ms": round(ms[1], 5),
            "concat_GB/s": round(cat_bytes / (ms[1] * 1e-3) / 1e9, 3), "attention_ms": round(ms[2], 4),
            "path_ms": round(ms[1] + ms[2], 4)}


def time_qkv_proj(torch, jano, cfg, idx, reps=5):
    """jano_qkv_proj on the active tokens: hidden size H*d (5120 for 40 x 128),
    random weights, rotary encoding on the token grid. Rows of the hidden
    states that are not active are never read."""
    H, d = cfg.heads, cfg.d
    Dm, n = H * d, idx.numel()
    g = torch.Generator(device="cuda")
    g.manual_seed(9)
    X = torch.randn((cfg.N, Dm), generator=g, device="cuda").to(torch.bfloat16)
    W = (torch.randn((3 * H * d, Dm), generator=g, device="cuda") / 64).to(torch.bfloat16)
    spec = jano.GridSpec.of(cfg)
    out = tuple(torch.empty((n, H, d), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    for _ in range(2):
        jano.qkv_proj(X, idx, W, H, d, spec, 10000.0, out=out)
    a, b = _ev(torch), _ev(torch)
    a.record()
    for _ in range(reps):
        jano.qkv_proj(X, idx, W, H, d, spec, 10000.0, out=out)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    flops = 2.0 * n * Dm * 3 * H * d
    tf = flops / (ms * 1e-3) / 1e12
    # the vendor GEMM on the same product shape, rows pre-gathered and no
    # rotation (the same FLOPs, less work): a ceiling for this shape
    Xa = X[idx.long()].contiguous()
    Wt = W.t().contiguous()
    C = torch.empty((n, 3 * H * d), dtype=torch.bfloat16, device="cuda")
    for _ in range(2):
        torch.matmul(Xa, Wt, out=C)
    a.record()
    for _ in range(reps):
        torch.matmul(Xa, Wt, out=C)
    b.record()
    torch.cuda.synchronize()
    vtf = flops / (a.elapsed_time(b) / reps * 1e-3) / 1e12
    del X, W, out, Xa, Wt, C
    return {"ms": round(ms, 4), "n_act": n, "hidden": Dm, "out_features": 3 * H * d,
            "flops": flops, "TFLOP/s": round(tf, 2), "frac_mfma": round(tf / PEAK_BF16_TFLOPS, 5),
            "vendor_gemm_same_shape_TFLOP/s": round(vtf, 2),
            "frac_of_vendor_same_shape": round(tf / vtf, 4)}


def time_dense(torch, jano, Q, Kc, Vc, reps=20, workspace=None):
    """Median over `reps` launches of attention of the queries Q against the
    whole cache (all tokens for the dense reference), each launch between its
    own pair of events."""
    out = torch.empty_like(Q)
    jano.attention(Q, Kc, Vc, out=out, workspace=workspace)
    torch.cuda.synchronize()
    ev = [(_ev(torch), _ev(torch)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        jano.attention(Q, Kc, Vc, out=out, workspace=workspace)
        b.record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev]))


def time_configs(torch, jano, synth, configs):
    """Active-query attention on the smaller grids at their active shares
    (the first n_act rows of the config's seeded Q against its whole K/V):
    median of 20 launches each, as TFLOP/s and as a fraction of the bf16
    peak (d = 64 for the tiny grid runs the d = 64 kernel); where the launch
    splits the keys when given a workspace, also with one."""
    out = {}
    for cfg in (configs.TINY, configs.IMAGE, configs.V480):
        Q, K, V = make_qkv(torch, synth, cfg)
        N, H, d = cfg.N, cfg.heads, cfg.d
        for frac in cfg.active_fracs:
            n_act = max(1, round(frac * N))
            Qa = Q[:n_act].contiguous()
            flops = 4.0 * n_act * N * H * d
            ms = time_dense(torch, jano, Qa, K, V, 20)
            tf = flops / (ms * 1e-3) / 1e12
            rec = {"tokens": N, "heads": H, "head_dim": d, "n_act": n_act, "ms": round(ms, 4),
                   "TFLOP/s": round(tf, 2), "frac_mfma": round(tf / PEAK_BF16_TFLOPS, 4)}
            ws = jano.attention_workspace(n_act, N, H, d, "cuda")
            if ws is not None:
                ms_ws = time_dense(torch, jano, Qa, K, V, 20, workspace=ws)
                tf_ws = flops / (ms_ws * 1e-3) / 1e12
                rec["with_workspace"] = {"key_ranges": jano.attention_plan_ws(n_act, N, H, d)[3],
                                         "workspace_MB": round(ws.numel() / 1e6, 2), "ms": round(ms_ws, 4),
                                         "TFLOP/s": round(tf_ws, 2),
                                         "frac_mfma": round(tf_ws / PEAK_BF16_TFLOPS, 4)}
                del ws
            out["%s-%d%%" % (cfg.name, round(100 * frac))] = rec
        del Q, K, V
    return out


def sched_run(torch, jano, synth, cfg):
    """50-step interleaved run on the 480p grid: analyzer once after the
    warm-up steps, then per step schedule -> gather -> scatter -> attention
    (dense steps use all tokens); total versus 50 dense attention steps."""
    dev = "cuda"
    H, d, N = cfg.heads, cfg.d, cfg.N
    sc = cfg.schedule
    spec = jano.GridSpec.of(cfg)
    lat = torch.from_numpy(synth.latents(cfg)).to(dev)
    Q, K, V = make_qkv(torch, synth, cfg)
    Kc, Vc = K.clone(), V.clone()
    B, _ = jano.grid_sizes(spec)
    idx = torch.empty(N, dtype=torch.int32, device=dev)
    n_dev = torch.empty(1, dtype=torch.int32, device=dev)
    q_act = torch.empty_like(Q)
    out = torch.empty_like(Q)
    ws = torch.empty(jano.analyze_workspace_bytes(spec), dtype=torch.uint8, device=dev)
    scores, levels, counts = jano.analyze(lat, spec, workspace=ws)
    torch.cuda.synchronize()
    cnt = counts.cpu().tolist()
    n_per = [jano.schedule_count(cnt, sc.T, sc.W, sc.Cd, sc.periods, s) for s in range(sc.T)]

    def body():
        jano.analyze(lat, spec, 400, 300, scores, levels, counts, workspace=ws)
        for s in range(sc.T):
            n = n_per[s]
            jano.schedule(levels, spec, s, sc.T, sc.W, sc.Cd, sc.periods, idx, n_dev)
            ii = idx[:n]
            jano.gather_rows(Q, ii, n, out=q_act[:n])
            jano.scatter_kv(K, V, ii, Kc, Vc, n_act=n)   # stand-in fresh rows: same bytes
            jano.attention(q_act, Kc, Vc, out=out, n_q=n)

    def one_run(ev_a, ev_b):
        ev_a.record()
        body()
        ev_b.record()

    a, b = _ev(torch), _ev(torch)
    one_run(a, b)
    torch.cuda.synchronize()
    a, b = _ev(torch), _ev(torch)
    one_run(a, b)
    torch.cuda.synchronize()
    total = a.elapsed_time(b)
    # the same 50 steps captured once as a HIP graph and replayed (the entry
    # points allocate nothing and never synchronise)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    g.replay()
    torch.cuda.synchronize()
    a, b = _ev(torch), _ev(torch)
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    graph_total = a.elapsed_time(b)
    del g
    dense = time_dense(torch, jano, Q, Kc, Vc, 20)
    return {"workload": "480p-32760tok-12h-d128-50steps", "n_act_per_step": n_per,
            "dense_ms_median_of_20": round(dense, 4),
            "dense_TFLOP/s": round(4.0 * N * N * H * d / (dense * 1e-3) / 1e12, 2),
            "tiles_per_head_384_256": {"dense": list(jano.attention_plan(N, H, d)[:2]),
                                       "interleaved": sorted({tuple(jano.attention_plan(n, H, d)[:2]) for n in n_per})},
            "total_ms": round(total, 3), "graph_total_ms": round(graph_total, 3),
            "dense_50_steps_ms": round(50 * dense, 3),
            "speedup": round(50 * dense / total, 4), "graph_speedup": round(50 * dense / graph_total, 4),
            "ideal_attention_speedup": round(50 * N / sum(n_per), 4)}


def _host_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        return os.cpu_count()


def cpu_baseline(cfg, synth, Qb, Kb, Vb, spm, mpm, step_id, seconds_hint=15.0):
    """The oracle, as it stands, timed on this host's cores beside the GPU.

    Every step of the path but attention runs in full at the workload's size
    (the analyzer over all warm-up latents, levels, the step's index list, the
    gather of the active query rows and the scatter of their fresh K/V rows).
    Attention runs on a sample of active queries (all heads) against the full
    K/V cache; its time for all active queries is extrapolated linearly and
    labelled as such. `value` is the oracle's attention TFLOP/s on the sample."""
    from oracle import jano_oracle as O
    threads = _host_threads()
    N, H, d = cfg.N, cfg.heads, cfg.d
    legs = {}

    def timed(name, fn):
        t0 = time.perf_counter()
        r = fn()
        legs[name] = round((time.perf_counter() - t0) * 1e3, 2)
        return r

    lat = synth.latents(cfg)
    scores = timed("analyze_scores", lambda: O.analyze_scores(lat, cfg.block))
    del lat
    fhw = (cfg.F, cfg.H, cfg.W)
    def levels_and_counts():
        lv = O.assign_levels(scores, spm, mpm)
        return lv, O.level_token_counts(lv, fhw, cfg.patch, cfg.block)
    lv, _ = timed("levels", levels_and_counts)
    sc = cfg.schedule
    idx = timed("schedule", lambda: O.schedule(O.token_levels(lv, fhw, cfg.patch, cfg.block), step_id,
                                               sc.T, sc.W, sc.Cd, sc.periods))
    n_act = len(idx)
    timed("gather", lambda: O.gather_rows(Qb, idx))
    Kn, Vn = Kb[idx], Vb[idx]
    timed("scatter", lambda: (O.scatter_rows(Kb, idx, Kn), O.scatter_rows(Vb, idx, Vn)))
    del Kn, Vn

    n_s = 64
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(n_act, size=n_s, replace=False))
    Kf, Vf = O.bf16_to_f64(Kb), O.bf16_to_f64(Vb)
    t0 = time.perf_counter()
    O.attention(O.bf16_to_f64(Qb[idx[rows]]), Kf, Vf)
    t = time.perf_counter() - t0
    # grow the sample until one pass takes about half the time hint or more
    # (small samples run slower per query, so one extrapolation falls short)
    while t < seconds_hint / 2 and n_s < n_act:
        n_s = int(min(n_act, n_s * max(1.5, seconds_hint / max(t, 1e-3))))
        rows = np.sort(rng.choice(n_act, size=n_s, replace=False))
        t0 = time.perf_counter()
        O.attention(O.bf16_to_f64(Qb[idx[rows]]), Kf, Vf)
        t = time.perf_counter() - t0
    del Kf, Vf
    flops = 4.0 * n_s * N * H * d
    attn_ms = t * 1e3 * n_act / n_s
    step_ms = sum(legs[k] for k in ("analyze_scores", "levels", "schedule", "gather", "scatter")) + attn_ms
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(flops / t / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "seconds": round(t, 2), "cpu_model": model,
            "host_cpus": os.cpu_count(),
            "sample": "attention: %d of the step's %d active queries x %d heads against the full "
                      "%d-token K/V cache (fp64 NumPy); analyzer, levels, schedule, gather and "
                      "scatter in full at the same size" % (n_s, n_act, H, N),
            "oracle_ms": legs,
            "oracle_attention_ms_extrapolated": round(attn_ms, 1),
            "oracle_step_ms_extrapolated": round(step_ms, 1)}


def time_vendor_attention(torch, shapes, reps=5):
    """PyTorch's fused scaled-dot-product attention (its flash backend only;
    the math fallback stays disabled) on the same shapes with random bf16
    Q [1,H,n,d], K/V [1,H,N,d] in the layout it takes: the attention the
    framework itself offers on this part, timed like this path (median of
    `reps` after two warm calls). Returns {shape: {...}} or a note when the
    backend is not available."""
    try:
        from torch.nn.attention import SDPBackend, sdpa_kernel
    except ImportError as e:
        return {"unavailable": str(e)}
    out = {"backend": "torch.nn.functional.scaled_dot_product_attention, flash backend"}
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    for name, nq, N, H, d in shapes:
        q = torch.randn((1, H, nq, d), generator=g, device="cuda").to(torch.bfloat16)
        k = torch.randn((1, H, N, d), generator=g, device="cuda").to(torch.bfloat16)
        v = torch.randn((1, H, N, d), generator=g, device="cuda").to(torch.bfloat16)
        try:
            with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
                for _ in range(2):
                    torch.nn.functional.scaled_dot_product_attention(q, k, v)
                ev = [(_ev(torch), _ev(torch)) for _ in range(reps)]
                for a, b in ev:
                    a.record()
                    torch.nn.functional.scaled_dot_product_attention(q, k, v)
                    b.record()
                torch.cuda.synchronize()
            ms = sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]
            out[name] = {"ms": round(ms, 4), "TFLOP/s": round(4.0 * nq * N * H * d / (ms * 1e-3) / 1e12, 2)}
        except Exception as e:  # noqa: BLE001 -- an optional comparison must not cost the bench line
            out[name] = {"unavailable": (str(e).splitlines() or [type(e).__name__])[0][:200]}
        del q, k, v
    torch.cuda.empty_cache()
    return out


def measure_ceilings(torch, reps=10):
    """Ceilings re-measured on this part in this run, beside the published
    peaks: the best of two large square bf16 GEMMs through torch.matmul (the
    vendor GEMM library, contiguous operands) for the matrix cores, and a
    1 GiB device-to-device copy for HBM (read + write bytes)."""
    best, best_n = 0.0, 0
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    for n, r in ((8192, reps), (16384, max(2, reps // 4))):
        A = torch.randn((n, n), generator=g, device="cuda").to(torch.bfloat16)
        B = torch.randn((n, n), generator=g, device="cuda").to(torch.bfloat16)
        C = torch.empty((n, n), dtype=torch.bfloat16, device="cuda")
        for _ in range(2):
            torch.matmul(A, B, out=C)
        a, b = _ev(torch), _ev(torch)
        a.record()
        for _ in range(r):
            torch.matmul(A, B, out=C)
        b.record()
        torch.cuda.synchronize()
        tf = 2.0 * n ** 3 * r / (a.elapsed_time(b) * 1e-3) / 1e12
        if tf > best:
            best, best_n = tf, n
        del A, B, C
    gemm = best
    loop = measure_mfma_loop(torch)
    x = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    x.fill_(1.0)
    for _ in range(3):
        y.copy_(x)
    a, b = _ev(torch), _ev(torch)
    a.record()
    for _ in range(reps):
        y.copy_(x)
    b.record()
    torch.cuda.synchronize()
    copy = 2.0 * x.numel() * 4 * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del x, y
    torch.cuda.empty_cache()
    out = {"gemm_bf16_TFLOP/s": round(gemm, 2), "gemm_size": best_n, "copy_1GiB_GB/s": round(copy, 1)}
    out.update(loop)
    out.update(measure_streaming(torch, reps))
    return out


def measure_streaming(torch, reps=10):
    """HBM rates of plain streaming on this part: the calibration library's
    16-byte non-temporal copy (1 GiB read + 1 GiB written) and read (1 GiB),
    best over a few grid sizes, each timed over `reps` back-to-back calls on
    two alternating buffer pairs (4 GiB in all, far past the last-level cache)."""
    import ctypes
    from token_sparse_attention_block_amd import build as B
    f = ctypes.CDLL(B.CALIB_LIB).jano_calib_stream
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    nbytes = 1 << 30
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(4)]
    for b_ in bufs:
        b_.fill_(1)
    sink = torch.empty(8192 * 256, dtype=torch.float32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = {}
    for mode, name, moved in ((0, "stream_copy_GB/s", 2 * nbytes), (1, "stream_read_GB/s", nbytes)):
        best = 0.0
        for wgs in (1024, 2048, 4096, 8192):
            def call(i):
                src, dst = bufs[2 * (i % 2)], bufs[2 * (i % 2) + 1]
                if f(mode, ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), nbytes, wgs,
                     ctypes.c_void_p(sink.data_ptr()), st) != 0:
                    raise RuntimeError("jano_calib_stream failed")
            for i in range(2):
                call(i)
            a, b = _ev(torch), _ev(torch)
            a.record()
            for i in range(reps):
                call(i)
            b.record()
            torch.cuda.synchronize()
            best = max(best, moved * reps / (a.elapsed_time(b) * 1e-3) / 1e9)
        res[name] = round(best, 1)
    del bufs, sink
    torch.cuda.empty_cache()
    return res


def measure_mfma_loop(torch, iters=30000):
    """The bf16 matrix-core rate this part sustains under full load: the
    calibration library's register-only MFMA loop (no memory traffic, no other
    instructions) on one workgroup of 8 waves per CU, timed with events, for
    both MFMA shapes; also the shader clock each ran at (a wave's loop cycles
    over the launch time)."""
    import ctypes
    from token_sparse_attention_block_amd import build as B
    if not os.path.exists(B.CALIB_LIB):
        raise RuntimeError("%s is not built (run __graft_entry__.build())" % B.CALIB_LIB)
    f = ctypes.CDLL(B.CALIB_LIB).jano_calib_mfma_loop
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(ncu * 512, dtype=torch.float32, device="cuda")
    cyc = torch.empty(ncu * 8, dtype=torch.int64, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = {}
    for shape, name in ((0, "16x16x32"), (1, "32x32x16")):
        if f(shape, ncu, 500, ctypes.c_void_p(sink.data_ptr()), None, st) != 0:
            raise RuntimeError("jano_calib_mfma_loop failed")
        a, b = _ev(torch), _ev(torch)
        a.record()
        rc = f(shape, ncu, iters, ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(cyc.data_ptr()), st)
        b.record()
        torch.cuda.synchronize()
        if rc != 0:
            raise RuntimeError("jano_calib_mfma_loop failed")
        ms = a.elapsed_time(b)
        flop = ncu * 8 * iters * 524288.0
        res["mfma_loop_%s_TFLOP/s" % name] = round(flop / (ms * 1e-3) / 1e12, 2)
        res["mfma_loop_%s_GHz" % name] = round(float(cyc.max().item()) / (ms * 1e-3) / 1e9, 3)
    res["mfma_loop_bf16_TFLOP/s"] = max(res["mfma_loop_16x16x32_TFLOP/s"], res["mfma_loop_32x32x16_TFLOP/s"])
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--frac", type=float, default=0.25)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="headline fraction only")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--trace-summary", nargs=4, metavar=("TRACE_CSV", "BENCH_LOG", "OUT_MD", "COMMAND"),
                    help="write a markdown summary of a rocprofv3 kernel trace of a bench run and exit")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH", "WRITE"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc outputs (CSV or .db) and exit")
    args = ap.parse_args()
    if args.trace_summary:
        summarize_trace(*args.trace_summary)
        return
    if args.ingest_counters:
        ingest_counters(*args.ingest_counters, "720p-active%d" % round(100 * args.frac))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the path has no multi-GPU mode "
              "(heads would shard across GPUs with no exchange inside the path)", file=sys.stderr)
        sys.exit(2)
    if args.frac not in MIX_FOR_ACTIVE:
        sys.exit("--frac must be one of %s" % sorted(MIX_FOR_ACTIVE))

    import torch
    from token_sparse_attention_block_amd import configs, jano, synth
    jano.lib()
    torch.cuda.set_device(0)
    cfg = configs.V720
    N, H, d = cfg.N, cfg.heads, cfg.d
    if args.calibrate_copy:
        # a copy of known size: 1 GiB read + 1 GiB written per dispatch
        src = torch.empty(1 << 29, dtype=torch.bfloat16, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        print("bench: calibration copy of %d bytes done" % (src.numel() * 2), file=sys.stderr, flush=True)
        del src, dst
    print("bench: generating %s inputs" % cfg.name, file=sys.stderr, flush=True)
    Qb, Kb, Vb = synth.qkv_bits(cfg)
    Q, K, V = (upload_bf16(torch, b) for b in (Qb, Kb, Vb))
    if args.no_cpu:
        del Qb, Kb, Vb
    layers = make_layers(torch, jano, Q, K, V)

    print("bench: headline fraction %.2f" % args.frac, file=sys.stderr, flush=True)
    p, n_act, ms_step, per = time_fraction(torch, jano, synth, cfg, args.frac, K, V, layers,
                                           args.steps, args.warmup)
    small = time_small_calls(torch, p)
    per.update(small)
    per["analyze"] = per["analyze_scores"] + per["levels"]
    attn_flops = 4.0 * n_act * N * H * d
    value = attn_flops / (ms_step * 1e-3) / 1e12
    achieved = attn_flops / (per["attention_mean"] * 1e-3) / 1e12   # average launch
    lat_bytes = cfg.latent_bytes + p.B * 4      # latents read, scores written
    fft_bytes = cfg.latent_bytes // cfg.K + p.B * 4   # the latest latent read, scores written
    row_bytes = H * d * 2
    kernels = {
        "analyze_scores": {"ms": per["analyze_scores"], "bytes": lat_bytes,
                           "GB/s": lat_bytes / (per["analyze_scores"] * 1e-3) / 1e9},
        "levels": {"ms": per["levels"]},
        "analyze": {"ms": per["analyze"]},
        "schedule": {"ms": per["schedule"]},
        "gather": {"ms": per["gather"], "bytes": 2 * n_act * row_bytes,
                   "GB/s": 2 * n_act * row_bytes / (per["gather"] * 1e-3) / 1e9},
        "scatter": {"ms": per["scatter"], "bytes": 4 * n_act * row_bytes,
                    "GB/s": 4 * n_act * row_bytes / (per["scatter"] * 1e-3) / 1e9},
        "attention": {"ms": per["attention"], "flops": attn_flops, "TFLOP/s": achieved},
        "fft_scores": {"ms": per["fft_scores"], "bytes": fft_bytes,
                       "GB/s": fft_bytes / (per["fft_scores"] * 1e-3) / 1e9},
    }
    wl = "720p-active%d" % round(100 * args.frac)
    kernels["fft_scores"]["frac_hbm"] = kernels["fft_scores"]["GB/s"] / PEAK_HBM_GBS
    for k in ("analyze_scores", "gather", "scatter"):
        kernels[k]["frac_hbm"] = kernels[k]["GB/s"] / PEAK_HBM_GBS
        kernels[k]["traffic"] = load_traffic("analyze_stream" if k == "analyze_scores" else k, wl)
    kernels["attention"]["frac_mfma"] = achieved / PEAK_BF16_TFLOPS
    for v in kernels.values():
        for kk in list(v):
            if isinstance(v[kk], float):
                v[kk] = round(v[kk], 5)

    concat = None
    if not args.no_extra:
        print("bench: concatenated layout", file=sys.stderr, flush=True)
        concat = time_concat_layout(torch, jano, p, Q, K, V)
        concat["scatter_path_ms"] = round(per["scatter"] + per["attention"], 4)

    proj = None
    if not args.no_extra:
        print("bench: QKV projection", file=sys.stderr, flush=True)
        proj = time_qkv_proj(torch, jano, cfg, p.idx[:n_act])

    per_config = None
    if not args.no_extra:
        print("bench: attention on the smaller grids", file=sys.stderr, flush=True)
        per_config = time_configs(torch, jano, synth, configs)

    vendor_attn = None
    if not args.no_extra:
        print("bench: vendor attention", file=sys.stderr, flush=True)
        vendor_attn = time_vendor_attention(torch, (("active", n_act, N, H, d), ("dense", N, N, H, d)))

    print("bench: write-back step", file=sys.stderr, flush=True)
    writeback = time_writeback(torch, jano, cfg, p.idx[:n_act])

    print("bench: dense reference", file=sys.stderr, flush=True)
    dense_ms = time_dense(torch, jano, Q, layers[0]["Kc"], layers[0]["Vc"], 20)
    dense_tflops = 4.0 * N * N * H * d / (dense_ms * 1e-3) / 1e12
    speedups = {}
    path_ms_head = per["gather"] + per["scatter"] + per["attention"]
    speedups["%d%%" % round(100 * args.frac)] = {
        "n_act": n_act, "path_ms": round(path_ms_head, 4), "speedup": round(dense_ms / path_ms_head, 4),
        "attention_TFLOP/s": round(achieved, 2)}
    extra = {}
    if not args.no_extra:
        for f in (0.10, 0.25, 0.50):
            if abs(f - args.frac) < 1e-9:
                continue
            print("bench: fraction %.2f" % f, file=sys.stderr, flush=True)
            pf, nf, _, perf = time_fraction(torch, jano, synth, cfg, f, K, V, layers, 6, 3)
            pm = perf["gather"] + perf["scatter"] + perf["attention"]
            speedups["%d%%" % round(100 * f)] = {
                "n_act": nf, "path_ms": round(pm, 4), "speedup": round(dense_ms / pm, 4),
                "attention_TFLOP/s": round(4.0 * nf * N * H * d / (perf["attention"] * 1e-3) / 1e12, 2)}
            del pf
        del Q, K, V, layers
        torch.cuda.empty_cache()
        print("bench: 50-step interleaved run (480p)", file=sys.stderr, flush=True)
        extra["sched480p"] = sched_run(torch, jano, synth, configs.SCHED480)

    print("bench: measured ceilings", file=sys.stderr, flush=True)
    ceilings = measure_ceilings(torch)
    ceilings["attention_frac_of_gemm"] = round(achieved / ceilings["gemm_bf16_TFLOP/s"], 4)
    ceilings["attention_frac_of_mfma_loop"] = round(achieved / ceilings["mfma_loop_bf16_TFLOP/s"], 4)
    for k in ("gather", "scatter", "analyze_scores"):
        if "GB/s" in kernels[k]:
            ceilings["%s_frac_of_copy" % k] = round(kernels[k]["GB/s"] / ceilings["copy_1GiB_GB/s"], 4)
    # against plain streaming of the same kind: row copies read and write,
    # the analyzer only reads
    for k, c in (("gather", "stream_copy_GB/s"), ("scatter", "stream_copy_GB/s"),
                 ("analyze_scores", "stream_read_GB/s")):
        if "GB/s" in kernels[k] and ceilings.get(c):
            ceilings["%s_frac_of_%s" % (k, c[:-5])] = round(kernels[k]["GB/s"] / ceilings[c], 4)

    cpu = None
    if not args.no_cpu:
        print("bench: CPU oracle sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(cfg, synth, Qb, Kb, Vb, p.spm, p.mpm, p.step_id)

    line = {
        "metric": "active-query attention TFLOP/s + step speedup vs dense at 75.6k tokens",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V; x_t=(1-t)x0+t*eps warm-up latents)",
        "config": {"workload": "720p-75600tok-40h-d128-active%d" % round(100 * args.frac),
                   "tokens": N, "heads": H, "head_dim": d, "n_act": n_act,
                   "latents": list(cfg.latent_shape), "block_latent_px": list(cfg.block),
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 5),
                     "traffic": load_traffic("attention", wl),
                     "kernel": "attn_fwd_d128_kernel",
                     "tiles_per_head_384_256": list(jano.attention_plan(n_act, H, d)[:2]),
                     "launch_ms_median": round(per["attention"], 4),
                     "launch_ms_mean": round(per["attention_mean"], 4)},
        "cpu_baseline": cpu,
        "step_speedup_vs_dense": speedups,
        "dense": {"ms": round(dense_ms, 4), "TFLOP/s": round(dense_tflops, 3)},
        "kernels": kernels,
        "ceilings": ceilings,
        "writeback": writeback,
    }
    if concat is not None:
        line["concat_layout"] = concat
    if proj is not None:
        line["qkv_proj"] = proj
    if per_config is not None:
        line["attention_other_grids"] = per_config
    if vendor_attn is not None:
        for key, ours in (("active", achieved), ("dense", dense_tflops)):
            if "TFLOP/s" in vendor_attn.get(key, {}):
                vendor_attn[key]["this_kernel_TFLOP/s"] = round(ours, 2)
                vendor_attn[key]["speedup_of_this_kernel"] = round(ours / vendor_attn[key]["TFLOP/s"], 3)
        line["vendor_attention"] = vendor_attn
    line.update(extra)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
