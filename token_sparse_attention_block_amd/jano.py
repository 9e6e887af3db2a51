"""Python binding of libjano (ctypes). Argument marshalling only.

Every function takes torch tensors that live on a ROCm device, checks dtype,
shape, contiguity and device, and hands raw pointers plus the current HIP
stream to the C ABI declared in include/jano.h. All computation happens in the
library's HIP kernels; there is no CPU fallback. If libjano.so is missing the
first call raises, naming the build command.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

PKG = os.path.dirname(os.path.abspath(__file__))
# JANO_LIB selects another build of the same library (the host-ASan build in
# the host-only ABI tests); the default is the in-tree libjano.so
LIB_PATH = os.environ.get("JANO_LIB") or os.path.join(PKG, "lib", "libjano.so")

JANO_OK, JANO_E_INVAL, JANO_E_UNSUPPORTED, JANO_E_RANGE, JANO_E_WORKSPACE, JANO_E_HIP = 0, -1, -2, -3, -4, -5
JANO_E_SCRATCH = -6
NOALLOC_SCRATCH_BYTES = 4 << 20

EXPORTS = (
    "jano_abi_version", "jano_status_string", "jano_grid_sizes", "jano_schedule_count",
    "jano_analyze_workspace_bytes", "jano_analyze_scores", "jano_fft_scores", "jano_levels",
    "jano_analyze", "jano_analyze_noalloc",
    "jano_schedule", "jano_schedule_frozen", "jano_concat_kv", "jano_gather_rows",
    "jano_writeback_step", "jano_qkv_proj",
    "jano_scatter_kv", "jano_attention", "jano_attention_plan", "jano_attn_step", "jano_check_idx",
    "jano_attention_ws", "jano_attn_step_ws", "jano_attention_workspace_bytes", "jano_attention_plan_ws",
)


class JanoError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__("%s failed with status %d (%s)" % (fn, status, msg))
        self.status = status


class Grid(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("K", "C", "F", "H", "W", "bF", "bH", "bW", "pF", "pH", "pW")]


class Sched(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("W", ctypes.c_int32), ("Cd", ctypes.c_int32),
                ("period", ctypes.c_int32 * 3)]


@dataclass(frozen=True)
class GridSpec:
    """Latent/token geometry: K x [C,F,H,W] latents, block and patch in latent px."""
    K: int
    C: int
    F: int
    H: int
    W: int
    block: tuple
    patch: tuple

    @classmethod
    def of(cls, cfg):
        return cls(cfg.K, cfg.C, cfg.F, cfg.H, cfg.W, tuple(cfg.block), tuple(cfg.patch))

    def c(self) -> Grid:
        return Grid(self.K, self.C, self.F, self.H, self.W, *self.block, *self.patch)


_lib = None


def lib():
    """Loads libjano.so once; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libjano.so not found at %s; build it with "
                               "`python -m token_sparse_attention_block_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
        gp, sp = ctypes.POINTER(Grid), ctypes.POINTER(Sched)
        sig = {
            "jano_abi_version": ([], i32),
            "jano_status_string": ([i32], ctypes.c_char_p),
            "jano_grid_sizes": ([gp, ctypes.POINTER(i64), ctypes.POINTER(i64)], i32),
            "jano_schedule_count": ([ctypes.POINTER(ctypes.c_int32), sp, i32, ctypes.POINTER(i64)], i32),
            "jano_analyze_workspace_bytes": ([gp], ctypes.c_size_t),
            "jano_schedule_frozen": ([vp, gp, sp, i32, vp, vp, vp], i32),
            "jano_concat_kv": ([vp, vp, i64, vp, vp, vp, i64, vp, vp, i64, vp], i32),
            "jano_qkv_proj": ([vp, i64, i64, vp, i64, vp, i32, i32, gp, ctypes.c_float, vp, vp, vp, vp], i32),
            "jano_writeback_step": ([vp, vp, i64, vp, vp, i64, i64, ctypes.c_float, vp], i32),
            "jano_analyze_scores": ([vp, gp, vp, vp, ctypes.c_size_t, vp], i32),
            "jano_fft_scores": ([vp, gp, vp, vp], i32),
            "jano_levels": ([vp, gp, i32, i32, vp, vp, vp], i32),
            "jano_analyze": ([vp, gp, i32, i32, vp, vp, vp, vp, ctypes.c_size_t, vp], i32),
            "jano_analyze_noalloc": ([vp, gp, i32, i32, vp, vp, vp, vp], i32),
            "jano_schedule": ([vp, gp, sp, i32, vp, vp, vp], i32),
            "jano_gather_rows": ([vp, i64, i64, vp, i64, vp, vp], i32),
            "jano_scatter_kv": ([vp, vp, vp, i64, vp, vp, i64, i64, vp], i32),
            "jano_attention": ([vp, i64, vp, vp, i64, i32, i32, f32, vp, vp], i32),
            "jano_attention_plan": ([i64, i32, i32, vp], i32),
            "jano_attn_step": ([vp, vp, vp, vp, i64, vp, vp, i64, i32, i32, f32, vp, vp], i32),
            "jano_attention_ws": ([vp, i64, vp, vp, i64, i32, i32, f32, vp, vp, ctypes.c_size_t, vp], i32),
            "jano_attn_step_ws": ([vp, vp, vp, vp, i64, vp, vp, i64, i32, i32, f32, vp, vp, ctypes.c_size_t,
                                   vp], i32),
            "jano_attention_workspace_bytes": ([i64, i64, i32, i32], ctypes.c_size_t),
            "jano_attention_plan_ws": ([i64, i64, i32, i32, vp], i32),
            "jano_check_idx": ([vp, i64, i64, vp, vp], i32),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _check(fn, status):
    if status != JANO_OK:
        raise JanoError(fn, status, lib().jano_status_string(status).decode())


def _torch():
    import torch
    return torch


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else ctypes.c_void_p(0)


def _need(t, name, dtype, shape=None, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be on a ROCm device, got %s" % (name, t.device))
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


# ------------------------------------------------------------------ helpers --

def abi_version() -> int:
    return lib().jano_abi_version()


def grid_sizes(spec: GridSpec):
    B, N = ctypes.c_int64(), ctypes.c_int64()
    g = spec.c()
    _check("jano_grid_sizes", lib().jano_grid_sizes(ctypes.byref(g), ctypes.byref(B), ctypes.byref(N)))
    return B.value, N.value


def analyze_workspace_bytes(spec: GridSpec) -> int:
    g = spec.c()
    return lib().jano_analyze_workspace_bytes(ctypes.byref(g))


def attention_plan(n_q, H, d) -> tuple:
    """jano_attention_plan: query tiles per head of the attention launch,
    (384-query tiles, 256-query tiles, 128-query tiles)."""
    t = (ctypes.c_int32 * 3)()
    _check("jano_attention_plan", lib().jano_attention_plan(int(n_q), int(H), int(d), t))
    return tuple(t)


def attention_plan_ws(n_q, N, H, d) -> tuple:
    """jano_attention_plan_ws: the plan of an attention launch given a
    workspace, (384-query tiles, 256-query tiles, 128-query tiles, key
    ranges per query tile)."""
    t = (ctypes.c_int32 * 4)()
    _check("jano_attention_plan_ws", lib().jano_attention_plan_ws(int(n_q), int(N), int(H), int(d), t))
    return tuple(t)


def attention_workspace_bytes(n_q, N, H, d) -> int:
    """jano_attention_workspace_bytes: workspace the key-split plan needs (0: none)."""
    return int(lib().jano_attention_workspace_bytes(int(n_q), int(N), int(H), int(d)))


def attention_workspace(n_q, N, H, d, device):
    """A workspace for attention(..., workspace=) / attn_step(..., workspace=)
    sized for this shape (None when the plan does not split)."""
    n = attention_workspace_bytes(n_q, N, H, d)
    return _torch().empty(n, dtype=_torch().uint8, device=device) if n else None


def schedule_count(level_tok_counts, T, W, Cd, periods, step) -> int:
    c = (ctypes.c_int32 * 3)(*[int(x) for x in level_tok_counts])
    sc = Sched(T, W, Cd, (ctypes.c_int32 * 3)(*periods))
    n = ctypes.c_int64()
    _check("jano_schedule_count", lib().jano_schedule_count(c, ctypes.byref(sc), int(step), ctypes.byref(n)))
    return n.value


# ------------------------------------------------------------ entry points --

def analyze(lat, spec: GridSpec, static_permille=400, moderate_permille=300,
            scores=None, levels=None, counts=None, workspace=None):
    """jano_analyze. lat fp32 [K,C,F,H,W] on device -> (scores fp32 [B],
    levels uint8 [B], counts int32 [3]); all outputs stay on the device."""
    torch = _torch()
    _need(lat, "lat", torch.float32, (spec.K, spec.C, spec.F, spec.H, spec.W))
    B, _ = grid_sizes(spec)
    dev = lat.device
    scores = torch.empty(B, dtype=torch.float32, device=dev) if scores is None else scores
    levels = torch.empty(B, dtype=torch.uint8, device=dev) if levels is None else levels
    counts = torch.empty(3, dtype=torch.int32, device=dev) if counts is None else counts
    _need(scores, "scores", torch.float32, (B,), dev)
    _need(levels, "levels", torch.uint8, (B,), dev)
    _need(counts, "counts", torch.int32, (3,), dev)
    nbytes = analyze_workspace_bytes(spec)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, None, dev)
    g = spec.c()
    _check("jano_analyze", lib().jano_analyze(
        _ptr(lat), ctypes.byref(g), int(static_permille), int(moderate_permille), _ptr(scores),
        _ptr(levels), _ptr(counts), _ptr(workspace), workspace.numel(), _stream(lat)))
    return scores, levels, counts


def analyze_noalloc(lat, spec: GridSpec, scores, levels, counts, static_permille=400,
                    moderate_permille=300):
    """jano_analyze_noalloc: jano_analyze into caller-given outputs (scores
    fp32 [B], levels uint8 [B], counts int32 [3] on lat's device) with the
    library's fixed scratch array as workspace. Nothing is allocated."""
    torch = _torch()
    _need(lat, "lat", torch.float32, (spec.K, spec.C, spec.F, spec.H, spec.W))
    B, _ = grid_sizes(spec)
    dev = lat.device
    _need(scores, "scores", torch.float32, (B,), dev)
    _need(levels, "levels", torch.uint8, (B,), dev)
    _need(counts, "counts", torch.int32, (3,), dev)
    g = spec.c()
    with torch.cuda.device(dev):
        _check("jano_analyze_noalloc", lib().jano_analyze_noalloc(
            _ptr(lat), ctypes.byref(g), int(static_permille), int(moderate_permille), _ptr(scores),
            _ptr(levels), _ptr(counts), _stream(lat)))
    return scores, levels, counts


def analyze_scores(lat, spec: GridSpec, scores=None, workspace=None):
    """jano_analyze_scores. lat fp32 [K,C,F,H,W] on device -> scores fp32 [B]
    on the device."""
    torch = _torch()
    _need(lat, "lat", torch.float32, (spec.K, spec.C, spec.F, spec.H, spec.W))
    B, _ = grid_sizes(spec)
    dev = lat.device
    scores = torch.empty(B, dtype=torch.float32, device=dev) if scores is None else scores
    _need(scores, "scores", torch.float32, (B,), dev)
    nbytes = analyze_workspace_bytes(spec)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, None, dev)
    g = spec.c()
    _check("jano_analyze_scores", lib().jano_analyze_scores(
        _ptr(lat), ctypes.byref(g), _ptr(scores), _ptr(workspace), workspace.numel(), _stream(lat)))
    return scores


def fft_scores(lat, spec: GridSpec, scores=None):
    """jano_fft_scores. lat fp32 [K,C,F,H,W] on device -> the FFT complexity
    baseline's block scores fp32 [B] on the device (an alternative index
    source: rank them with levels() like the analyzer's scores)."""
    torch = _torch()
    _need(lat, "lat", torch.float32, (spec.K, spec.C, spec.F, spec.H, spec.W))
    B, _ = grid_sizes(spec)
    scores = torch.empty(B, dtype=torch.float32, device=lat.device) if scores is None else scores
    _need(scores, "scores", torch.float32, (B,), lat.device)
    g = spec.c()
    _check("jano_fft_scores", lib().jano_fft_scores(_ptr(lat), ctypes.byref(g), _ptr(scores), _stream(lat)))
    return scores


def levels(scores, spec: GridSpec, static_permille=400, moderate_permille=300, levels=None,
           counts=None):
    """jano_levels. scores fp32 [B] on device -> (levels uint8 [B],
    counts int32 [3]) on the device."""
    torch = _torch()
    B, _ = grid_sizes(spec)
    _need(scores, "scores", torch.float32, (B,))
    dev = scores.device
    lv = torch.empty(B, dtype=torch.uint8, device=dev) if levels is None else levels
    counts = torch.empty(3, dtype=torch.int32, device=dev) if counts is None else counts
    _need(lv, "levels", torch.uint8, (B,), dev)
    _need(counts, "counts", torch.int32, (3,), dev)
    g = spec.c()
    _check("jano_levels", lib().jano_levels(
        _ptr(scores), ctypes.byref(g), int(static_permille), int(moderate_permille), _ptr(lv),
        _ptr(counts), _stream(scores)))
    return lv, counts


def schedule(levels, spec: GridSpec, step, T=50, W=5, Cd=5, periods=(4, 2, 1), idx=None, n_act=None,
             frozen=False):
    """jano_schedule (frozen=False) or jano_schedule_frozen (frozen=True) ->
    (idx int32 [N] (first n valid), n int32 [1]) on device."""
    torch = _torch()
    B, N = grid_sizes(spec)
    _need(levels, "levels", torch.uint8, (B,))
    dev = levels.device
    idx = torch.empty(N, dtype=torch.int32, device=dev) if idx is None else idx
    n_act = torch.empty(1, dtype=torch.int32, device=dev) if n_act is None else n_act
    _need(idx, "idx", torch.int32, None, dev)
    if idx.numel() < N:
        raise ValueError("idx needs capacity for %d tokens" % N)
    _need(n_act, "n_act", torch.int32, (1,), dev)
    g = spec.c()
    sc = Sched(T, W, Cd, (ctypes.c_int32 * 3)(*periods))
    name = "jano_schedule_frozen" if frozen else "jano_schedule"
    _check(name, getattr(lib(), name)(_ptr(levels), ctypes.byref(g), ctypes.byref(sc), int(step),
                                      _ptr(idx), _ptr(n_act), _stream(levels)))
    return idx, n_act


def gather_rows(X, idx, n_act=None, out=None):
    """jano_gather_rows: X [N, ...] bf16, idx int32 -> X[idx[:n_act]]."""
    torch = _torch()
    _need(X, "X", torch.bfloat16)
    _need(idx, "idx", torch.int32, None, X.device)
    n = idx.numel() if n_act is None else int(n_act)
    if n > idx.numel():
        raise ValueError("n_act exceeds idx length")
    N = X.shape[0]
    D = X.numel() // max(N, 1)
    out = torch.empty((n,) + tuple(X.shape[1:]), dtype=X.dtype, device=X.device) if out is None else out
    _need(out, "out", torch.bfloat16, (n,) + tuple(X.shape[1:]), X.device)
    _check("jano_gather_rows", lib().jano_gather_rows(_ptr(X), N, D, _ptr(idx), n, _ptr(out), _stream(X)))
    return out


def scatter_kv(K_new, V_new, idx, Kc, Vc, n_act=None):
    """jano_scatter_kv: Kc[idx[i]] = K_new[i], Vc[idx[i]] = V_new[i] in place."""
    torch = _torch()
    _need(Kc, "Kc", torch.bfloat16)
    dev = Kc.device
    _need(Vc, "Vc", torch.bfloat16, tuple(Kc.shape), dev)
    n = idx.numel() if n_act is None else int(n_act)
    _need(K_new, "K_new", torch.bfloat16, None, dev)
    _need(V_new, "V_new", torch.bfloat16, None, dev)
    _need(idx, "idx", torch.int32, None, dev)
    N = Kc.shape[0]
    HD = Kc.numel() // N
    for name, t in (("K_new", K_new), ("V_new", V_new)):
        if t.numel() < n * HD or tuple(t.shape[1:]) != tuple(Kc.shape[1:]):
            raise ValueError("%s must be [>= n_act] x %s" % (name, tuple(Kc.shape[1:])))
    if n > idx.numel():
        raise ValueError("n_act exceeds idx length")
    _check("jano_scatter_kv", lib().jano_scatter_kv(_ptr(K_new), _ptr(V_new), _ptr(idx), n,
                                                    _ptr(Kc), _ptr(Vc), N, HD, _stream(Kc)))


def _attn_shapes(Q, Kc, Vc, n):
    torch = _torch()
    _need(Kc, "Kc", torch.bfloat16)
    dev = Kc.device
    if Kc.dim() != 3:
        raise ValueError("Kc must be [N, H, d]")
    N, H, d = Kc.shape
    _need(Vc, "Vc", torch.bfloat16, (N, H, d), dev)
    _need(Q, "Q", torch.bfloat16, None, dev)
    if Q.dim() != 3 or tuple(Q.shape[1:]) != (H, d) or Q.shape[0] < n:
        raise ValueError("Q must be [>= n, %d, %d], got %s" % (H, d, tuple(Q.shape)))
    return N, H, d


def attention(Q, Kc, Vc, scale=0.0, out=None, n_q=None, workspace=None):
    """jano_attention: softmax(Q K^T * scale) V per head over all N cache rows.
    With a workspace (uint8 on the device, see attention_workspace) the call is
    jano_attention_ws, which may split the keys over workgroups."""
    torch = _torch()
    n = Q.shape[0] if n_q is None else int(n_q)
    N, H, d = _attn_shapes(Q, Kc, Vc, n)
    out = torch.empty((n, H, d), dtype=torch.bfloat16, device=Kc.device) if out is None else out
    _need(out, "out", torch.bfloat16, None, Kc.device)
    if out.shape[0] < n or tuple(out.shape[1:]) != (H, d):
        raise ValueError("out must be [>= n, H, d]")
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, None, Kc.device)
        _check("jano_attention_ws", lib().jano_attention_ws(
            _ptr(Q), n, _ptr(Kc), _ptr(Vc), N, H, d, float(scale), _ptr(out), _ptr(workspace),
            workspace.numel(), _stream(Kc)))
        return out
    _check("jano_attention", lib().jano_attention(_ptr(Q), n, _ptr(Kc), _ptr(Vc), N, H, d,
                                                  float(scale), _ptr(out), _stream(Kc)))
    return out


def attn_step(Q_act, K_new, V_new, idx, Kc, Vc, scale=0.0, out=None, n_act=None, workspace=None):
    """jano_attn_step: scatter the fresh K/V rows into the cache, then
    attention of the active queries against the whole cache. With a workspace
    the call is jano_attn_step_ws (keys may be split over workgroups)."""
    torch = _torch()
    n = idx.numel() if n_act is None else int(n_act)
    N, H, d = _attn_shapes(Q_act, Kc, Vc, n)
    dev = Kc.device
    for name, t in (("K_new", K_new), ("V_new", V_new)):
        _need(t, name, torch.bfloat16, None, dev)
        if t.dim() != 3 or tuple(t.shape[1:]) != (H, d) or t.shape[0] < n:
            raise ValueError("%s must be [>= n_act, %d, %d]" % (name, H, d))
    _need(idx, "idx", torch.int32, None, dev)
    if n > idx.numel():
        raise ValueError("n_act exceeds idx length")
    out = torch.empty((n, H, d), dtype=torch.bfloat16, device=dev) if out is None else out
    _need(out, "out", torch.bfloat16, None, dev)
    if out.shape[0] < n or tuple(out.shape[1:]) != (H, d):
        raise ValueError("out must be [>= n_act, H, d]")
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, None, dev)
        _check("jano_attn_step_ws", lib().jano_attn_step_ws(
            _ptr(Q_act), _ptr(K_new), _ptr(V_new), _ptr(idx), n, _ptr(Kc), _ptr(Vc), N, H, d,
            float(scale), _ptr(out), _ptr(workspace), workspace.numel(), _stream(Kc)))
        return out
    _check("jano_attn_step", lib().jano_attn_step(
        _ptr(Q_act), _ptr(K_new), _ptr(V_new), _ptr(idx), n, _ptr(Kc), _ptr(Vc), N, H, d,
        float(scale), _ptr(out), _stream(Kc)))
    return out


def concat_kv(K_new, V_new, Kc, Vc, frozen_idx, n_act=None, n_frozen=None, Kcat=None, Vcat=None):
    """jano_concat_kv: [fresh rows ; cached rows of the frozen tokens] for K
    and V. K_new/V_new [>= n_act, H, d], Kc/Vc [N, H, d] bf16 on device ->
    (Kcat, Vcat) [n_act + n_frozen, H, d]."""
    torch = _torch()
    _need(Kc, "Kc", torch.bfloat16)
    if Kc.dim() != 3:
        raise ValueError("Kc must be [N, H, d]")
    N, H, d = Kc.shape
    dev = Kc.device
    _need(Vc, "Vc", torch.bfloat16, (N, H, d), dev)
    na = K_new.shape[0] if n_act is None else int(n_act)
    nf = frozen_idx.numel() if n_frozen is None else int(n_frozen)
    for name, t in (("K_new", K_new), ("V_new", V_new)):
        _need(t, name, torch.bfloat16, None, dev)
        if t.dim() != 3 or tuple(t.shape[1:]) != (H, d) or t.shape[0] < na:
            raise ValueError("%s must be [>= n_act, %d, %d]" % (name, H, d))
    _need(frozen_idx, "frozen_idx", torch.int32, None, dev)
    if nf > frozen_idx.numel():
        raise ValueError("n_frozen exceeds frozen_idx length")
    rows = na + nf
    Kcat = torch.empty((rows, H, d), dtype=torch.bfloat16, device=dev) if Kcat is None else Kcat
    Vcat = torch.empty((rows, H, d), dtype=torch.bfloat16, device=dev) if Vcat is None else Vcat
    for name, t in (("Kcat", Kcat), ("Vcat", Vcat)):
        _need(t, name, torch.bfloat16, None, dev)
        if t.dim() != 3 or tuple(t.shape[1:]) != (H, d) or t.shape[0] < rows:
            raise ValueError("%s must be [>= n_act + n_frozen, %d, %d]" % (name, H, d))
    _check("jano_concat_kv", lib().jano_concat_kv(
        _ptr(K_new), _ptr(V_new), na, _ptr(Kc), _ptr(Vc), _ptr(frozen_idx), nf, _ptr(Kcat),
        _ptr(Vcat), H * d, _stream(Kc)))
    return Kcat, Vcat


def qkv_proj(X, idx, Wqkv, H, d, spec: GridSpec = None, rope_base=10000.0, n_act=None, out=None):
    """jano_qkv_proj: X bf16 [N, Dm], idx int32, Wqkv bf16 [3*H*d, Dm] on
    device -> (Q, K_new, V_new) bf16 [n_act, H, d]; rotary encoding on Q and
    K when spec is given and rope_base > 0."""
    torch = _torch()
    _need(X, "X", torch.bfloat16)
    if X.dim() != 2:
        raise ValueError("X must be [N, Dm]")
    N, Dm = X.shape
    dev = X.device
    _need(Wqkv, "Wqkv", torch.bfloat16, (3 * H * d, Dm), dev)
    _need(idx, "idx", torch.int32, None, dev)
    n = idx.numel() if n_act is None else int(n_act)
    if n > idx.numel():
        raise ValueError("n_act exceeds idx length")
    if out is None:
        out = tuple(torch.empty((n, H, d), dtype=torch.bfloat16, device=dev) for _ in range(3))
    for name, t in zip(("Q", "K_new", "V_new"), out):
        _need(t, name, torch.bfloat16, None, dev)
        if t.dim() != 3 or tuple(t.shape[1:]) != (H, d) or t.shape[0] < n:
            raise ValueError("%s must be [>= n_act, %d, %d]" % (name, H, d))
    gp_ = ctypes.byref(spec.c()) if spec is not None else None
    _check("jano_qkv_proj", lib().jano_qkv_proj(
        _ptr(X), N, Dm, _ptr(idx), n, _ptr(Wqkv), int(H), int(d), gp_,
        float(rope_base if spec is not None else 0.0), _ptr(out[0]), _ptr(out[1]), _ptr(out[2]),
        _stream(X)))
    return out


def writeback_step(out_act, idx, out_full, x, dt, n_act=None):
    """jano_writeback_step: out_full[idx] = out_act (bf16 rows), then
    x += dt * out_full for every token (x fp32 [N, P], updated in place)."""
    torch = _torch()
    _need(out_full, "out_full", torch.bfloat16)
    if out_full.dim() != 2:
        raise ValueError("out_full must be [N, P]")
    N, P = out_full.shape
    dev = out_full.device
    _need(x, "x", torch.float32, (N, P), dev)
    n = idx.numel() if n_act is None else int(n_act)
    _need(idx, "idx", torch.int32, None, dev)
    _need(out_act, "out_act", torch.bfloat16, None, dev)
    if n > idx.numel() or out_act.dim() != 2 or out_act.shape[1] != P or out_act.shape[0] < n:
        raise ValueError("out_act must be [>= n_act, P] and idx hold >= n_act entries")
    _check("jano_writeback_step", lib().jano_writeback_step(
        _ptr(out_act), _ptr(idx), n, _ptr(out_full), _ptr(x), N, P, float(dt), _stream(out_full)))
    return out_full, x


def check_idx(idx, N, n_act=None, flag=None):
    """jano_check_idx -> int32 device flag (0 valid, JANO_E_RANGE otherwise)."""
    torch = _torch()
    _need(idx, "idx", torch.int32)
    n = idx.numel() if n_act is None else int(n_act)
    flag = torch.empty(1, dtype=torch.int32, device=idx.device) if flag is None else flag
    _need(flag, "flag", torch.int32, (1,), idx.device)
    _check("jano_check_idx", lib().jano_check_idx(_ptr(idx), n, int(N), _ptr(flag), _stream(idx)))
    return flag
