"""Shared helpers of the GPU parity tests (host <-> device moves, tolerances).

Tolerances are the ones the parity bar fixes:
  * analyzer scores: |gpu - oracle| <= 1e-5 * |oracle| (exact zeros stay zero)
  * levels, index lists, scatter positions: bit-exact, except blocks whose
    oracle score lies within 1e-5 relative of a level threshold
  * attention: bf16 output vs the oracle, max |diff| <= 2e-2 and
    ||diff||_2 / ||ref||_2 <= 1e-2
"""
import numpy as np

SCORE_RTOL = 1e-5
ATTN_MAX_ABS = 2e-2
ATTN_REL_RMS = 1e-2


def torch():
    import torch as t
    return t


def dev_bf16(bits: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(t.bfloat16).to("cuda")


def host_bits(x) -> np.ndarray:
    t = torch()
    return x.contiguous().view(t.int16).cpu().numpy().view(np.uint16)


def host_bf16_f64(x) -> np.ndarray:
    b = host_bits(x).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def dev(a: np.ndarray):
    return torch().from_numpy(np.ascontiguousarray(a)).to("cuda")


def attn_errors(gpu, ref):
    """gpu: float array [n, H, d]; ref: float64 [n, H, d].
    Returns (max_abs, rel_rms, worst_head_rel_rms)."""
    diff = gpu - ref
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300))
    per_head = [float(np.linalg.norm(diff[:, h]) / max(np.linalg.norm(ref[:, h]), 1e-300))
                for h in range(ref.shape[1])]
    return max_abs, rel, max(per_head) if per_head else 0.0


def assert_attn_close(gpu, ref, what=""):
    max_abs, rel, worst = attn_errors(gpu, ref)
    print("%s attention: max|d|=%.3e rel_rms=%.3e worst_head=%.3e" % (what, max_abs, rel, worst),
          flush=True)
    assert max_abs <= ATTN_MAX_ABS, (what, max_abs)
    assert rel <= ATTN_REL_RMS, (what, rel)


def threshold_band(scores_ref: np.ndarray, static_pm: int, moderate_pm: int) -> np.ndarray:
    """Boolean mask of blocks whose score is within SCORE_RTOL of a level
    threshold (the scores at ranks nS and nSM of the oracle order)."""
    B = scores_ref.shape[0]
    order = np.lexsort((np.arange(B), scores_ref))
    nS = (static_pm * B + 500) // 1000
    nSM = ((static_pm + moderate_pm) * B + 500) // 1000
    band = np.zeros(B, dtype=bool)
    for r in (nS, nSM):
        if 0 <= r < B:
            tau = float(scores_ref[order[r]])
            band |= np.abs(scores_ref.astype(np.float64) - tau) <= SCORE_RTOL * abs(tau)
    return band
