"""MI355X-native hot path of Jano's convergence-adaptive DiT generation.

    from token_sparse_attention_block_amd import jano
    scores, levels, counts = jano.analyze(lat, jano.GridSpec.of(cfg))
    idx, n_act = jano.schedule(levels, spec, step)
    out = jano.attn_step(Q_act, K_new, V_new, idx, Kc, Vc)

The kernels live in libjano.so (HIP, gfx950); `jano` is a ctypes binding.
"""
from . import configs, synth  # noqa: F401
