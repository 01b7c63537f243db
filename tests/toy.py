"""Tiny drafter shapes for oracle tests (CPU, float64 in seconds)."""
import numpy as np

from drafting_eagle_draft_amd import synth


def toy_cfg(**kw):
    base = dict(name="toy", seed=77, hidden=32, n_layers=2, n_q_heads=4, n_kv_heads=2,
                head_dim=8, intermediate=48, vocab=29, K=4, dtype="f32", batch=2, ctx=6,
                rope_theta=500000.0)
    base.update(kw)
    return synth.DrafterShape(**base)


def toy_problem(cfg=None, gain_jitter=0.1, ctx_lens=None, batch=None, K=None, tag=""):
    """Weights (with embed_rows filled) and decode inputs for a toy drafter."""
    cfg = cfg or toy_cfg()
    w = synth.drafter_weights(cfg, gain_jitter=gain_jitter)
    # Scale projections up so attention and logits are not all near-uniform.
    for lw in w["layers"]:
        for key in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"):
            lw[key] = lw[key] * np.float32(10.0)
    w["fc"] = w["fc"] * np.float32(5.0)
    w["lm_head"] = w["lm_head"] * np.float32(20.0)
    inp = synth.decode_inputs(cfg, batch=batch, ctx_lens=ctx_lens, K=K, tag=tag)
    w["embed_rows"] = w["embed"][inp["token_ids"]]
    return cfg, w, inp
