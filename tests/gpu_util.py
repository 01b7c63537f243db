"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
and the CPU oracle on the same seeded inputs, then compare.

Parity rule: draft tokens equal the oracle's argmax wherever the oracle's
top-2 logit margin exceeds 0.1; logits agree within max-abs 5e-2 for bf16
drafters (bf16 weights and activations, fp32 accumulation) and within 1e-3
for fp32 drafters.
"""
import sys
import time

import numpy as np

from drafting_eagle_draft_amd import runner, synth
from oracle import peagle_oracle as po

MARGIN = 0.1
TOL = {"bf16": 5e-2, "f32": 1e-3}


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def oracle_logits(cfg, w, inp, N=None):
    wr = dict(w)
    if "embed" in w:
        wr["embed_rows"] = w["embed"][inp["token_ids"]]
    else:
        wr["embed_rows"] = synth.embed_rows(cfg, inp["token_ids"])
    return po.draft_forward(wr, cfg, inp["hidden3"], inp["token_ids"], inp["mask_emb"],
                            inp["h_shared"], inp["ctx_lens"], inp["k_cache"], inp["v_cache"],
                            inp["K"], N)


def check_parity(cfg, ref, draft, logits=None, tol=None):
    """Assert the parity rule; returns a dict of statistics."""
    tol = TOL[cfg.dtype] if tol is None else tol
    margin = po.top2_margin(ref)
    ok = margin > MARGIN
    ref_tok = po.argmax_lowest(ref)
    mism = int(np.sum(draft[ok] != ref_tok[ok]))
    stats = {"rows": int(ref.shape[0] * ref.shape[1]), "decided": int(ok.sum()),
             "token_mismatch_decided": mism,
             "token_mismatch_all": int(np.sum(draft != ref_tok))}
    if logits is not None:
        err = np.abs(logits.astype(np.float64) - ref)
        stats["max_abs"] = float(err.max())
        assert stats["max_abs"] <= tol, stats
    assert mism == 0, stats
    assert np.all((draft >= 0) & (draft < cfg.vocab)), "draft ids out of range"
    return stats


def run_case(cfg, w, inp, N=None, want_logits=True, drafter=None):
    """GPU forward plus oracle; returns (stats, draft, logits, ref)."""
    t0 = time.time()
    d = drafter or runner.Drafter(cfg, w)
    draft, logits = runner.draft_forward(d, inp, N=N, want_logits=want_logits)
    t1 = time.time()
    ref = oracle_logits(cfg, w, inp, N)
    t2 = time.time()
    stats = check_parity(cfg, ref, draft, logits)
    log(f"  {cfg.name}: gpu {t1 - t0:.1f}s oracle {t2 - t1:.1f}s {stats}")
    if drafter is None:
        d.close()
    return stats, draft, logits, ref
