"""GPU test of the argmax tie rule: ties go to the lowest index ("Speeding
LLM inference with P-EAGLE in vLLM Speculators", section "Flex-attention
mask", and greedy drafting in general: the draft is the argmax of the
logits; the lowest index among equal maxima is this build's reading).

Random weights never tie exactly, so the ties are planted: the LM head is
zero except rows i = 37 and j = V - 5, which hold the same vector u.  Rows
i and j then produce bit-identical logits (same arithmetic, same operands),
and every other logit is exactly zero.  A draft row with z.u > 0 has its
maximum tied between i and j, in different workgroups' strips, and must
pick i; a row with z.u < 0 has its maximum (zero) tied over every other
row of the vocabulary and must pick 0.  Both the decode forward and the
training-shape forward are checked: against the lowest index of the
maximum of the GPU's own logits (every row), and against the oracle where
the oracle's |z.u| exceeds the parity margin.
"""
import numpy as np
import pytest
import torch

from drafting_eagle_draft_amd import runner, synth
from oracle import peagle_oracle as po
from tests.gpu_util import log, oracle_logits

pytestmark = pytest.mark.gpu

I_LOW = 37


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from drafting_eagle_draft_amd import binding
    binding.load()


def _tied_weights(cfg, seed):
    w = synth.drafter_weights(cfg, gain_jitter=0.1)
    V, H = cfg.vocab, cfg.hidden
    u = synth.tensor(seed, "tie_u", (H,), 0.05, dtype=cfg.dtype)
    lm = np.zeros((V, H), dtype=np.float32)
    lm[I_LOW] = u
    lm[V - 5] = u
    w["lm_head"] = lm
    return w


def _lowest_max(logits):
    """Lowest index of the maximum, comparing values (so -0.0 == 0.0)."""
    lg = np.asarray(logits, np.float64)
    return np.argmax(lg == lg.max(axis=-1, keepdims=True), axis=-1)


def _check(drafts, gpu_logits, ref, V):
    drafts = np.asarray(drafts).reshape(-1)
    gl = np.asarray(gpu_logits).reshape(drafts.size, V)
    rf = np.asarray(ref).reshape(drafts.size, V)
    # the planted structure holds on the GPU: the two rows are bit-identical
    assert np.array_equal(gl[:, I_LOW].view(np.uint32), gl[:, V - 5].view(np.uint32))
    np.testing.assert_array_equal(drafts, _lowest_max(gl))
    assert set(np.unique(drafts)) <= {0, I_LOW}
    decided = np.abs(rf[:, I_LOW]) > 0.1
    np.testing.assert_array_equal(drafts[decided], po.argmax_lowest(rf)[decided])
    return {"rows": drafts.size, "to_low_row": int(np.sum(drafts == I_LOW)), "to_zero": int(np.sum(drafts == 0)),
            "decided": int(decided.sum())}


@pytest.mark.parametrize("name", ["tiny_f32", "small_bf16"])
def test_decode_ties_go_to_lowest_index(name):
    if name == "tiny_f32":
        cfg = synth.config("tiny_f32")
        B, K, ctx = 3, 4, [20, 33, 64]
    else:
        cfg = synth.DrafterShape(name="ties_bf16", seed=2301, hidden=512, n_layers=2, n_q_heads=8, n_kv_heads=2,
                                 head_dim=64, intermediate=768, vocab=8192 + 48, K=8, dtype="bf16", batch=4, ctx=0,
                                 ctx_range=(50, 300))
        B, K, ctx = 4, 8, None
    w = _tied_weights(cfg, 77)
    inp = synth.decode_inputs(cfg, batch=B, K=K, ctx_lens=ctx, tag="ties")
    d = runner.Drafter(cfg, w)
    try:
        draft, logits = runner.draft_forward(d, inp, want_logits=True)
    finally:
        d.close()
    ref = oracle_logits(cfg, w, inp)
    stats = _check(draft, logits, ref, cfg.vocab)
    log(f"  {cfg.name} decode ties: {stats}")
    assert stats["to_low_row"] > 0 and stats["to_zero"] > 0, "both kinds of tie must occur"


@pytest.mark.parametrize("name", ["tiny_f32", "small_bf16"])
def test_train_ties_go_to_lowest_index(name):
    if name == "tiny_f32":
        cfg = synth.config("tiny_f32")
    else:
        cfg = synth.DrafterShape(name="ties_bf16t", seed=2302, hidden=512, n_layers=1, n_q_heads=8, n_kv_heads=2,
                                 head_dim=64, intermediate=768, vocab=8192 + 48, K=4, dtype="bf16", seq_len=60,
                                 n_max=64)
    n, K = 40, 4
    w = _tied_weights(cfg, 78)
    inp = synth.train_inputs(cfg, n=n, tag="ties")
    U = synth.cod_uniforms(cfg, n, K, tag="ties")
    rows = po.cod_rows(po.cod_keep(n, K, U, r=0.8, floor=0.2))
    d = runner.Drafter(cfg, w)
    mask = runner.TrainMask(n, K)
    try:
        argmax, logits = runner.train_forward(d, mask, inp, rows)
    finally:
        mask.close()
        d.close()
    wr = dict(w, embed_rows=w["embed"][inp["token_ids"]])
    ref = po.train_forward(wr, cfg, inp["hidden3"], inp["token_ids"], inp["mask_emb"], inp["h_shared"], rows, K)
    stats = _check(argmax, logits, ref, cfg.vocab)
    log(f"  {cfg.name} training ties: {stats}")
    assert stats["to_low_row"] > 0 and stats["to_zero"] > 0, "both kinds of tie must occur"
