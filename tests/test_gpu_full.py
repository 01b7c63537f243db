"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (same model plan, same workspace, logits requested).

The oracle computes every logit of these decode workloads (B*K rows), so the
comparison is element by element over all B*K*V logits and all draft tokens.
"""
import numpy as np
import pytest
import torch

from drafting_eagle_draft_amd import runner, synth
from oracle import peagle_oracle as po
from tests.gpu_util import log, run_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _accept_check(cfg, draft, ref):
    """Acceptance of the real drafts.

    * planted targets (breaks drawn from the acceptance table of "Speeding
      LLM inference with P-EAGLE in vLLM Speculators", section "Example
      model") and uniform-random targets on [0, V): pe_accept equals the
      oracle's accept on the same drafts, bit for bit;
    * against the oracle's own drafts: for targets planted from the oracle's
      argmax, every sequence whose GPU drafts agree with the oracle's at
      positions k <= min(a_oracle, K - 1) has the oracle's accept length;
      every other sequence differs there only at a position whose top-2
      margin is at most 0.1 (where the parity rule leaves the draft open).
    Returns the number of sequence draws whose accept lengths were compared.
    """
    V = cfg.vocab
    B, K = draft.shape
    tgt, _ = synth.planted_targets(draft, V, seed=11)
    uni = np.random.default_rng(12).integers(0, V, (B, K + 1)).astype(np.int32)
    for target in (tgt, uni):
        alen, toks = runner.accept(draft, target)
        ralen, rtoks = po.accept(draft, target)
        np.testing.assert_array_equal(alen, ralen)
        np.testing.assert_array_equal(toks, rtoks)
    odraft = po.argmax_lowest(ref).astype(np.int32)
    margin = po.top2_margin(ref)
    compared = 0
    for seed in range(13, 33):
        otgt, _ = synth.planted_targets(odraft, V, seed=seed)
        alen, _ = runner.accept(draft, otgt)
        ralen, _ = po.accept(odraft, otgt)
        for b in range(B):
            upto = min(int(ralen[b]), K - 1)
            differ = draft[b, :upto + 1] != odraft[b, :upto + 1]
            if not differ.any():
                assert alen[b] == ralen[b], (b, alen[b], ralen[b])
                compared += 1
            else:
                assert np.all(margin[b, :upto + 1][differ] <= 0.1), (b, seed)
    return compared


@pytest.mark.parametrize("name", ["gptoss20b_k8_ctx4k", "qwen3coder30b_k8_ragged",
                                  "gptoss20b_k8_ctx16k"])
def test_full_workload(name):
    cfg = synth.config(name)
    log(f"{name}: generating weights")
    w = synth.drafter_weights(cfg)
    inp = synth.decode_inputs(cfg)
    log(f"{name}: ctx_lens {inp['ctx_lens'].tolist()} stride {inp['ctx_stride']}")
    stats, draft, logits, ref = run_case(cfg, w, inp)
    assert stats["decided"] >= stats["rows"] // 2
    compared = _accept_check(cfg, draft, ref)
    log(f"{name}: accept lengths compared with the oracle's for {compared} sequence draws")
    assert compared > 0


def test_full_workload_repeat_is_identical():
    """The benchmark workload run 20 times on one set of buffers: drafts and
    all B*K*V logits bit-identical every time."""
    cfg = synth.config("gptoss20b_k8_ctx4k")
    w = synth.drafter_weights(cfg)
    inp = synth.decode_inputs(cfg)
    d = runner.Drafter(cfg, w)
    buf = runner.DecodeBuffers(d, inp, want_logits=True)
    buf.launch(d)
    torch.cuda.synchronize()
    ref_d, ref_l = buf.draft.clone(), buf.logits.clone().view(torch.int32)
    for rep in range(20):
        buf.launch(d)
        torch.cuda.synchronize()
        assert torch.equal(buf.draft, ref_d), rep
        assert torch.equal(buf.logits.view(torch.int32), ref_l), rep
    d.close()
