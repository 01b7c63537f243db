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


def _accept_check(draft):
    # Acceptance of the real drafts against planted and uniform targets.
    V = 201088
    tgt, a = synth.planted_targets(draft, V, seed=11)
    alen, toks = runner.accept(draft, tgt)
    ralen, rtoks = po.accept(draft, tgt)
    np.testing.assert_array_equal(alen, ralen)
    np.testing.assert_array_equal(toks, rtoks)


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
    _accept_check(draft)
