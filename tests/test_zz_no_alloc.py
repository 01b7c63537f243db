"""GPU test of pe_draft_forward_noalloc, the forward that allocates nothing
(its workspace is the library's per-device scratch array).

Two calls in a row through the C ABI, the second with a smaller input, each
compared bit for bit with pe_draft_forward on a caller-owned workspace (same
kernels, same arithmetic) and against the CPU oracle under the parity rule;
then a shape whose workspace exceeds the scratch array is rejected with
PE_ERR_UNSUPPORTED before anything is launched.
"""
import numpy as np
import pytest
import torch

from drafting_eagle_draft_amd import binding as pe
from drafting_eagle_draft_amd import runner, synth
from tests.gpu_util import check_parity, log, oracle_logits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pe.load()


def _cfg(**kw):
    base = dict(name="noalloc_bf16", seed=2101, hidden=512, n_layers=2, n_q_heads=8, n_kv_heads=2,
                head_dim=64, intermediate=768, vocab=8192 + 48, K=8, dtype="bf16", batch=2, ctx=0,
                ctx_range=(50, 400))
    base.update(kw)
    return synth.DrafterShape(**base)


def _both(d, inp):
    """(draft, logits) of the workspace forward and of the allocation-free one."""
    buf = runner.DecodeBuffers(d, inp, want_logits=True)
    buf.launch(d)
    torch.cuda.synchronize()
    ref = (buf.draft.cpu().numpy().copy(), buf.logits.cpu().numpy().copy())
    buf.draft.fill_(-1)
    buf.logits.fill_(float("nan"))
    pe.pe_draft_forward_noalloc(
        d.handle, buf.N, buf.B, buf.K, buf.hidden3.data_ptr(), buf.token_ids.data_ptr(),
        buf.mask_emb.data_ptr(), buf.h_shared.data_ptr(), buf.ctx_lens.data_ptr(), buf.ctx_stride,
        [t.data_ptr() for t in buf.k_cache], [t.data_ptr() for t in buf.v_cache],
        buf.draft.data_ptr(), buf.logits.data_ptr(), runner.stream_handle())
    torch.cuda.synchronize()
    return ref, (buf.draft.cpu().numpy(), buf.logits.cpu().numpy())


def test_noalloc_matches_workspace_forward_twice():
    cfg = _cfg()
    w = synth.drafter_weights(cfg, gain_jitter=0.1)
    d = runner.Drafter(cfg, w)
    try:
        # First call: B = 2, K = 8, ragged contexts up to 400.
        inp1 = synth.decode_inputs(cfg, batch=2, K=8, tag="noalloc1")
        log(f"noalloc call 1: B=2 K=8 ctx={list(inp1['ctx_lens'])}")
        (da, la), (db, lb) = _both(d, inp1)
        np.testing.assert_array_equal(db, da)
        np.testing.assert_array_equal(lb.view(np.uint32), la.view(np.uint32))
        check_parity(cfg, oracle_logits(cfg, w, inp1), db, lb)
        # Second call, smaller: B = 1, K = 4, a shorter context and stride.
        inp2 = synth.decode_inputs(cfg, batch=1, K=4, ctx_lens=[73], ctx_stride=128, tag="noalloc2")
        log("noalloc call 2: B=1 K=4 ctx=[73]")
        (da, la), (db, lb) = _both(d, inp2)
        np.testing.assert_array_equal(db, da)
        np.testing.assert_array_equal(lb.view(np.uint32), la.view(np.uint32))
        check_parity(cfg, oracle_logits(cfg, w, inp2), db, lb)
    finally:
        d.close()


def test_noalloc_rejects_shapes_beyond_the_scratch():
    # head_dim 128, B = 8, a 200000-position stride: the attention split
    # partials (64 splits x 16 (sequence, kv head) pairs x 33 KB) alone exceed
    # the 32 MiB array.  Every buffer is sized for the shape, so nothing could
    # read out of bounds even if a launch happened.
    cfg = _cfg(name="noalloc_big", hidden=512, n_layers=1, n_q_heads=4, n_kv_heads=2, head_dim=128)
    w = synth.drafter_weights(cfg)
    d = runner.Drafter(cfg, w)
    try:
        B, K, C = 8, 8, 200000
        ws_bytes = pe.pe_draft_workspace_size(d.handle, B, K, C)
        assert ws_bytes > pe.PE_NOALLOC_SCRATCH_BYTES
        dev = d.device
        hidden3 = torch.zeros((B, 3 * cfg.hidden), dtype=torch.bfloat16, device=dev)
        tok = torch.zeros(B, dtype=torch.int32, device=dev)
        vec = torch.zeros(3 * cfg.hidden, dtype=torch.bfloat16, device=dev)
        ctx = torch.full((B,), 100, dtype=torch.int32, device=dev)
        kc = torch.zeros((B, cfg.n_kv_heads, C, cfg.head_dim), dtype=torch.bfloat16, device=dev)
        vc = torch.zeros_like(kc)
        draft = torch.full((B, K), -7, dtype=torch.int32, device=dev)
        with pytest.raises(pe.PeagleError) as ei:
            pe.pe_draft_forward_noalloc(d.handle, 1, B, K, hidden3.data_ptr(), tok.data_ptr(), vec.data_ptr(),
                                        vec.data_ptr(), ctx.data_ptr(), C, [kc.data_ptr()], [vc.data_ptr()],
                                        draft.data_ptr(), None, runner.stream_handle())
        assert ei.value.status == pe.PE_ERR_UNSUPPORTED and "scratch" in ei.value.message
        torch.cuda.synchronize()
        assert bool((draft == -7).all()), "a rejected call wrote its output"
    finally:
        d.close()
