"""Argument validation that needs a real model (survey section 5, failure
detection): every call below is rejected with its status before anything
is enqueued, which the test checks by keeping sentinel values in the
outputs and synchronising after each rejected call."""
import numpy as np
import pytest
import torch

from drafting_eagle_draft_amd import binding as pe
from drafting_eagle_draft_amd import runner, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pe.load()


@pytest.fixture(scope="module")
def tiny():
    cfg = synth.config("tiny_f32")
    w = synth.drafter_weights(cfg)
    d = runner.Drafter(cfg, w)
    yield cfg, w, d
    d.close()


def _rejects(code, fn, *args, **kw):
    with pytest.raises(pe.PeagleError) as ei:
        fn(*args, **kw)
    assert ei.value.status == code, (ei.value.status, ei.value.message)
    torch.cuda.synchronize()
    return ei.value.message


def _forward_args(buf, d, **over):
    a = dict(model=d.handle, N=buf.N, B=buf.B, K=buf.K, hidden3=buf.hidden3.data_ptr(),
             token_ids=buf.token_ids.data_ptr(), mask_emb=buf.mask_emb.data_ptr(),
             h_shared=buf.h_shared.data_ptr(), ctx_lens=buf.ctx_lens.data_ptr(), ctx_stride=buf.ctx_stride,
             k_cache=[t.data_ptr() for t in buf.k_cache], v_cache=[t.data_ptr() for t in buf.v_cache],
             draft_out=buf.draft.data_ptr(), logits_out=None, workspace=buf.ws.data_ptr(),
             ws_bytes=buf.ws.numel(), stream=runner.stream_handle())
    a.update(over)
    return list(a.values())


def test_draft_forward_rejections_enqueue_nothing(tiny):
    cfg, w, d = tiny
    inp = synth.decode_inputs(cfg, batch=2, K=4, ctx_lens=[10, 30], tag="err")
    buf = runner.DecodeBuffers(d, inp)
    buf.draft.fill_(-7)
    need = pe.pe_draft_workspace_size(d.handle, buf.B, buf.K, buf.ctx_stride)
    # workspace one byte short, and none at all
    _rejects(pe.PE_ERR_WORKSPACE, pe.pe_draft_forward, *_forward_args(buf, d, ws_bytes=need - 1))
    _rejects(pe.PE_ERR_WORKSPACE, pe.pe_draft_forward, *_forward_args(buf, d, workspace=None))
    # more layers than the model holds
    msg = _rejects(pe.PE_ERR_INVALID_ARGUMENT, pe.pe_draft_forward,
                   *_forward_args(buf, d, N=cfg.n_layers + 1,
                                  k_cache=[buf.k_cache[0].data_ptr()] * (cfg.n_layers + 1),
                                  v_cache=[buf.v_cache[0].data_ptr()] * (cfg.n_layers + 1)))
    assert "n_layers" in msg
    # B*K beyond the 64 activation rows, and K beyond K_MAX
    _rejects(pe.PE_ERR_UNSUPPORTED, pe.pe_draft_forward, *_forward_args(buf, d, B=9, K=8))
    _rejects(pe.PE_ERR_UNSUPPORTED, pe.pe_draft_forward, *_forward_args(buf, d, K=pe.PE_K_MAX + 1))
    # a misaligned device pointer and a missing cache pointer
    _rejects(pe.PE_ERR_INVALID_ARGUMENT, pe.pe_draft_forward, *_forward_args(buf, d, hidden3=buf.hidden3.data_ptr() + 4))
    _rejects(pe.PE_ERR_INVALID_ARGUMENT, pe.pe_draft_forward, *_forward_args(buf, d, k_cache=[0]))
    assert bool((buf.draft == -7).all()), "a rejected call wrote its output"
    # the same buffers run when the arguments are valid
    buf.launch(d)
    torch.cuda.synchronize()
    assert bool((buf.draft >= 0).all())


def test_draft_forward_noalloc_rejections(tiny):
    cfg, w, d = tiny
    inp = synth.decode_inputs(cfg, batch=1, K=4, ctx_lens=[12], tag="err2")
    buf = runner.DecodeBuffers(d, inp)
    buf.draft.fill_(-7)
    args = _forward_args(buf, d, B=9, K=8)
    _rejects(pe.PE_ERR_UNSUPPORTED, pe.pe_draft_forward_noalloc, *(args[:14] + [args[-1]]))
    assert bool((buf.draft == -7).all())


def test_extend_rejections(tiny):
    cfg, w, d = tiny
    B, T = 2, 3
    inp = synth.decode_inputs(cfg, batch=B, K=T, ctx_lens=[5, 9], ctx_stride=32, tag="err3")
    dev = d.device
    kc = [runner.to_device(k, cfg, dev) for k in inp["k_cache"]]
    vc = [runner.to_device(v, cfg, dev) for v in inp["v_cache"]]
    x = torch.zeros((B, T, 3 * cfg.hidden), dtype=torch.float32, device=dev)
    tok = torch.zeros((B, T), dtype=torch.int32, device=dev)
    ctx = torch.tensor([5, 9], dtype=torch.int32, device=dev)
    draft = torch.full((B, T), -7, dtype=torch.int32, device=dev)
    ws = d.workspace(B, T, 32)
    before = [k.clone() for k in kc]

    def call(**over):
        a = dict(model=d.handle, N=1, B=B, T=T, inputs=x.data_ptr(), kind=pe.PE_INPUT_TARGET,
                 tok=tok.data_ptr(), ctx=ctx.data_ptr(), off=0, C=32, kc=[t.data_ptr() for t in kc],
                 vc=[t.data_ptr() for t in vc], draft=draft.data_ptr(), logits=None, z=None,
                 ws=ws.data_ptr(), wsb=ws.numel(), stream=runner.stream_handle())
        a.update(over)
        pe.pe_draft_extend(*a.values())

    _rejects(pe.PE_ERR_INVALID_ARGUMENT, call, kind=7)
    _rejects(pe.PE_ERR_UNSUPPORTED, call, T=pe.PE_K_MAX + 1)
    _rejects(pe.PE_ERR_INVALID_ARGUMENT, call, off=-1)
    _rejects(pe.PE_ERR_WORKSPACE, call, wsb=16)
    assert bool((draft == -7).all())
    for a, b in zip(kc, before):
        assert torch.equal(a, b), "a rejected extension wrote the cache"


def test_train_rejections_enqueue_nothing(tiny):
    cfg, w, d = tiny
    n, K = 24, 4
    inp = synth.train_inputs(cfg, n=n, tag="err4")
    U = synth.cod_uniforms(cfg, n, K, tag="err4")
    rows = pe.pe_cod_rows(n, K, 0.8, 0.2, U.reshape(-1))
    mask = runner.TrainMask(n, K)          # n_max = n
    mask8 = runner.TrainMask(n, 8)         # a mask built for another K
    try:
        buf = runner.TrainBuffers(d, mask, inp, rows)
        buf.argmax.fill_(-7)
        L = len(rows)

        def call(m=mask, **over):
            a = dict(model=d.handle, mask=m.handle, N=buf.N, n=n, K=K, h=buf.hidden3.data_ptr(),
                     tok=buf.token_ids.data_ptr(), me=buf.mask_emb.data_ptr(), hs=buf.h_shared.data_ptr(),
                     rows=buf.rows.data_ptr(), L=L, logits=None, argmax=buf.argmax.data_ptr(),
                     ws=buf.ws.data_ptr(), wsb=buf.ws.numel(), stream=runner.stream_handle())
            a.update(over)
            pe.pe_train_forward(*a.values())

        msg = _rejects(pe.PE_ERR_INVALID_ARGUMENT, call, n=n + 1, L=L)  # n beyond the mask's n_max
        assert "n_max" in msg
        msg = _rejects(pe.PE_ERR_INVALID_ARGUMENT, lambda: call(m=mask8))  # K differs from the mask's
        assert "K=" in msg
        _rejects(pe.PE_ERR_INVALID_ARGUMENT, call, N=cfg.n_layers + 1)
        _rejects(pe.PE_ERR_INVALID_ARGUMENT, call, L=n * K + 1)
        _rejects(pe.PE_ERR_WORKSPACE, call, wsb=16)
        assert bool((buf.argmax == -7).all())
        # a training step on a model without the backward's transposed tiles
        labels = np.arange(n, dtype=np.int32) % cfg.vocab
        st = runner.TrainStep(d, mask, inp, rows, labels)
        st.loss.fill_(-7.0)
        msg = _rejects(pe.PE_ERR_INVALID_ARGUMENT, st.launch, d, mask)
        assert "prepare_backward" in msg
        assert float(st.loss.cpu()[0]) == -7.0
        del st, buf
    finally:
        mask8.close()
        mask.close()
