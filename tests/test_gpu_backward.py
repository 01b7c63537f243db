"""GPU parity of the training step (forward, cross-entropy loss, backward)
against the oracle's hand-written, finite-difference-pinned backward,
through the C ABI ("P-EAGLE: A Technical Deep Dive into Parallel
Speculative Decoding", section "Memory and Training Complexity"; paper
notes, sections 3 and 3.2).

Every gradient tensor is compared twice: as max |gpu - oracle| / max
|oracle| (the backward's GEMMs take bf16 operands for bf16 drafters, so
errors scale with each tensor's own magnitude), and element by element,
|gpu - oracle| <= rtol * (|oracle| + rms(oracle)), each entry against its
own magnitude plus the tensor's typical one (the terms a small entry's sum
cancels are of that size), so that no small entry can be wrong unnoticed.
The loss is compared relatively.
Chunked steps (each chunk scored on its own cells with the whole sequence's
scale) must add up to the whole step.
"""
import numpy as np
import pytest
import torch

from drafting_eagle_draft_amd import runner, synth
from oracle import peagle_oracle as po
from tests.gpu_util import log

pytestmark = pytest.mark.gpu

# max |gpu - oracle| / max |oracle| per gradient tensor
# (fp32: accumulation order only; bf16: about five chained roundings of GEMM
# operands at 2^-9 each -- dlogits, dx, dout, dS/P, dqkv -- with room 2x)
GRAD_TOL = {"f32": 1e-4, "bf16": 2e-2}
# |gpu - oracle| <= ELEM_TOL * (|oracle| + rms(oracle)) per entry.  bf16: the
# same five stages, each rounding both operands of a GEMM (2 * 2^-9 per
# product), as a random-sign error of about 2^-8 * rms per stage: a standard
# deviation of sqrt(5) * 2^-8 * rms, and the largest of up to ~10^6 entries
# within 5 of them -- 5 * sqrt(5) * 2^-8 = 0.044, taken as 0.05.
ELEM_TOL = {"f32": 1e-4, "bf16": 5e-2}
LOSS_TOL = {"f32": 1e-5, "bf16": 5e-3}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from drafting_eagle_draft_amd import binding
    binding.load()


def train_small(name="bwd_small", **kw):
    base = dict(name=name, seed=4001, hidden=512, n_layers=2, n_q_heads=8, n_kv_heads=2,
                head_dim=64, intermediate=768, vocab=8192 + 48, K=8, dtype="bf16", seq_len=160,
                n_max=256)
    base.update(kw)
    return synth.DrafterShape(**base)


def _labels(cfg, n, seed):
    rng = np.random.default_rng(seed)
    lab = rng.integers(0, cfg.vocab, n).astype(np.int32)
    lab[rng.random(n) < 0.15] = -1
    lab[-1] = -1   # no token after the last position
    return lab


def _compare(cfg, got, ref, gl, rl, tag):
    tol, etol = GRAD_TOL[cfg.dtype], ELEM_TOL[cfg.dtype]
    worst, elem = {}, {}
    def one(name, a, b):
        a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
        den = max(float(np.max(np.abs(b))), 1e-30)
        worst[name] = float(np.max(np.abs(a - b))) / den
        scale = np.abs(b) + max(float(np.sqrt(np.mean(b * b))), 1e-30)
        elem[name] = float(np.max(np.abs(a - b) / scale))
    for k in ("fc", "final_norm", "lm_head", "mask_emb", "h_shared", "embed_rows"):
        one(k, got[k], ref[k])
    for l in range(len(ref["layers"])):
        for k, v in ref["layers"][l].items():
            one(f"L{l}.{k}", got["layers"][l][k], v)
    rel_loss = abs(gl - rl) / max(abs(rl), 1e-30)
    top = sorted(worst.items(), key=lambda kv: -kv[1])[:4]
    log(f"  {tag}: loss {gl:.6f} vs {rl:.6f} (rel {rel_loss:.2e}); worst grads {top}")
    assert rel_loss <= LOSS_TOL[cfg.dtype]
    top_e = sorted(elem.items(), key=lambda kv: -kv[1])[:3]
    log(f"  {tag}: worst element-wise {top_e}")
    bad = {k: v for k, v in worst.items() if not v <= tol}
    assert not bad, bad
    bad = {k: v for k, v in elem.items() if not v <= etol}
    assert not bad, bad


def _oracle(cfg, w, inp, rows, K, labels, N=None):
    wr = dict(w, embed_rows=w["embed"][inp["token_ids"]])
    return po.train_loss_grads(wr, cfg, inp["hidden3"], inp["token_ids"], inp["mask_emb"], inp["h_shared"],
                               rows, K, labels, N=N)


def _layout(cfg, n, K, r=0.8, tag=""):
    U = synth.cod_uniforms(cfg, n, K, tag=tag)
    return po.cod_rows(po.cod_keep(n, K, U, r=r, floor=0.2))


def _run(cfg, w, inp, rows, K, labels, N=None, S=None, n_max=None):
    d = runner.Drafter(cfg, w, backward=True)
    mask = runner.TrainMask(n_max or len(inp["token_ids"]), K)
    n = len(inp["token_ids"])
    if S is None:
        st = runner.TrainStep(d, mask, inp, rows, labels, N=N)
        st.launch(d, mask)
        grads, loss = st.grads.numpy(), float(st.loss.cpu()[0])
    else:
        from drafting_eagle_draft_amd import binding as pe
        scored = int(np.sum(labels[rows // K] >= 0))
        grads = runner.Grads(cfg, n, N)
        loss = 0.0
        for s in range(S):
            cells, lead, _, nc = pe.pe_partition_chunk(n, K, S, s, rows)
            st = runner.TrainStep(d, mask, inp, cells, labels, N=N, n_lead=lead, n=nc, loss_scale=1.0 / scored,
                                  grads=grads)
            st.launch(d, mask)
            torch.cuda.synchronize()
            loss += float(st.loss.cpu()[0])
            del st
        grads = grads.numpy()
    mask.close()
    d.close()
    return loss, grads


@pytest.mark.parametrize("n,K,N", [(40, 4, 1), (70, 8, 1), (23, 1, 1), (30, 4, 0)])
def test_step_tiny_f32(n, K, N):
    cfg = synth.config("tiny_f32")
    w = synth.drafter_weights(cfg, gain_jitter=0.1)
    inp = synth.train_inputs(cfg, n=n, tag=f"b{n}_{K}")
    rows = _layout(cfg, n, K, tag=f"b{n}_{K}")
    labels = _labels(cfg, n, n + K)
    loss, grads = _run(cfg, w, inp, rows, K, labels, N=N, n_max=n + 3)
    rl, rg = _oracle(cfg, w, inp, rows, K, labels, N=N)
    _compare(cfg, grads, rg, loss, rl, f"tiny_f32 n={n} K={K} N={N} L={len(rows)}")


def test_step_bf16_small():
    cfg = train_small()
    w = synth.drafter_weights(cfg, gain_jitter=0.1)
    inp = synth.train_inputs(cfg)
    rows = _layout(cfg, cfg.seq_len, cfg.K)
    labels = _labels(cfg, cfg.seq_len, 7)
    loss, grads = _run(cfg, w, inp, rows, cfg.K, labels, n_max=cfg.n_max)
    rl, rg = _oracle(cfg, w, inp, rows, cfg.K, labels)
    _compare(cfg, grads, rg, loss, rl, f"{cfg.name} n={cfg.seq_len} L={len(rows)}")


def test_step_bf16_hd128_g4():
    cfg = train_small(name="bwd_small_hd128", seed=4002, head_dim=128, n_q_heads=8, n_kv_heads=2,
                      n_layers=1, seq_len=100)
    w = synth.drafter_weights(cfg, gain_jitter=0.1)
    inp = synth.train_inputs(cfg)
    rows = _layout(cfg, cfg.seq_len, cfg.K)
    labels = _labels(cfg, cfg.seq_len, 8)
    loss, grads = _run(cfg, w, inp, rows, cfg.K, labels, n_max=cfg.n_max)
    rl, rg = _oracle(cfg, w, inp, rows, cfg.K, labels)
    _compare(cfg, grads, rg, loss, rl, f"{cfg.name} n={cfg.seq_len} L={len(rows)}")


def test_step_bf16_wide_tiles():
    """Hidden 640 (40 strips of 16 columns): the plain-store and accumulate
    GEMMs whose output is hidden wide take 20-strip tiles (2 tiles of 320
    columns instead of 2.5 of 256), in the forward and the backward."""
    cfg = train_small(name="bwd_small_h640", seed=4003, hidden=640, n_layers=1, seq_len=120)
    w = synth.drafter_weights(cfg, gain_jitter=0.1)
    inp = synth.train_inputs(cfg)
    rows = _layout(cfg, cfg.seq_len, cfg.K)
    labels = _labels(cfg, cfg.seq_len, 9)
    loss, grads = _run(cfg, w, inp, rows, cfg.K, labels, n_max=cfg.n_max)
    rl, rg = _oracle(cfg, w, inp, rows, cfg.K, labels)
    _compare(cfg, grads, rg, loss, rl, f"{cfg.name} n={cfg.seq_len} L={len(rows)}")


def test_step_f32_wide_tiles():
    """fp32 with hidden 320 (20 strips: one 20-strip tile instead of two of 16)."""
    cfg = synth.config("tiny_f32", hidden=320)
    w = synth.drafter_weights(cfg, gain_jitter=0.1)
    n, K = 44, 4
    inp = synth.train_inputs(cfg, n=n, tag="bwide")
    rows = _layout(cfg, n, K, tag="bwide")
    labels = _labels(cfg, n, 5)
    loss, grads = _run(cfg, w, inp, rows, K, labels, n_max=n)
    rl, rg = _oracle(cfg, w, inp, rows, K, labels)
    _compare(cfg, grads, rg, loss, rl, f"tiny_f32 hidden 320 n={n} K={K} L={len(rows)}")


@pytest.mark.parametrize("S", [2, 3])
def test_chunked_steps_accumulate_to_whole(S):
    cfg = synth.config("tiny_f32")
    w = synth.drafter_weights(cfg, gain_jitter=0.1)
    n, K = 50, 4
    inp = synth.train_inputs(cfg, n=n, tag="bchunk")
    rows = _layout(cfg, n, K, tag="bchunk")
    labels = _labels(cfg, n, 3)
    loss_w, g_w = _run(cfg, w, inp, rows, K, labels, n_max=n)
    loss_c, g_c = _run(cfg, w, inp, rows, K, labels, S=S, n_max=n)
    # the chunked sum against the oracle and against the whole step
    rl, rg = _oracle(cfg, w, inp, rows, K, labels)
    _compare(cfg, g_c, rg, loss_c, rl, f"tiny_f32 n={n} S={S} chunked")
    _compare(cfg, g_c, g_w, loss_c, loss_w, f"tiny_f32 n={n} S={S} chunked vs whole")


@pytest.mark.timeout(600)
def test_step_full_size_chunks_and_loss():
    """The training size (GPT-OSS-20B-shaped layer, n = 8192, K = 8, COD
    r = 0.8, L ~ 34K): the loss equals the cross-entropy of the training
    forward's own logits (computed on the host in fp64), every gradient is
    finite, and two chunks add up to the whole step."""
    cfg = synth.config("train_gptoss20b_n8192_k8")
    n, K = cfg.seq_len, cfg.K
    w = synth.drafter_weights(cfg)
    inp = synth.train_inputs(cfg)
    rows = _layout(cfg, n, K)
    labels = _labels(cfg, n, 11)
    d = runner.Drafter(cfg, w, backward=True)
    mask = runner.TrainMask(cfg.n_max, K)
    # loss from the forward's logits, 512 sampled scored rows at a time
    fwd = runner.TrainBuffers(d, mask, inp, rows, want_argmax=False)
    fwd.launch(d, mask)
    torch.cuda.synchronize()
    lab = torch.from_numpy(labels[rows // K].astype(np.int64)).cuda()
    scored = torch.nonzero(lab >= 0).flatten()
    tot = 0.0
    for i in range(0, scored.numel(), 512):
        idx = scored[i:i + 512]
        lg = fwd.logits[idx].double().cpu()
        tot += float(torch.sum(torch.logsumexp(lg, dim=1) - lg[torch.arange(idx.numel()), lab[idx].cpu()]))
    ref_loss = tot / scored.numel()
    del fwd
    torch.cuda.empty_cache()
    st = runner.TrainStep(d, mask, inp, rows, labels)
    st.launch(d, mask)
    torch.cuda.synchronize()
    loss = float(st.loss.cpu()[0])
    whole = st.grads
    finite = all(bool(torch.isfinite(v).all()) for v in whole.t.values()) and all(
        bool(torch.isfinite(v).all()) for g in whole.layers for v in g.values())
    del st
    torch.cuda.empty_cache()
    from drafting_eagle_draft_amd import binding as pe
    acc = runner.Grads(cfg, n)
    loss_c = 0.0
    for s in range(2):
        cells, lead, _, nc = pe.pe_partition_chunk(n, K, 2, s, rows)
        ch = runner.TrainStep(d, mask, inp, cells, labels, n_lead=lead, n=nc, loss_scale=1.0 / scored.numel(),
                              grads=acc)
        ch.launch(d, mask)
        torch.cuda.synchronize()
        loss_c += float(ch.loss.cpu()[0])
        del ch
        torch.cuda.empty_cache()
    rel = {}
    for k in whole.t:
        rel[k] = float((acc.t[k] - whole.t[k]).abs().max() / whole.t[k].abs().max().clamp_min(1e-30))
    for l, g in enumerate(whole.layers):
        for k in g:
            rel[f"L{l}.{k}"] = float((acc.layers[l][k] - g[k]).abs().max() / g[k].abs().max().clamp_min(1e-30))
    top = sorted(rel.items(), key=lambda kv: -kv[1])[:4]
    log(f"  {cfg.name} L={len(rows)}: loss {loss:.6f} (forward logits {ref_loss:.6f}), chunks {loss_c:.6f}; "
        f"finite {finite}; chunks vs whole worst {top}")
    mask.close()
    d.close()
    assert finite
    assert abs(loss - ref_loss) <= 1e-3 * abs(ref_loss)
    assert abs(loss_c - loss) <= 1e-5 * abs(loss)
    # Each chunk rounds its own share of a cell's data gradient (dq/dk/dv,
    # dx) to bf16 before the weight-gradient GEMMs, the whole step rounds the
    # sum once: the two agree to the bf16 rounding level, not bit for bit.
    assert max(rel.values()) <= 1e-2
