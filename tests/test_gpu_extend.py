"""GPU parity of the drafter-cache extension (pe_draft_extend) and of the
autoregressive EAGLE-3 chain built on it, against the oracle's draft_extend
and eagle3_chain, through the C ABI.

Extension: logits, draft tokens, final-norm outputs and the appended cache
rows (rotated keys, values) for target-state and fed-back-state rows, with
and without a position offset; the cache rows before the block stay as they
were.  Chain: every step's logits and draft token, the oracle chain fed the GPU
chain's tokens (a near-tied argmax may go either way; such a token must be
within the tolerance of the maximum), and the one-step chain against the
parallel forward with K = 1.
"""
import numpy as np
import pytest
import torch

from drafting_eagle_draft_amd import binding as pe
from drafting_eagle_draft_amd import runner, synth
from oracle import peagle_oracle as po
from tests.gpu_util import MARGIN, TOL, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pe.load()


def small_bf16(name="ext_small_bf16", **kw):
    base = dict(name=name, seed=2201, hidden=512, n_layers=2, n_q_heads=8, n_kv_heads=2,
                head_dim=64, intermediate=768, vocab=8192 + 48, K=8, dtype="bf16", batch=2, ctx=0,
                ctx_range=(50, 400))
    base.update(kw)
    return synth.DrafterShape(**base)


def _margin(cfg):
    """Top-2 gap beyond which the argmax is decided at this precision."""
    return MARGIN if cfg.dtype == "bf16" else 1e-4


def _embed(cfg, w, ids):
    ids = np.asarray(ids)
    return w["embed"][ids] if "embed" in w else synth.embed_rows(cfg, ids).reshape(ids.shape + (-1,))


def _check_extend(cfg, w, inp, T, kind, pos_offset, seed):
    B, H, N = len(inp["token_ids"]), cfg.hidden, cfg.n_layers
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, cfg.vocab, (B, T)).astype(np.int32)
    if kind == pe.PE_INPUT_TARGET:
        inputs = synth.tensor(cfg.seed, f"ext_in{seed}", (B, T, 3 * H), 1.0, dtype=cfg.dtype)
    else:
        inputs = rng.standard_normal((B, T, H)).astype(np.float32)
    ctx = np.asarray(inp["ctx_lens"])
    d = runner.Drafter(cfg, w)
    dev = d.device
    kc = [runner.cache_with_room(runner.to_device(k, cfg, dev), pos_offset + T) for k in inp["k_cache"]]
    vc = [runner.cache_with_room(runner.to_device(v, cfg, dev), pos_offset + T) for v in inp["v_cache"]]
    before = [k.float().cpu().numpy() for k in kc]
    vbefore = [v.float().cpu().numpy() for v in vc]
    buf = runner.ExtendBuffers(d, inputs, kind, ids, ctx, kc, vc, pos_offset=pos_offset)
    buf.launch(d)
    torch.cuda.synchronize()
    lg, z, dr = buf.logits.cpu().numpy(), buf.z.cpu().numpy(), buf.draft.cpu().numpy()
    kn_gpu = [k.float().cpu().numpy() for k in kc]
    vn_gpu = [v.float().cpu().numpy() for v in vc]
    d.close()
    # oracle: the block sits at P_b = ctx + pos_offset and attends to the
    # cache rows before it as they were before the call
    kcp = [np.asarray(k, np.float64) for k in before]
    vcp = [np.asarray(v, np.float64) for v in vbefore]
    P = ctx + pos_offset
    rlg, rz, rk, rv = po.draft_extend(w, cfg, inputs, "target" if kind == pe.PE_INPUT_TARGET else "drafter",
                                      _embed(cfg, w, ids), P, kcp, vcp)
    tol = TOL[cfg.dtype]
    err = float(np.max(np.abs(lg - rlg)))
    zerr = float(np.max(np.abs(z - rz)))
    # bf16 bounds from the rounding the path applies (unit roundoff u = 2^-9):
    # each bf16-rounded operand stage perturbs the terms an output sums by at
    # most u of their size, so it adds an error of about u * rms(output) with
    # a random sign; s stages give a standard deviation of sqrt(s) * u * rms,
    # and the largest of the ~10^4 entries compared lies within 4.5 of them.
    # A stored value adds its own rounding, u * |value|.  z sits behind fc
    # and five GEMM operands per layer (1 + 5N stages); the appended rows of
    # layer l behind fc, 5 l, the attention norm's operand and their storage.
    u = 2.0 ** -9

    def within(got, ref, stages):
        ref = np.asarray(ref, np.float64)
        rms = float(np.sqrt(np.mean(ref * ref)))
        bound = u * np.abs(ref) + 4.5 * np.sqrt(stages) * u * rms
        return bool(np.all(np.abs(np.asarray(got, np.float64) - ref) <= bound))
    ok = po.top2_margin(rlg) > _margin(cfg)
    mism = int(np.sum(dr[ok] != po.argmax_lowest(rlg)[ok]))
    kerr = 0.0
    kv_ok = True
    for l in range(N):
        for b in range(B):
            got_k = kn_gpu[l][b, :, P[b]:P[b] + T]
            got_v = vn_gpu[l][b, :, P[b]:P[b] + T]
            kerr = max(kerr, float(np.max(np.abs(got_k - rk[l][b]))), float(np.max(np.abs(got_v - rv[l][b]))))
            if cfg.dtype == "bf16":
                kv_ok &= within(got_k, rk[l][b], 3 + 5 * l) and within(got_v, rv[l][b], 3 + 5 * l)
            # rows before the block are untouched
            np.testing.assert_array_equal(kn_gpu[l][b, :, :P[b]], before[l][b, :, :P[b]])
    log(f"  {cfg.name} T={T} kind={kind} off={pos_offset}: logits {err:.3g} z {zerr:.3g} kv {kerr:.3g} "
        f"decided {int(ok.sum())}/{ok.size} mismatches {mism}")
    assert err <= tol and mism == 0
    if cfg.dtype == "f32":
        assert zerr <= tol and kerr <= 1e-3
    else:
        assert within(z, rz, 1 + 5 * N), f"z beyond the bf16 rounding bound ({zerr:.3g})"
        assert kv_ok, f"appended rows beyond the bf16 rounding bound ({kerr:.3g})"


@pytest.mark.parametrize("T,kind,off", [(3, 0, 0), (1, 0, 2), (4, 1, 0), (2, 1, 3)])
def test_extend_tiny_f32(T, kind, off):
    cfg = synth.config("tiny_f32")
    w = synth.drafter_weights(cfg, gain_jitter=0.1)
    inp = synth.decode_inputs(cfg, batch=3, ctx_lens=[0, 17, 40], K=T, ctx_stride=48, tag=f"x{T}{kind}")
    _check_extend(cfg, w, inp, T, kind, off, seed=10 * T + kind)


@pytest.mark.parametrize("T,kind,off", [(8, 0, 0), (1, 1, 5)])
def test_extend_bf16_small(T, kind, off):
    cfg = small_bf16()
    w = synth.drafter_weights(cfg, gain_jitter=0.1)
    inp = synth.decode_inputs(cfg)
    _check_extend(cfg, w, inp, T, kind, off, seed=20 + T)


@pytest.mark.parametrize("T,kind,off", [(8, 0, 0), (1, 1, 3)])
def test_extend_bf16_split_projections(T, kind, off):
    """One GPT-OSS-shaped layer (H 2880, 64q/8kv, hd 64) with I = 4096 and a
    small vocabulary: the planner splits fc, QKV (3 ways), O and down (4
    ways) over K, so every split projection finishes in-kernel, QKV writing
    the appended cache rows from the strip's last workgroup."""
    cfg = small_bf16("ext_split_bf16", seed=2301, hidden=2880, n_layers=1, n_q_heads=64, n_kv_heads=8,
                     intermediate=4096, vocab=8192 + 48)
    w = synth.drafter_weights(cfg, gain_jitter=0.1)
    inp = synth.decode_inputs(cfg)
    _check_extend(cfg, w, inp, T, kind, off, seed=40 + T)


def _check_chain(cfg, w, inp, K):
    d = runner.Drafter(cfg, w)
    ch = runner.Eagle3Chain(d, inp, K, want_logits=True)
    ch.launch(d)
    drafts, logits = ch.result()
    d.close()
    # The oracle follows the GPU chain's tokens, so every step is compared
    # even past a near tie; each GPU token must be the oracle's argmax where
    # that is decided and within the tolerance of the maximum where it is not.
    rd, rl = po.eagle3_chain(w, cfg, inp["hidden3"], inp["token_ids"], inp["ctx_lens"], inp["k_cache"],
                             inp["v_cache"], K, lambda ids: _embed(cfg, w, ids), feed_tokens=drafts)
    tol, margin = TOL[cfg.dtype], _margin(cfg)
    err = float(np.max(np.abs(logits - rl)))
    dec = po.top2_margin(rl) > margin
    picked = np.take_along_axis(rl, drafts[..., None].astype(np.int64), axis=-1)[..., 0]
    log(f"  {cfg.name} chain K={K}: logits {err:.3g}, decided {int(dec.sum())}/{dec.size}")
    assert err <= tol
    assert np.array_equal(drafts[dec], rd[dec])
    assert np.all(picked >= rl.max(axis=-1) - 2 * tol)
    return drafts


def test_chain_tiny_f32():
    cfg = synth.config("tiny_f32")
    w = synth.drafter_weights(cfg, gain_jitter=0.1)
    inp = synth.decode_inputs(cfg, batch=2, ctx_lens=[30, 64], K=6, ctx_stride=64, tag="chain")
    _check_chain(cfg, w, inp, 6)


def test_chain_bf16_small():
    cfg = small_bf16(name="ext_chain_bf16", seed=2202)
    w = synth.drafter_weights(cfg, gain_jitter=0.1)
    inp = synth.decode_inputs(cfg)
    _check_chain(cfg, w, inp, 5)


def test_one_step_chain_equals_parallel_k1():
    cfg = synth.config("tiny_f32")
    w = synth.drafter_weights(cfg, gain_jitter=0.1)
    inp = synth.decode_inputs(cfg, batch=2, ctx_lens=[12, 50], K=1, ctx_stride=64, tag="k1")
    d = runner.Drafter(cfg, w)
    ch = runner.Eagle3Chain(d, inp, 1, want_logits=True)
    ch.launch(d)
    drafts, logits = ch.result()
    pdraft, plogits = runner.draft_forward(d, inp, want_logits=True)
    d.close()
    np.testing.assert_array_equal(drafts, pdraft)
    assert np.max(np.abs(logits - plogits)) < 1e-4
