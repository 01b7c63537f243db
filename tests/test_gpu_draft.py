"""GPU parity of pe_draft_forward and pe_accept against the CPU oracle.

Every call goes through the C ABI (libpeagle.so via ctypes).  Small shapes
span several weight tiles, several KV tiles and splits, ragged context
lengths and the edge cases of the block (K = 1, K = 16, empty context,
N = 0, 64 activation rows).
"""
import itertools

import numpy as np
import pytest
import torch

from drafting_eagle_draft_amd import runner, synth
from oracle import peagle_oracle as po
from tests.gpu_util import check_parity, log, oracle_logits, run_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from drafting_eagle_draft_amd import binding
    binding.load()


def small_bf16(name="small_bf16", **kw):
    base = dict(name=name, seed=2001, hidden=512, n_layers=2, n_q_heads=8, n_kv_heads=2,
                head_dim=64, intermediate=768, vocab=8192 + 48, K=8, dtype="bf16", batch=2, ctx=0,
                ctx_range=(50, 400))
    base.update(kw)
    return synth.DrafterShape(**base)


# ---------------------------------------------------------------- accept


def test_accept_exhaustive():
    for K in list(range(1, 9)) + [16]:
        if K <= 8:
            pats = np.array(list(itertools.product([0, 1], repeat=K)), dtype=bool)
        else:
            pats = np.random.default_rng(K).random((512, K)) < 0.8
        B = len(pats)
        draft = (np.arange(B * K).reshape(B, K) % 1000).astype(np.int32)
        target = np.where(pats, draft, draft + 1).astype(np.int32)
        target = np.concatenate([target, np.full((B, 1), 9, np.int32)], axis=1)
        alen, toks = runner.accept(draft, target)
        ralen, rtoks = po.accept(draft, target)
        np.testing.assert_array_equal(alen, ralen)
        np.testing.assert_array_equal(toks, rtoks)
        alen2, none = runner.accept(draft, target, with_tokens=False)
        np.testing.assert_array_equal(alen2, ralen)
        assert none is None


def test_accept_planted_table_rates():
    B, K, V = 4096, 8, 201088
    rng = np.random.default_rng(0)
    drafts = rng.integers(0, V, (B, K)).astype(np.int32)
    target, a = synth.planted_targets(drafts, V, seed=3)
    alen, toks = runner.accept(drafts, target)
    np.testing.assert_array_equal(alen, a)
    ralen, rtoks = po.accept(drafts, target)
    np.testing.assert_array_equal(toks, rtoks)


# ---------------------------------------------------------------- fp32 tiny


def test_tiny_f32_workload():
    cfg = synth.config("tiny_f32")
    w = synth.drafter_weights(cfg)
    log("tiny_f32 default inputs")
    run_case(cfg, w, synth.decode_inputs(cfg))


@pytest.mark.parametrize("B,K,ctx,N", [
    (1, 4, [37], 1),          # ragged single tile
    (3, 4, [0, 17, 64], 1),   # empty context, partial tiles
    (1, 1, [64], 1),          # K = 1: plain EAGLE-3 next-token step
    (2, 16, [5, 63], 1),      # K = 16, 32 rows
    (4, 16, [64, 1, 33, 60], 1),  # 64 rows (four MFMA column blocks)
    (2, 4, [10, 20], 0),      # N = 0: fusion, final norm, LM head
])
def test_tiny_f32_variants(B, K, ctx, N):
    cfg = synth.config("tiny_f32")
    w = synth.drafter_weights(cfg, gain_jitter=0.1)
    inp = synth.decode_inputs(cfg, batch=B, ctx_lens=ctx, K=K, ctx_stride=64, tag=f"v{B}{K}")
    log(f"tiny_f32 B={B} K={K} ctx={ctx} N={N}")
    run_case(cfg, w, inp, N=N)


def test_k1_matches_eagle3_step():
    cfg = synth.config("tiny_f32")
    w = synth.drafter_weights(cfg, gain_jitter=0.1)
    inp = synth.decode_inputs(cfg, batch=2, ctx_lens=[64, 9], K=1, tag="e3")
    d = runner.Drafter(cfg, w)
    draft, logits = runner.draft_forward(d, inp, want_logits=True)
    d.close()
    for b in range(2):
        wb = dict(w, embed_rows=w["embed"][inp["token_ids"][b:b + 1]])
        ref = po.eagle3_step(wb, cfg, inp["hidden3"][b], inp["token_ids"][b],
                             int(inp["ctx_lens"][b]), [k[b] for k in inp["k_cache"]],
                             [v[b] for v in inp["v_cache"]])
        assert np.max(np.abs(logits[b, 0] - ref)) < 1e-3


# ---------------------------------------------------------------- bf16 small


@pytest.mark.parametrize("kw", [
    dict(),                                                   # hd 64, G 4
    dict(name="small_bf16_hd128", n_q_heads=8, n_kv_heads=2, head_dim=128, seed=2002),
    dict(name="small_bf16_g8", n_q_heads=16, n_kv_heads=2, head_dim=64, seed=2003, batch=3),
    # Hidden 2048: fc's contraction (3 x 2048) is split over two workgroup
    # columns, so the shared row h_shared goes through the split-K instance;
    # the LM head's 515 strips give its workgroups two or three strips each.
    dict(name="small_bf16_h2048", hidden=2048, n_layers=1, n_q_heads=32, n_kv_heads=4, head_dim=64,
         intermediate=2048, seed=2007),
])
def test_bf16_small(kw):
    cfg = small_bf16(**kw)
    w = synth.drafter_weights(cfg, gain_jitter=0.1)
    inp = synth.decode_inputs(cfg)
    log(f"{cfg.name} ctx={inp['ctx_lens'].tolist()} stride={inp['ctx_stride']}")
    run_case(cfg, w, inp)


@pytest.mark.parametrize("kw", [
    dict(name="small_bf16_straddle"),
    dict(name="small_bf16_straddle_hd128", n_q_heads=8, n_kv_heads=2, head_dim=128, seed=2006),
])
def test_bf16_block_keys_across_splits(kw):
    # With a 256-position cache the attention splits hold 64 keys each.  The
    # contexts put the K = 8 block keys across a split boundary (60: keys
    # 60..67; 250: keys 250..257), at the start of a split with no cached keys
    # (128), and alone (empty context).
    cfg = small_bf16(**kw)
    w = synth.drafter_weights(cfg, gain_jitter=0.1)
    inp = synth.decode_inputs(cfg, batch=4, ctx_lens=[60, 128, 0, 250], ctx_stride=256, tag="straddle")
    log(f"{cfg.name} ctx={inp['ctx_lens'].tolist()} stride={inp['ctx_stride']}")
    run_case(cfg, w, inp)


def test_bf16_small_k16_wide_group():
    # K * G = 128 query rows per kv head: two 64-row query partitions.
    cfg = small_bf16(name="small_bf16_k16", n_q_heads=16, n_kv_heads=2, seed=2004, K=16, batch=2)
    w = synth.drafter_weights(cfg, gain_jitter=0.1)
    inp = synth.decode_inputs(cfg)
    run_case(cfg, w, inp)


def test_logits_off_and_repeat_are_identical():
    cfg = small_bf16(name="small_bf16_rep", seed=2005)
    w = synth.drafter_weights(cfg)
    inp = synth.decode_inputs(cfg)
    d = runner.Drafter(cfg, w)
    buf = runner.DecodeBuffers(d, inp, want_logits=True)
    outs = []
    for _ in range(20):  # repeat-run bit identity over 20 runs: fixed reduction orders
        buf.launch(d)
        torch.cuda.synchronize()
        outs.append((buf.draft.cpu().numpy().copy(), buf.logits.cpu().numpy().copy()))
    for dr, lg in outs[1:]:
        np.testing.assert_array_equal(dr, outs[0][0])
        np.testing.assert_array_equal(lg, outs[0][1])
    nolog = runner.DecodeBuffers(d, inp, want_logits=False)
    nolog.launch(d)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(nolog.draft.cpu().numpy(), outs[0][0])
    d.close()


def test_graph_replays_equal_eager():
    """The forward captured once in a hipGraph and replayed, with eager
    forwards and synchronisations between the replays: every replay equals
    the eager result bit for bit (the library records only kernel launches,
    no memset or copy nodes)."""
    cfg = small_bf16(name="small_bf16_graph", seed=2006)
    w = synth.drafter_weights(cfg)
    inp = synth.decode_inputs(cfg)
    d = runner.Drafter(cfg, w)
    buf = runner.DecodeBuffers(d, inp, want_logits=True)
    buf.launch(d)
    torch.cuda.synchronize()
    ref_d, ref_l = buf.draft.clone(), buf.logits.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        buf.launch(d)
    torch.cuda.current_stream().wait_stream(s)
    with torch.cuda.graph(g):
        buf.launch(d)
    for rep in range(5):
        buf.draft.fill_(-1)
        buf.logits.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(buf.draft, ref_d), rep
        assert torch.equal(buf.logits.view(torch.int32), ref_l.view(torch.int32)), rep
        buf.launch(d)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(buf.draft, ref_d)
    del g
    d.close()
