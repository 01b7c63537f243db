"""Pins of the oracle's cache extension (depth-0 rows appended to the
drafter cache) and of the autoregressive EAGLE-3 chain built on it.

- T rows in one block equal T one-row steps, each appending its keys and
  values before the next (the causal depth-0 context of "Speeding LLM
  inference with P-EAGLE in vLLM Speculators", "Flex-attention mask").
- One target row equals the separately written EAGLE-3 step.
- A one-step chain equals the parallel drafter with K = 1 ("P-EAGLE: A
  Technical Deep Dive ...", section 2: the NTP position is plain EAGLE
  next-token prediction).
- A two-step chain (token and normalized output fed back) equals a brute
  force written with Python loops over explicit key lists.
"""
import math

import numpy as np

from oracle import peagle_oracle as po
from tests.toy import toy_problem


def _cache_copy(inp, N, extra):
    kc, vc = [], []
    for l in range(N):
        k = np.asarray(inp["k_cache"][l], float)
        v = np.asarray(inp["v_cache"][l], float)
        pad = np.zeros(k.shape[:2] + (extra, k.shape[3]))
        kc.append(np.concatenate([k, pad], axis=2))
        vc.append(np.concatenate([v, pad.copy()], axis=2))
    return kc, vc


def test_extend_block_equals_one_row_steps():
    cfg, w, inp = toy_problem(ctx_lens=[3, 6], tag="ext")
    B, T, N = 2, 3, cfg.n_layers
    rng = np.random.default_rng(5)
    h = rng.standard_normal((B, T, 3 * cfg.hidden))
    ids = rng.integers(0, cfg.vocab, (B, T))
    emb = w["embed"][ids]
    ctx = np.asarray(inp["ctx_lens"])
    lg, z, kn, vn = po.draft_extend(w, cfg, h, "target", emb, ctx, inp["k_cache"], inp["v_cache"])
    kc, vc = _cache_copy(inp, N, T)
    for t in range(T):
        lg1, z1, kn1, vn1 = po.draft_extend(w, cfg, h[:, t:t + 1], "target", emb[:, t:t + 1], ctx + t, kc, vc)
        np.testing.assert_allclose(lg1[:, 0], lg[:, t], rtol=0, atol=1e-10)
        np.testing.assert_allclose(z1[:, 0], z[:, t], rtol=0, atol=1e-12)
        for l in range(N):
            np.testing.assert_allclose(kn1[l][:, :, 0], kn[l][:, :, t], rtol=0, atol=1e-12)
            np.testing.assert_allclose(vn1[l][:, :, 0], vn[l][:, :, t], rtol=0, atol=1e-12)
            for b in range(B):
                kc[l][b, :, ctx[b] + t] = kn1[l][b, :, 0]
                vc[l][b, :, ctx[b] + t] = vn1[l][b, :, 0]


def test_extend_one_target_row_equals_eagle3_step():
    cfg, w, inp = toy_problem(ctx_lens=[4, 6], tag="e3x")
    lg, _, _, _ = po.draft_extend(w, cfg, np.asarray(inp["hidden3"])[:, None], "target",
                                  w["embed_rows"][:, None], inp["ctx_lens"], inp["k_cache"], inp["v_cache"])
    for b in range(2):
        wb = dict(w, embed_rows=w["embed_rows"][b:b + 1])
        ref = po.eagle3_step(wb, cfg, inp["hidden3"][b], inp["token_ids"][b], int(inp["ctx_lens"][b]),
                             [k[b] for k in inp["k_cache"]], [v[b] for v in inp["v_cache"]])
        np.testing.assert_allclose(lg[b, 0], ref, rtol=0, atol=1e-10)


def test_chain_of_one_step_equals_parallel_k1():
    cfg, w, inp = toy_problem(K=1, tag="c1")
    drafts, lg = po.eagle3_chain(w, cfg, inp["hidden3"], inp["token_ids"], inp["ctx_lens"], inp["k_cache"],
                                 inp["v_cache"], 1, lambda ids: w["embed"][ids])
    ref = po.draft_forward(w, cfg, inp["hidden3"], inp["token_ids"], inp["mask_emb"], inp["h_shared"],
                           inp["ctx_lens"], inp["k_cache"], inp["v_cache"], 1)
    np.testing.assert_allclose(lg, ref, rtol=0, atol=1e-10)
    np.testing.assert_array_equal(drafts, po.argmax_lowest(ref))


def _brute_chain(w, cfg, hidden3, tok, C, kcache, vcache, K, feed=None):
    """Two or more EAGLE-3 steps for one sequence with explicit loops; step
    j + 1 takes token feed[j] when feed is given, else step j's argmax."""
    H, nq, nkv, hd = cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim

    def mv(W, v):
        W = np.asarray(W, float)
        return [sum(W[o, i] * v[i] for i in range(len(v))) for o in range(W.shape[0])]

    def norm(v, g):
        r = 1.0 / math.sqrt(sum(t * t for t in v) / len(v) + cfg.rms_eps)
        return [v[i] * r * float(g[i]) for i in range(len(v))]

    def rot(v, pos):
        half = len(v) // 2
        out = list(v)
        for i in range(half):
            a = pos * cfg.rope_theta ** (-2.0 * i / len(v))
            out[i] = v[i] * math.cos(a) - v[i + half] * math.sin(a)
            out[i + half] = v[i + half] * math.cos(a) + v[i] * math.sin(a)
        return out

    keys = [[[list(map(float, kcache[l][g, j])) for j in range(C)] for g in range(nkv)]
            for l in range(cfg.n_layers)]
    vals = [[[list(map(float, vcache[l][g, j])) for j in range(C)] for g in range(nkv)]
            for l in range(cfg.n_layers)]
    e = [float(t) for t in w["embed"][tok]]
    h = mv(w["fc"], [float(t) for t in hidden3])
    x = [e[i] + h[i] for i in range(H)]
    out = []
    for j in range(K):
        pos = C + j
        for l in range(cfg.n_layers):
            lw = w["layers"][l]
            u = norm(x, lw["attn_norm"])
            q, kk, vv = mv(lw["wq"], u), mv(lw["wk"], u), mv(lw["wv"], u)
            for g in range(nkv):
                keys[l][g].append(rot(kk[g * hd:(g + 1) * hd], pos))
                vals[l][g].append(vv[g * hd:(g + 1) * hd])
            o = []
            for hh in range(nq):
                g = hh // (nq // nkv)
                qh = rot(q[hh * hd:(hh + 1) * hd], pos)
                sc = [sum(qh[i] * kv[i] for i in range(hd)) / math.sqrt(hd) for kv in keys[l][g]]
                mx = max(sc)
                ex = [math.exp(t - mx) for t in sc]
                zz = sum(ex)
                o += [sum(ex[m] / zz * vm[i] for m, vm in enumerate(vals[l][g])) for i in range(hd)]
            x = [x[i] + t for i, t in enumerate(mv(lw["wo"], o))]
            u = norm(x, lw["mlp_norm"])
            gt, up = mv(lw["w_gate"], u), mv(lw["w_up"], u)
            x = [x[i] + t for i, t in enumerate(mv(lw["w_down"], [gt[i] / (1 + math.exp(-gt[i])) * up[i]
                                                                   for i in range(len(gt))]))]
        zf = norm(x, w["final_norm"])
        lg = mv(w["lm_head"], zf)
        out.append(lg)
        d = int(np.argmax(lg)) if feed is None else int(feed[j])
        e = [float(t) for t in w["embed"][d]]
        x = [e[i] + zf[i] for i in range(H)]   # the next step's input: E[draft] + normalized output
    return np.array(out)


def test_chain_matches_brute_force_with_feedback():
    cfg, w, inp = toy_problem(ctx_lens=[5, 2], tag="chain")
    K = 3
    drafts, lg = po.eagle3_chain(w, cfg, inp["hidden3"], inp["token_ids"], inp["ctx_lens"], inp["k_cache"],
                                 inp["v_cache"], K, lambda ids: w["embed"][ids])
    for b in range(2):
        ref = _brute_chain(w, cfg, inp["hidden3"][b], int(inp["token_ids"][b]), int(inp["ctx_lens"][b]),
                           [k[b] for k in inp["k_cache"]], [v[b] for v in inp["v_cache"]], K)
        np.testing.assert_allclose(lg[b], ref, rtol=0, atol=1e-9)
        np.testing.assert_array_equal(drafts[b], np.argmax(ref, axis=1))


def test_chain_with_fed_tokens_matches_brute_force():
    """feed_tokens replaces only the token of the next step: the state fed
    back is still the step's own normalized output, and drafts stay argmaxes."""
    cfg, w, inp = toy_problem(ctx_lens=[3, 6], tag="feed")
    K = 3
    feed = np.array([[7, 1, 0], [2, 9, 4]], dtype=np.int32) % cfg.vocab
    drafts, lg = po.eagle3_chain(w, cfg, inp["hidden3"], inp["token_ids"], inp["ctx_lens"], inp["k_cache"],
                                 inp["v_cache"], K, lambda ids: w["embed"][ids], feed_tokens=feed)
    for b in range(2):
        ref = _brute_chain(w, cfg, inp["hidden3"][b], int(inp["token_ids"][b]), int(inp["ctx_lens"][b]),
                           [k[b] for k in inp["k_cache"]], [v[b] for v in inp["v_cache"]], K, feed=feed[b])
        np.testing.assert_allclose(lg[b], ref, rtol=0, atol=1e-9)
        np.testing.assert_array_equal(drafts[b], np.argmax(ref, axis=1))
    # the fed tokens differ from the chain's own argmaxes, so steps 1.. differ
    own, own_lg = po.eagle3_chain(w, cfg, inp["hidden3"], inp["token_ids"], inp["ctx_lens"], inp["k_cache"],
                                  inp["v_cache"], K, lambda ids: w["embed"][ids])
    assert not np.array_equal(own[:, :-1], feed[:, :-1])
    np.testing.assert_allclose(lg[:, 0], own_lg[:, 0], rtol=0, atol=0)
    assert np.max(np.abs(lg[:, 1:] - own_lg[:, 1:])) > 1e-6
