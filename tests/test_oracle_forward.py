"""Pins of the oracle's decode and training-shape forwards.

Brute force on tiny inputs, the K = 1 reduction to an EAGLE-3 step, prefix
consistency of the block-causal mask, RoPE relative-position invariance and
the equivalence of the cached decode block with training-layout rows.
"""
import math

import numpy as np
import pytest

from oracle import peagle_oracle as po
from tests.toy import toy_cfg, toy_problem


def _brute_forward(w, cfg, inp, K):
    """Definition written with Python loops over explicit key lists."""
    H, nq, nkv, hd = cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    B = len(inp["token_ids"])
    fc = np.asarray(w["fc"], float)

    def mv(W, v):
        W = np.asarray(W, float)
        return [sum(W[o, i] * v[i] for i in range(len(v))) for o in range(W.shape[0])]

    def norm(v, g):
        ms = sum(t * t for t in v) / len(v)
        r = 1.0 / math.sqrt(ms + cfg.rms_eps)
        return [v[i] * r * float(g[i]) for i in range(len(v))]

    def rot(v, pos):
        half = len(v) // 2
        out = list(v)
        for i in range(half):
            ang = pos * cfg.rope_theta ** (-2.0 * i / len(v))
            out[i] = v[i] * math.cos(ang) - v[i + half] * math.sin(ang)
            out[i + half] = v[i + half] * math.cos(ang) + v[i] * math.sin(ang)
        return out

    logits = np.zeros((B, K, cfg.vocab))
    for b in range(B):
        C = int(inp["ctx_lens"][b])
        xs = []
        for k in range(K):
            if k == 0:
                e = [float(t) for t in w["embed_rows"][b]]
                h = mv(fc, [float(t) for t in inp["hidden3"][b]])
            else:
                e = [float(t) for t in inp["mask_emb"]]
                h = mv(fc, [float(t) for t in inp["h_shared"]])
            xs.append([e[i] + h[i] for i in range(H)])
        for l in range(cfg.n_layers):
            lw = w["layers"][l]
            qs, ks, vs = [], [], []
            for k in range(K):
                u = norm(xs[k], lw["attn_norm"])
                q, kk, vv = mv(lw["wq"], u), mv(lw["wk"], u), mv(lw["wv"], u)
                pos = C + k
                qs.append([rot(q[h * hd:(h + 1) * hd], pos) for h in range(nq)])
                ks.append([rot(kk[g * hd:(g + 1) * hd], pos) for g in range(nkv)])
                vs.append([vv[g * hd:(g + 1) * hd] for g in range(nkv)])
            new = []
            for k in range(K):
                o = []
                for h in range(nq):
                    g = h // (nq // nkv)
                    keys = [list(map(float, inp["k_cache"][l][b, g, j])) for j in range(C)]
                    vals = [list(map(float, inp["v_cache"][l][b, g, j])) for j in range(C)]
                    keys += [ks[j][g] for j in range(k + 1)]
                    vals += [vs[j][g] for j in range(k + 1)]
                    sc = [sum(qs[k][h][i] * kv[i] for i in range(hd)) / math.sqrt(hd) for kv in keys]
                    mx = max(sc)
                    ex = [math.exp(t - mx) for t in sc]
                    z = sum(ex)
                    o += [sum(ex[j] / z * vals[j][i] for j in range(len(keys))) for i in range(hd)]
                x1 = [xs[k][i] + t for i, t in enumerate(mv(lw["wo"], o))]
                u = norm(x1, lw["mlp_norm"])
                gt, up = mv(lw["w_gate"], u), mv(lw["w_up"], u)
                hmid = [gt[i] / (1 + math.exp(-gt[i])) * up[i] for i in range(len(gt))]
                new.append([x1[i] + t for i, t in enumerate(mv(lw["w_down"], hmid))])
            xs = new
        for k in range(K):
            logits[b, k] = mv(w["lm_head"], norm(xs[k], w["final_norm"]))
    return logits


def _fwd(cfg, w, inp, K=None, N=None):
    K = inp["K"] if K is None else K
    return po.draft_forward(w, cfg, inp["hidden3"], inp["token_ids"], inp["mask_emb"],
                            inp["h_shared"], inp["ctx_lens"], inp["k_cache"], inp["v_cache"],
                            K, N)


def test_forward_matches_brute_force_tiny():
    cfg = toy_cfg(hidden=16, intermediate=24, vocab=13, K=3, n_layers=2, head_dim=4,
                  n_q_heads=4, n_kv_heads=2)
    cfg, w, inp = toy_problem(cfg, ctx_lens=[3, 5])
    ref = _brute_forward(w, cfg, inp, 3)
    got = _fwd(cfg, w, inp)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-10)


def test_k1_equals_eagle3_step():
    cfg, w, inp = toy_problem(ctx_lens=[6, 2])
    got = _fwd(cfg, w, inp, K=1)
    for b in range(2):
        wb = dict(w, embed_rows=w["embed_rows"][b:b + 1])
        ref = po.eagle3_step(wb, cfg, inp["hidden3"][b], inp["token_ids"][b], int(inp["ctx_lens"][b]),
                             [kc[b] for kc in inp["k_cache"]], [vc[b] for vc in inp["v_cache"]])
        np.testing.assert_allclose(got[b, 0], ref, rtol=1e-11, atol=1e-11)


def test_prefix_consistency_block_causal():
    # Row k never sees rows after it, so the first k+1 rows of a K block equal
    # a (k+1)-row block.
    cfg, w, inp = toy_problem(ctx_lens=[4, 1])
    full = _fwd(cfg, w, inp, K=4)
    for k in range(1, 4):
        np.testing.assert_allclose(_fwd(cfg, w, inp, K=k), full[:, :k], rtol=1e-12, atol=1e-12)
    # Changing a later row's input must change nothing earlier: perturb the
    # mask embedding, which only rows >= 1 use; row 0 must stay fixed.
    inp2 = dict(inp, mask_emb=inp["mask_emb"] + 0.5)
    other = _fwd(cfg, w, inp2, K=4)
    np.testing.assert_allclose(other[:, 0], full[:, 0], rtol=1e-13, atol=1e-13)
    assert np.max(np.abs(other[:, 1:] - full[:, 1:])) > 1e-3


def test_mtp_rows_share_inputs():
    cfg, w, inp = toy_problem()
    x = po.fuse_inputs(w, inp["hidden3"], inp["token_ids"], inp["mask_emb"], inp["h_shared"], 4)
    for b in range(2):
        for k in range(2, 4):
            np.testing.assert_array_equal(x[b, k], x[b, 1])
    assert not np.allclose(x[0, 0], x[0, 1])


def test_rope_shift_invariance_of_forward():
    # Regenerate the cache from pre-rotation keys at positions shifted by s;
    # queries shift with ctx_len, so every score and logit is unchanged.
    cfg, w, inp = toy_problem(ctx_lens=[6, 6])
    pre_k = [np.asarray(k, float) for k in inp["k_cache"]]
    C = inp["k_cache"][0].shape[2]

    def cache_at(offset):
        out = []
        for l in range(cfg.n_layers):
            pos = (np.arange(C) + offset)[None, None, :]
            out.append(po.rope(pre_k[l], pos, cfg.rope_theta))
        return out

    base = dict(inp, k_cache=cache_at(0), ctx_lens=np.array([6, 6]))
    ref = _fwd(cfg, w, base)
    for s in (1, 1000, 77777):
        # Cache rows rotated at j + s and block rows at ctx_len + k + s.
        shifted = dict(inp, k_cache=cache_at(s))
        got = _fwd_with_offset(cfg, w, shifted, s)
        np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-9)


def _fwd_with_offset(cfg, w, inp, s):
    """Forward where the cache and the block both start s positions later."""
    orig = po.rope

    def shifted_rope(a, pos, theta):
        return orig(a, np.asarray(pos, float) + s, theta)

    po.rope = shifted_rope
    try:
        return _fwd(cfg, w, inp)
    finally:
        po.rope = orig


def test_decode_block_equals_training_rows():
    """Decode row d of the block anchored at a equals training row (a+d, d).

    The decode cache is the depth-0 prefill of positions 0..a-1 computed by
    the training forward itself (rotated keys and values of each layer).
    """
    cfg = toy_cfg(K=4, n_layers=2)
    _, w, _ = toy_problem(cfg)
    n, K = 9, 4
    rng = np.random.default_rng(5)
    hidden3 = rng.standard_normal((n, 3 * cfg.hidden))
    tokens = rng.integers(0, cfg.vocab, n)
    mask_emb = rng.standard_normal(cfg.hidden) * 0.5
    h_shared = rng.standard_normal(3 * cfg.hidden)
    w_t = dict(w, embed_rows=w["embed"][tokens])
    full_rows = np.arange(n * K)
    keep = np.array([divmod(r, K)[0] >= divmod(r, K)[1] for r in full_rows])
    rows = full_rows[keep]
    logits_t, kv = po.train_forward(w_t, cfg, hidden3, tokens, mask_emb, h_shared, rows, K,
                                    return_kv=True)
    for a in (0, 3, 5):
        if a + K - 1 >= n:
            continue
        depth0_idx = [int(np.where(rows == p * K)[0][0]) for p in range(a)]
        k_cache = [kv[l][0][depth0_idx].transpose(1, 0, 2)[None] for l in range(cfg.n_layers)]
        v_cache = [kv[l][1][depth0_idx].transpose(1, 0, 2)[None] for l in range(cfg.n_layers)]
        if a == 0:
            k_cache = [np.zeros((1, cfg.n_kv_heads, 1, cfg.head_dim))] * cfg.n_layers
            v_cache = k_cache
        w_d = dict(w, embed_rows=w["embed"][tokens[a:a + 1]])
        dec = po.draft_forward(w_d, cfg, hidden3[a:a + 1], tokens[a:a + 1], mask_emb, h_shared,
                               [a], k_cache, v_cache, K)
        for d in range(K):
            i = int(np.where(rows == (a + d) * K + d)[0][0])
            np.testing.assert_allclose(dec[0, d], logits_t[i], rtol=1e-10, atol=1e-10)


def test_train_forward_row_sampling_matches_full():
    cfg = toy_cfg(K=3, n_layers=1)
    _, w, _ = toy_problem(cfg)
    n, K = 7, 3
    rng = np.random.default_rng(9)
    hidden3 = rng.standard_normal((n, 3 * cfg.hidden))
    tokens = rng.integers(0, cfg.vocab, n)
    w_t = dict(w, embed_rows=w["embed"][tokens])
    keep = po.cod_keep(n, K, rng.random((n, K)), r=0.8)
    rows = po.cod_rows(keep)
    args = (w_t, cfg, hidden3, tokens, rng.standard_normal(cfg.hidden), rng.standard_normal(3 * cfg.hidden), rows, K)
    full = po.train_forward(*args)
    sel = np.array([0, 3, len(rows) - 1])
    np.testing.assert_allclose(po.train_forward(*args, lm_rows=sel), full[sel], rtol=1e-13)
