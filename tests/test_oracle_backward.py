"""Pins of the oracle's training loss and gradients (CPU, float64).

The backward is written out by hand in the oracle; here it is checked
against central finite differences of a loss assembled from the oracle's
separately written training forward (train_forward) and a library
log-sum-exp, entry by entry on every parameter tensor; against gradient
accumulation over the chunks of a sequence partition ("P-EAGLE: A Technical
Deep Dive into Parallel Speculative Decoding", section "Memory and Training
Complexity"; paper notes, section 3.2); and on the degenerate cases.
"""
import copy

import numpy as np
import pytest
from scipy.special import logsumexp

from oracle import peagle_oracle as po
from tests.toy import toy_cfg, toy_problem


def _problem(n=7, K=3, N=2, seed=5):
    cfg, w, _ = toy_problem(toy_cfg(n_layers=N, K=K, vocab=23))
    rng = np.random.default_rng(seed)
    w = copy.deepcopy(w)
    for key in ("fc", "final_norm", "lm_head", "embed"):
        w[key] = np.asarray(w[key], np.float64)
    w["layers"] = [{k: np.asarray(v, np.float64) for k, v in lw.items()} for lw in w["layers"]]
    rows = po.cod_rows(po.cod_keep(n, K, rng.random((n, K)), r=0.8))
    hidden3 = rng.standard_normal((n, 3 * cfg.hidden))
    tok = rng.integers(0, cfg.vocab, n)
    w["embed_rows"] = w["embed"][tok].copy()
    mask_emb = rng.standard_normal(cfg.hidden) * 0.3
    h_shared = rng.standard_normal(3 * cfg.hidden)
    labels = rng.integers(0, cfg.vocab, n)
    labels[rng.random(n) < 0.2] = -1
    return cfg, w, rows, hidden3, tok, mask_emb, h_shared, labels


def _loss_from_forward(w, cfg, hidden3, tok, mask_emb, h_shared, rows, K, labels, scale):
    lg = po.train_forward(w, cfg, hidden3, tok, mask_emb, h_shared, rows, K)
    lab = labels[np.asarray(rows) // K]
    i = np.flatnonzero(lab >= 0)
    return scale * float(np.sum(logsumexp(lg[i], axis=1) - lg[i, lab[i]]))


def test_gradients_match_finite_differences():
    cfg, w, rows, hidden3, tok, mask_emb, h_shared, labels = _problem()
    K = 3
    scored = int(np.sum(labels[rows // K] >= 0))
    loss, g = po.train_loss_grads(w, cfg, hidden3, tok, mask_emb, h_shared, rows, K, labels)
    ref = _loss_from_forward(w, cfg, hidden3, tok, mask_emb, h_shared, rows, K, labels, 1.0 / scored)
    assert abs(loss - ref) < 1e-12 * max(1.0, abs(ref))
    rng = np.random.default_rng(1)
    eps = 1e-5

    def fd(get, n_entries=4):
        """Central differences of the loss in n_entries random entries of the array get() returns."""
        arr = get()
        out = []
        for flat in rng.choice(arr.size, size=min(n_entries, arr.size), replace=False):
            ix = np.unravel_index(flat, arr.shape)
            old = arr[ix]
            arr[ix] = old + eps
            lp = _loss_from_forward(w, cfg, hidden3, tok, mask_emb, h_shared, rows, K, labels, 1.0 / scored)
            arr[ix] = old - eps
            lm = _loss_from_forward(w, cfg, hidden3, tok, mask_emb, h_shared, rows, K, labels, 1.0 / scored)
            arr[ix] = old
            out.append((ix, (lp - lm) / (2 * eps)))
        return out

    checks = [("fc", lambda: w["fc"], g["fc"]), ("final_norm", lambda: w["final_norm"], g["final_norm"]),
              ("lm_head", lambda: w["lm_head"], g["lm_head"]), ("mask_emb", lambda: mask_emb, g["mask_emb"]),
              ("h_shared", lambda: h_shared, g["h_shared"]),
              ("embed_rows", lambda: w["embed_rows"], g["embed_rows"])]
    for l in range(cfg.n_layers):
        for key in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down"):
            checks.append((f"L{l}.{key}", (lambda l=l, key=key: w["layers"][l][key]), g["layers"][l][key]))
    for name, get, grad in checks:
        assert grad.shape == get().shape, name
        for ix, num in fd(get):
            assert abs(grad[ix] - num) <= 2e-7 * max(1.0, abs(num)), (name, ix, grad[ix], num)


@pytest.mark.parametrize("S", [2, 3])
def test_gradients_accumulate_over_partition_chunks(S):
    """Each chunk scores only its own cells with the whole sequence's scale;
    the chunks' gradients sum to the whole forward's."""
    cfg, w, rows, hidden3, tok, mask_emb, h_shared, labels = _problem(n=11, K=3, seed=8)
    K, n = 3, 11
    scored = int(np.sum(labels[rows // K] >= 0))
    loss, g = po.train_loss_grads(w, cfg, hidden3, tok, mask_emb, h_shared, rows, K, labels)
    acc_loss, acc = 0.0, None
    for s in range(S):
        cells, own = po.chunk_cells(n, K, S, rows, s)
        lc, gc = po.train_loss_grads(w, cfg, hidden3, tok, mask_emb, h_shared, cells, K, labels,
                                     loss_scale=1.0 / scored, loss_rows=np.searchsorted(cells, rows[own]))
        acc_loss += lc
        if acc is None:
            acc = gc
        else:
            for key in ("fc", "final_norm", "lm_head", "mask_emb", "h_shared", "embed_rows"):
                acc[key] = acc[key] + gc[key]
            for l in range(cfg.n_layers):
                for key in acc["layers"][l]:
                    acc["layers"][l][key] = acc["layers"][l][key] + gc["layers"][l][key]
    assert abs(acc_loss - loss) < 1e-12
    for key in ("fc", "final_norm", "lm_head", "mask_emb", "h_shared", "embed_rows"):
        np.testing.assert_allclose(acc[key], g[key], rtol=0, atol=1e-11)
    for l in range(cfg.n_layers):
        for key in g["layers"][l]:
            np.testing.assert_allclose(acc["layers"][l][key], g["layers"][l][key], rtol=0, atol=1e-11)


def test_no_scored_cell_gives_zero_gradients():
    cfg, w, rows, hidden3, tok, mask_emb, h_shared, labels = _problem()
    loss, g = po.train_loss_grads(w, cfg, hidden3, tok, mask_emb, h_shared, rows, 3, np.full(7, -1))
    assert loss == 0.0
    assert np.all(g["lm_head"] == 0) and np.all(g["fc"] == 0)
    assert all(np.all(v == 0) for v in g["layers"][0].values())


def test_single_cell_loss_gradient_of_lm_head_is_closed_form():
    """One depth-0 cell, no layers: dL/dW_lm = (softmax(l) - e_label) z^T
    with z the final-norm output, the textbook cross-entropy gradient."""
    cfg, w, _, hidden3, tok, mask_emb, h_shared, _ = _problem(N=0)
    rows = np.array([0])
    labels = np.array([4] + [-1] * 6)
    loss, g = po.train_loss_grads(w, cfg, hidden3, tok, mask_emb, h_shared, rows, 3, labels, N=0)
    x = w["embed_rows"][0] + w["fc"] @ hidden3[0]
    z = x / np.sqrt(np.mean(x * x) + cfg.rms_eps) * w["final_norm"]
    lg = w["lm_head"] @ z
    p = np.exp(lg - logsumexp(lg))
    e = np.zeros_like(p)
    e[4] = 1.0
    np.testing.assert_allclose(g["lm_head"], np.outer(p - e, z), rtol=0, atol=1e-13)
    assert abs(loss - (logsumexp(lg) - lg[4])) < 1e-13
