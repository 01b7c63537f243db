"""Pins of COD sampling, the attention mask (fresh and amortized) and the
sequence partition, against what the pages state."""
import json
import os

import numpy as np
import pytest

from oracle import peagle_oracle as po

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_mask_worked_example():
    fx = _load("mask_worked_example.json")
    p, d = fx["query"]
    for pk, dk in fx["visible"]:
        assert po.mask_allowed(p, d, pk, dk), (pk, dk)
    for pk, dk in fx["invisible"]:
        assert not po.mask_allowed(p, d, pk, dk), (pk, dk)


@pytest.mark.parametrize("n,K", [(6, 3), (9, 4), (5, 8)])
def test_mask_rules_and_row_sums(n, K):
    rows = np.array([r for r in range(n * K) if r // K >= r % K])  # every cell with an anchor
    m = po.mask_fresh(rows, K)
    for i, r in enumerate(rows):
        p, d = divmod(int(r), K)
        vis = [divmod(int(rows[j]), K) for j in np.where(m[i])[0]]
        # Depth-0 rows are causal among themselves.
        if d == 0:
            assert vis == [(q, 0) for q in range(p + 1)]
        # Every row sees exactly p + 1 keys: a + 1 base keys and d chain keys.
        assert len(vis) == p + 1
        # Never forward in the base sequence, never sideways into another rollout.
        for pk, dk in vis:
            if dk == 0:
                assert pk <= p - d
            else:
                assert pk - dk == p - d and dk <= d
        assert (p, d) in vis  # itself


def test_memory_arithmetic():
    fx = _load("cod_and_memory.json")["memory"]
    positions = fx["n"] * fx["K"]
    assert positions == fx["positions"]
    nbytes = positions * positions * 2  # one BF16 score per (query, key) of the full grid
    assert nbytes == 2 ** 33
    assert abs(nbytes - fx["approx_bytes_bf16"]) / fx["approx_bytes_bf16"] < 0.08


@pytest.mark.parametrize("n_max,n,K,seed", [(12, 7, 4, 0), (16, 16, 3, 1), (10, 4, 8, 2), (20, 13, 5, 3)])
def test_amortized_slice_equals_fresh(n_max, n, K, seed):
    m_pre = po.mask_precompute(n_max, K)
    rng = np.random.default_rng(seed)
    rows = po.cod_rows(po.cod_keep(n, K, rng.random((n, K)), r=0.7))
    np.testing.assert_array_equal(po.mask_slice(m_pre, n, K, rows), po.mask_fresh(rows, K))


def test_cod_chain_closure_and_depth0():
    rng = np.random.default_rng(4)
    n, K = 300, 8
    keep = po.cod_keep(n, K, rng.random((n, K)), r=0.8)
    assert keep[:, 0].all()
    for p in range(n):
        for d in range(1, K):
            if keep[p, d]:
                assert p >= d and keep[p - 1, d - 1]
    rows = po.cod_rows(keep)
    assert np.all(np.diff(rows) > 0)


def test_cod_rates_page_example():
    fx = _load("cod_and_memory.json")["rates_r07"]
    n, K = 60000, 3
    rng = np.random.default_rng(11)
    keep = po.cod_keep(n, K, rng.random((n, K)), r=fx["r"], floor=fx["floor"])
    for d, frac in fx["depth_fraction"].items():
        d = int(d)
        got = keep[d:, d].mean()
        assert abs(got - frac) < 0.01, (d, got, frac)


def test_cod_floor_binds():
    # r = 0.5: marginals 1, .5, .25, then the 0.2 floor: depth 3 and deeper
    # keep 0.2 of positions, so a kept depth-3 parent always keeps its child.
    n, K = 40000, 6
    rng = np.random.default_rng(12)
    keep = po.cod_keep(n, K, rng.random((n, K)), r=0.5, floor=0.2)
    for d, frac in [(1, 0.5), (2, 0.25), (3, 0.2), (4, 0.2), (5, 0.2)]:
        assert abs(keep[d:, d].mean() - frac) < 0.01, d
    assert np.array_equal(keep[4:, 4], keep[3:-1, 3])


def test_cod_count_matches_page():
    fx = _load("cod_and_memory.json")["count_r08"]
    n, K = fx["n"], fx["K"]
    counts = []
    for seed in range(4):
        rng = np.random.default_rng(100 + seed)
        counts.append(int(po.cod_keep(n, K, rng.random((n, K)), r=fx["r"]).sum()))
    mean = float(np.mean(counts))
    assert abs(mean - fx["approx_positions"]) / fx["approx_positions"] < fx["rel_tol"], counts


@pytest.mark.parametrize("S", [2, 3, 4, 7])
def test_partition_invariant_and_completion(S):
    rng = np.random.default_rng(S)
    n, K = 41, 5
    keep = po.cod_keep(n, K, rng.random((n, K)), r=0.8)
    rows = po.cod_rows(keep)
    chunk, bounds, completion = po.partition(n, K, S, rows)
    assert len(chunk) == len(rows)            # every retained row once
    assert bounds[0] == 0 and bounds[-1] == n
    where = {divmod(int(r), K): int(c) for r, c in zip(rows, chunk)}
    for (p, d), c in where.items():
        if d >= 2:
            assert c == where[(p - 1, d - 1)]   # Chunk(p, d) = Chunk(p-1, d-1)
        if d <= 1:
            assert bounds[c] <= p < bounds[c + 1]
    # Every allowed key of a row is in its chunk or in its depth-0 completion.
    m = po.mask_fresh(rows, K)
    for i, r in enumerate(rows):
        p, d = divmod(int(r), K)
        c = int(chunk[i])
        comp = set(int(x) for x in completion[c])
        for j in np.where(m[i])[0]:
            pk, dk = divmod(int(rows[j]), K)
            assert where[(pk, dk)] == c or (dk == 0 and pk in comp)


def test_key_closure_reproduces_sampled_rows():
    """One layer of the sampled rows depends only on their key closure: the
    oracle over that subset equals the oracle over the whole layout."""
    from tests.layout_util import key_closure
    from tests.toy import toy_problem, toy_cfg
    cfg, w, _ = toy_problem(toy_cfg(n_layers=1, K=5))
    n, K = 30, 5
    rng = np.random.default_rng(4)
    rows = po.cod_rows(po.cod_keep(n, K, rng.random((n, K)), r=0.8))
    hidden3 = rng.standard_normal((n, 3 * cfg.hidden)).astype(np.float32)
    tok = rng.integers(0, cfg.vocab, n)
    wr = dict(w, embed_rows=w["embed"][tok])
    mask_emb = rng.standard_normal(cfg.hidden).astype(np.float32) * 0.1
    h_shared = rng.standard_normal(3 * cfg.hidden).astype(np.float32)
    sample = np.array([3, 17, len(rows) // 2, len(rows) - 1])
    full = po.train_forward(wr, cfg, hidden3, tok, mask_emb, h_shared, rows, K)
    sub, lm = key_closure(rows, K, sample)
    assert len(sub) < len(rows)
    part = po.train_forward(wr, cfg, hidden3, tok, mask_emb, h_shared, sub, K, lm_rows=lm)
    np.testing.assert_allclose(part, full[sample], rtol=0, atol=1e-12)


@pytest.mark.parametrize("S", [2, 3, 4, 7])
def test_partitioned_forward_equals_whole_forward(S):
    """Sequence partitioning ("P-EAGLE: Parallel-Drafting EAGLE with Scalable
    Training", section 3.2): chunks that each recompute their depth-0
    completion through every layer and share nothing give every cell the
    logits of the unpartitioned forward (equal in exact arithmetic; two
    layers, so the completion's own keys are recomputed too)."""
    from tests.toy import toy_problem, toy_cfg
    cfg, w, _ = toy_problem(toy_cfg(n_layers=2, K=5))
    n, K = 23, 5
    rng = np.random.default_rng(40 + S)
    rows = po.cod_rows(po.cod_keep(n, K, rng.random((n, K)), r=0.8))
    hidden3 = rng.standard_normal((n, 3 * cfg.hidden)).astype(np.float32)
    tok = rng.integers(0, cfg.vocab, n)
    wr = dict(w, embed_rows=w["embed"][tok])
    mask_emb = rng.standard_normal(cfg.hidden).astype(np.float32) * 0.1
    h_shared = rng.standard_normal(3 * cfg.hidden).astype(np.float32)
    full = po.train_forward(wr, cfg, hidden3, tok, mask_emb, h_shared, rows, K)
    part = po.train_forward_partitioned(wr, cfg, hidden3, tok, mask_emb, h_shared, rows, K, S)
    np.testing.assert_allclose(part, full, rtol=0, atol=1e-10)
    # Each chunk's cells: chain-closed, every depth-0 cell up to the largest
    # anchor, own cells once over all chunks, and fewer cells than the whole.
    seen = np.zeros(len(rows), dtype=int)
    for s in range(S):
        cells, own = po.chunk_cells(n, K, S, rows, s)
        seen[own] += 1
        cs = set(int(c) for c in cells)
        amax = max(int(c) // K - int(c) % K for c in cells)
        assert all(p * K in cs for p in range(amax + 1))
        assert all((c - K - 1) in cs for c in cs if c % K >= 1)
        if s < S - 1:
            assert len(cells) < len(rows)
    assert np.all(seen == 1)


def test_partition_chunk_without_completion_differs():
    """A chunk's segment run with no completion sees no earlier context.
    Rotary attention depends on relative positions only, so running the
    segment's depth-0 cells as a sequence of their own changes nothing but
    the missing context, and their logits move: the completion is needed."""
    from tests.toy import toy_problem, toy_cfg
    cfg, w, _ = toy_problem(toy_cfg(n_layers=1, K=3))
    n, K, S = 12, 3, 3
    rows = np.array([p * K + d for p in range(n) for d in range(K) if p >= d], dtype=np.int64)
    rng = np.random.default_rng(9)
    hidden3 = rng.standard_normal((n, 3 * cfg.hidden)).astype(np.float32)
    tok = rng.integers(0, cfg.vocab, n)
    me, hs = np.zeros(cfg.hidden, np.float32), np.ones(3 * cfg.hidden, np.float32)
    full = po.train_forward(dict(w, embed_rows=w["embed"][tok]), cfg, hidden3, tok, me, hs, rows, K)
    _, bounds, _ = po.partition(n, K, S, rows)
    b0, b1 = int(bounds[1]), int(bounds[2])
    alone = po.train_forward(dict(w, embed_rows=w["embed"][tok[b0:b1]]), cfg, hidden3[b0:b1], tok[b0:b1],
                             me, hs, np.arange(b1 - b0) * K, K)
    ref = full[np.searchsorted(rows, np.arange(b0, b1) * K)]
    # the first cell of the segment keeps its own key but loses all earlier ones
    assert np.max(np.abs(alone - ref)) > 1e-3
    # sanity of the relative-position claim: the whole sequence shifted by
    # nothing reproduces itself through the same call pattern
    again = po.train_forward(dict(w, embed_rows=w["embed"][tok[:b1]]), cfg, hidden3[:b1], tok[:b1], me, hs,
                             np.arange(b1) * K, K)
    np.testing.assert_allclose(again[b0:], ref, rtol=0, atol=1e-10)
