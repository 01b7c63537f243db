"""Pins of greedy acceptance: exhaustive patterns and the acceptance table."""
import itertools
import json
import os

import numpy as np

from oracle import peagle_oracle as po
from drafting_eagle_draft_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_accept_exhaustive_patterns():
    for K in range(1, 9):
        pats = np.array(list(itertools.product([0, 1], repeat=K)), dtype=bool)
        B = len(pats)
        draft = np.arange(B * K).reshape(B, K) + 10
        target = np.where(pats, draft, -5)
        target = np.concatenate([target, np.full((B, 1), 7)], axis=1)
        alen, out = po.accept(draft, target)
        for b in range(B):
            first_miss = next((i for i in range(K) if not pats[b, i]), K)
            assert alen[b] == first_miss
            assert list(out[b, :alen[b] + 1]) == list(target[b, :alen[b] + 1])
            assert np.all(out[b, alen[b] + 1:] == -1)


def test_acceptance_table_identity_and_planted_rates():
    tab = json.load(open(os.path.join(GOLD, "acceptance_table.json")))["rows"]
    # The page's own table: average emitted length = 1 + sum of per-position rates.
    for name, row in tab.items():
        assert abs(1 + sum(row[:7]) - row[7]) <= 0.006, name
    # Planted targets reproduce the Average row through the oracle's accept.
    K, V, B = 7, 1000, 40000
    rng = np.random.default_rng(3)
    drafts = rng.integers(0, V, (B, K))
    target, a_planted = synth.planted_targets(drafts, V, seed=5, rates=synth.ACCEPT_TABLE_AVERAGE)
    alen, out = po.accept(drafts, target)
    np.testing.assert_array_equal(alen, a_planted)
    pos = [(alen >= k).mean() for k in range(1, K + 1)]
    np.testing.assert_allclose(pos, tab["Average"][:7], atol=0.01)
    emitted = (out >= 0).sum(1)
    assert abs(emitted.mean() - tab["Average"][7]) < 0.03
    np.testing.assert_allclose(emitted.mean(), 1 + sum(pos), rtol=1e-12)
