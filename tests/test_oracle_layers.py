"""Pins of the oracle's elementary layer pieces (closed forms, invariants)."""
import math

import numpy as np
import pytest

from oracle import peagle_oracle as po


def test_rmsnorm_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 37)) * 3.0
    u = po.rmsnorm(x, np.ones(37), 0.0)
    # With eps = 0 and unit gains the output has mean square exactly 1.
    np.testing.assert_allclose(np.mean(u * u, axis=-1), 1.0, rtol=1e-14)
    # RMSNorm(c x) = RMSNorm(x) for c > 0 (eps = 0), direction preserved.
    np.testing.assert_allclose(po.rmsnorm(7.5 * x, np.ones(37), 0.0), u, rtol=1e-13)
    cos = np.sum(u * x, -1) / np.linalg.norm(u, axis=-1) / np.linalg.norm(x, axis=-1)
    np.testing.assert_allclose(cos, 1.0, rtol=1e-14)


def test_rmsnorm_gain_is_elementwise_and_eps_closed_form():
    x = np.array([3.0, 4.0])
    g = np.array([2.0, -1.0])
    # mean square = 12.5; with eps = 0.5 the divisor is sqrt(13).
    np.testing.assert_allclose(po.rmsnorm(x, g, 0.5), [6 / math.sqrt(13), -4 / math.sqrt(13)],
                               rtol=1e-15)


def test_rope_closed_form_hd4():
    # Rotate-half convention: pair (0, 2) turns by pos * theta^0, pair (1, 3)
    # by pos * theta^(-1/2).  theta = 10000, pos = 1: angles 1 and 0.01 rad.
    a = np.array([1.0, 2.0, 3.0, 4.0])
    out = po.rope(a, 1.0, 10000.0)
    expect = [math.cos(1) - 3 * math.sin(1), 2 * math.cos(0.01) - 4 * math.sin(0.01),
              3 * math.cos(1) + math.sin(1), 4 * math.cos(0.01) + 2 * math.sin(0.01)]
    np.testing.assert_allclose(out, expect, rtol=1e-15)


def test_rope_preserves_norm_and_relative_position():
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for p in (0, 5, 4099, 16391):
        np.testing.assert_allclose(np.linalg.norm(po.rope(q, p, 5e5)), np.linalg.norm(q), rtol=1e-13)
    # Scores depend only on the position difference (appendix B of the paper
    # notes builds on exactly this property).
    s1 = po.rope(q, 100, 5e5) @ po.rope(k, 37, 5e5)
    s2 = po.rope(q, 100 + 9000, 5e5) @ po.rope(k, 37 + 9000, 5e5)
    np.testing.assert_allclose(s1, s2, rtol=1e-9)
    # Position 0 is the identity.
    np.testing.assert_allclose(po.rope(q, 0, 5e5), q, rtol=0, atol=0)


def test_silu_closed_forms():
    np.testing.assert_allclose(po.silu(np.array([0.0, 1.0, -1.0])),
                               [0.0, 1 / (1 + math.exp(-1)), -1 / (1 + math.e)], rtol=1e-15)
    np.testing.assert_allclose(po.silu(np.array([40.0])), [40.0], rtol=1e-15)
    assert abs(po.silu(np.array([-40.0]))[0]) < 1e-15


def test_softmax_attention_closed_forms():
    rng = np.random.default_rng(2)
    vals = rng.standard_normal((6, 8))
    # Equal keys: uniform weights, output is the mean of the values.
    keys = np.tile(rng.standard_normal(8), (6, 1))
    q = rng.standard_normal((3, 8))
    np.testing.assert_allclose(po.attend(q, keys, vals, 0.3), np.tile(vals.mean(0), (3, 1)),
                               rtol=1e-13)
    # A single key returns its value.
    np.testing.assert_allclose(po.attend(q, keys[:1], vals[:1], 0.3), np.tile(vals[0], (3, 1)))
    # Softmax is shift invariant and sums to one.
    s = rng.standard_normal((4, 9))
    np.testing.assert_allclose(po.softmax(s), po.softmax(s + 123.0), rtol=1e-12)
    np.testing.assert_allclose(po.softmax(s).sum(-1), 1.0, rtol=1e-15)
    # Two keys: weights are the logistic function of the score gap.
    p = po.softmax(np.array([0.0, 2.0]))
    np.testing.assert_allclose(p[1], 1 / (1 + math.exp(-2)), rtol=1e-15)


def test_linear_matches_dot_products_across_chunks():
    rng = np.random.default_rng(3)
    w = rng.standard_normal((37, 11)).astype(np.float32)
    x = rng.standard_normal((2, 11))
    y = po.linear(x, w, chunk_rows=5)
    for i in range(2):
        for o in range(37):
            assert abs(y[i, o] - sum(float(x[i, j]) * float(w[o, j]) for j in range(11))) < 1e-12


def test_argmax_ties_lowest_and_margin():
    lg = np.array([[0.0, 3.0, 1.0, 3.0], [5.0, 5.0, 5.0, 5.0], [-1.0, -2.0, -0.5, -3.0]])
    assert list(po.argmax_lowest(lg)) == [1, 0, 2]
    np.testing.assert_allclose(po.top2_margin(lg), [0.0, 0.0, 0.5])
