"""Pins for the oracle's Stage 0 summaries, Stage 2 prior softmax and the whole prefill
(CPU only)."""
import json
import math
import os

import numpy as np
import pytest

from oracle import dash_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


G = _golden("stage_closed_forms.json")


# ---------------------------------------------------------------- Stage 0

def _keys_jline(scale_first=1.0):
    j = np.arange(64, dtype=np.float64)
    return np.stack([j * scale_first, np.ones(64), -j / 2.0], axis=1)


def test_stage0_zero_query_is_mean_pool_golden():
    k = _keys_jline()[None, None]                     # [1,1,64,3]
    s = O.chunk_summaries(k, np.zeros((1, 3)), scale=0.37)
    np.testing.assert_allclose(s[0, 0, 0], G["stage0_mean_pool"]["summary"], rtol=0, atol=1e-15)


def test_stage0_zero_query_is_mean_pool_random():
    rng = np.random.default_rng(0)
    k = rng.normal(size=(2, 3, 64 * 5 + 17, 8))
    s = O.chunk_summaries(k, np.zeros((3, 8)), scale=1 / math.sqrt(8))
    ref = k[:, :, : 64 * 5].reshape(2, 3, 5, 64, 8).mean(axis=3)
    np.testing.assert_allclose(s, ref, rtol=0, atol=1e-15)
    assert s.shape == (2, 3, 5, 8), "the ragged tail chunk has no summary"


def test_stage0_sharp_query_selects_one_key_golden():
    k = _keys_jline(1.0 / 63.0)[None, None]
    s = O.chunk_summaries(k, np.array([[1000.0, 0.0, 0.0]]), scale=1.0)
    np.testing.assert_allclose(s[0, 0, 0], G["stage0_one_hot"]["summary"], atol=1e-6)


def test_stage0_is_convex_combination_and_uses_scale():
    rng = np.random.default_rng(1)
    k = rng.normal(size=(1, 2, 128, 4))
    hc = rng.normal(size=(2, 4))
    s1 = O.chunk_summaries(k, hc, scale=0.5)
    s2 = O.chunk_summaries(k, hc, scale=1.0)
    s3 = O.chunk_summaries(k, 2.0 * hc, scale=0.5)
    np.testing.assert_allclose(s2, s3, atol=1e-14)     # scale multiplies the logits
    assert np.abs(s1 - s2).max() > 1e-3
    # inside the per-coordinate hull of the chunk's keys
    kc = k.reshape(1, 2, 2, 64, 4)
    assert np.all(s1 <= kc.max(axis=3) + 1e-12) and np.all(s1 >= kc.min(axis=3) - 1e-12)
    # brute force: explicit loops over one chunk
    b, h, c = 0, 1, 1
    a = [0.5 * float(hc[h] @ k[b, h, 64 * c + j]) for j in range(64)]
    m = max(a)
    e = [math.exp(x - m) for x in a]
    ref = sum(e[j] / sum(e) * k[b, h, 64 * c + j] for j in range(64))
    np.testing.assert_allclose(s1[b, h, c], ref, atol=1e-14)


# ---------------------------------------------------------------- Stage 2

@pytest.mark.parametrize("case", G["prior_softmax"])
def test_prior_softmax_golden(case):
    p = O.prior_softmax(np.array(case["z"]), np.array(case["g"]))
    np.testing.assert_allclose(p, case["p"], atol=1e-15)


def test_prior_softmax_is_kl_maximiser():
    rng = np.random.default_rng(5)
    for n in (2, 4, 9):
        z = rng.normal(size=n)
        g = rng.dirichlet(np.ones(n))
        p = O.prior_softmax(z, g)
        obj = lambda q: float(q @ z - np.sum(np.where(q > 0, q * np.log(q / g), 0.0)))
        best = obj(p)
        for _ in range(2000):
            q = rng.dirichlet(np.ones(n))
            assert best >= obj(q) - 1e-12
        for _ in range(200):
            d = rng.normal(size=n) * 1e-4
            d -= d.mean()
            if np.all(p + d > 0):
                assert best >= obj(p + d) - 1e-12
        # uniform reference reduces to plain softmax
        np.testing.assert_allclose(O.prior_softmax(z, np.full(n, 1.0 / n)), O.softmax(z), atol=1e-15)


def test_attention_row_golden():
    a = G["attention_row"]
    k = np.array(a["k"])
    v = np.array(a["v"])
    o = O.attend_row(np.array(a["q"]), k, v, 1, np.zeros(0), scale=1.0)
    np.testing.assert_allclose(o, a["o_row1"], atol=1e-14)


@pytest.mark.parametrize("T", [64, 200, 320])
def test_all_blocks_uniform_prior_is_dense_causal(T):
    rng = np.random.default_rng(T)
    D = 16
    q = rng.normal(size=(T, D))
    k = rng.normal(size=(T, D))
    v = rng.normal(size=(T, D))
    ref = O.causal_attention(q, k, v)
    for t in range(T):
        o = O.attend_row(q[t], k, v, t, np.ones(t // 64), scale=1 / math.sqrt(D))
        np.testing.assert_allclose(o, ref[t], atol=1e-12)


def test_zero_weight_blocks_contribute_nothing():
    rng = np.random.default_rng(9)
    T, D = 300, 8
    q, k, v = (rng.normal(size=(T, D)) for _ in range(3))
    t = 299
    w = np.array([0.5, 0.0, 0.25, 0.25])
    o = O.attend_row(q[t], k, v, t, w, scale=0.3)
    k2, v2 = k.copy(), v.copy()
    k2[64:128] = rng.normal(size=(64, D)) * 10
    v2[64:128] = rng.normal(size=(64, D)) * 10
    np.testing.assert_allclose(O.attend_row(q[t], k2, v2, t, w, scale=0.3), o, atol=1e-15)
    # ... while a nonzero block does matter, with weight entering as a log-prior
    v3 = v.copy()
    v3[0:64] += 1.0
    assert np.abs(O.attend_row(q[t], k, v3, t, w, scale=0.3) - o).max() > 1e-3
    # keys after t never matter (causality inside the diagonal chunk)
    t = 270
    k4, v4 = k.copy(), v.copy()
    k4[t + 1:] = 99.0
    v4[t + 1:] = -99.0
    np.testing.assert_allclose(O.attend_row(q[t], k4, v4, t, w, scale=0.3),
                               O.attend_row(q[t], k, v, t, w, scale=0.3), atol=1e-15)


def test_prior_bias_equals_weighted_key_multiplicity():
    """A block of weight w behaves like the block's keys replicated with multiplicity w."""
    rng = np.random.default_rng(12)
    D = 4
    k = rng.normal(size=(130, D))
    v = rng.normal(size=(130, D))
    q = rng.normal(size=D)
    t = 129
    w = np.array([0.2, 0.8])
    o = O.attend_row(q, k, v, t, w, scale=1.0)
    e = np.exp(k @ q)
    wt = np.concatenate([np.full(64, 0.2), np.full(64, 0.8), np.ones(t + 1 - 128)])
    wt = wt * e[: t + 1]
    ref = (wt[:, None] * v[: t + 1]).sum(0) / wt.sum()
    np.testing.assert_allclose(o, ref, atol=1e-13)


def test_prior_strength_zero_uses_the_support_only():
    """sigma = 0: the prior is uniform over the active chunks, so the row is plain softmax
    attention over the keys of the chunks with w_bar > 0 plus the causal diagonal keys, and
    rescaling the positive weights changes nothing."""
    rng = np.random.default_rng(21)
    T, D = 300, 8
    q, k, v = (rng.normal(size=(T, D)) for _ in range(3))
    t = 290
    w = np.array([0.6, 0.0, 0.1, 0.3])
    o = O.attend_row(q[t], k, v, t, w, scale=0.4, sigma=0.0)
    keys = [j for j in range(t + 1) if j >= 256 or w[j // 64] > 0]
    s = 0.4 * k[keys] @ q[t]
    p = np.exp(s - s.max())
    np.testing.assert_allclose(o, (p / p.sum()) @ v[keys], atol=1e-13)
    w2 = np.where(w > 0, rng.uniform(0.01, 5.0, size=w.shape), 0.0)
    np.testing.assert_allclose(O.attend_row(q[t], k, v, t, w2, scale=0.4, sigma=0.0), o,
                               atol=1e-13)


@pytest.mark.parametrize("sigma", [0.5, 2.0])
def test_prior_strength_is_a_power_of_the_multiplicity(sigma):
    """A block of weight w with prior strength sigma behaves like its keys replicated with
    multiplicity w ** sigma."""
    rng = np.random.default_rng(13)
    D = 4
    k = rng.normal(size=(130, D))
    v = rng.normal(size=(130, D))
    q = rng.normal(size=D)
    t = 129
    w = np.array([0.2, 0.8])
    o = O.attend_row(q, k, v, t, w, scale=1.0, sigma=sigma)
    e = np.exp(k @ q)
    wt = np.concatenate([np.full(64, 0.2 ** sigma), np.full(64, 0.8 ** sigma), np.ones(t + 1 - 128)])
    wt = wt * e[: t + 1]
    ref = (wt[:, None] * v[: t + 1]).sum(0) / wt.sum()
    np.testing.assert_allclose(o, ref, atol=1e-13)


def test_zero_fraction_counts_routed_pairs_only():
    """zero_fraction: the share of (row, kv head, chunk c < t // 64) entries whose weight is
    exactly 0.  Hand-built weights with a known answer: row 0 routes nothing, row 64 routes
    chunk 0 only, row 200 routes chunks 0..2; the own chunk and everything past it (set to 0
    here on purpose) must not be counted."""
    rows = np.array([0, 64, 200])
    wb = np.full((1, 2, 3, 5), 0.25)
    wb[0, 0, 1, 0] = 0.0          # row 64, head 0: its one routed chunk is inactive
    wb[0, 1, 2, 1] = 0.0          # row 200, head 1: chunk 1 inactive
    wb[0, 0, 2, 3:] = 0.0         # row 200: own chunk 3 and chunk 4 are outside the count
    wb[0, :, 0, :] = 0.0          # row 0 routes no chunk at all
    # routed entries: 2 heads x (1 + 3) = 8, of which 2 are zero
    assert O.zero_fraction(wb, rows) == pytest.approx(2 / 8, abs=0)
    # every routed entry zero -> 1; no routed entry at all -> 0
    assert O.zero_fraction(np.zeros_like(wb), rows) == 1.0
    assert O.zero_fraction(wb[:, :, :1], rows[:1]) == 0.0
    # brute force over random sparsity patterns, counted a different way
    rng = np.random.default_rng(3)
    t = np.sort(rng.choice(np.arange(1024), size=40, replace=False))
    w = rng.random((2, 3, t.size, 16)) * (rng.random((2, 3, t.size, 16)) < 0.6)
    routed = np.arange(16)[None, :] < (t // 64)[:, None]           # [rows, chunks]
    zeros = ((w == 0.0) & routed[None, None]).sum()
    total = routed.sum() * 2 * 3
    assert O.zero_fraction(w, t) == pytest.approx(zeros / total, rel=0, abs=1e-15)
