"""Whole-pass pins for the oracle: the row-by-row block walk against an independently
written T x T masked-softmax formulation, decode against prefill, and the routing
invariants the pages state (CPU only)."""
import math

import numpy as np
import pytest

from oracle import dash_oracle as O
from long_context_sparse_stage0_amd import synth
from long_context_sparse_stage0_amd.workloads import Workload


def _rand(B, Hq, Hkv, T, D, seed, needle=0.0):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(B, Hq, T, D))
    k = rng.normal(size=(B, Hkv, T, D))
    v = rng.normal(size=(B, Hkv, T, D))
    hc = rng.normal(size=(Hkv, D)) / 8
    if needle:
        # make routing non-trivial: push a few chunks along the query direction
        G = Hq // Hkv
        for b in range(B):
            for h in range(Hkv):
                u = q[b, h * G:(h + 1) * G].mean(axis=(0, 1))
                u /= np.linalg.norm(u)
                for c in rng.choice(T // 64, size=min(2, T // 64), replace=False):
                    k[b, h, c * 64:(c + 1) * 64] += needle * u
    return q, k, v, hc


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0])
@pytest.mark.parametrize("G", [1, 4])
def test_block_walk_equals_dense_formulation(alpha, G):
    T, D = 300, 8                       # four full chunks and a ragged tail
    q, k, v, hc = _rand(1, 2 * G, 2, T, D, seed=int(alpha * 10) + G, needle=2.0)
    walk = O.prefill(q, k, v, hc, alpha=alpha)
    dense = O.prefill_dense_formulation(q, k, v, hc, alpha=alpha)
    np.testing.assert_allclose(walk["out"], dense, rtol=0, atol=1e-12)
    # the routing is genuinely sparse for some rows and dense for others
    frac = O.zero_fraction(walk["w_bar"], walk["rows"])
    assert 0.0 <= frac < 1.0


@pytest.mark.parametrize("sigma", [0.0, 2.0])
def test_block_walk_equals_dense_formulation_prior_strength(sigma):
    T, D = 300, 8
    q, k, v, hc = _rand(1, 8, 2, T, D, seed=77, needle=2.0)
    walk = O.prefill(q, k, v, hc, alpha=1.5, sigma=sigma)
    dense = O.prefill_dense_formulation(q, k, v, hc, alpha=1.5, sigma=sigma)
    np.testing.assert_allclose(walk["out"], dense, rtol=0, atol=1e-12)
    # and sigma matters whenever a routed weight lies strictly between 0 and 1
    ref = O.prefill(q, k, v, hc, alpha=1.5)
    assert np.abs(walk["out"] - ref["out"]).max() > 1e-6


def test_row_subset_equals_full():
    q, k, v, hc = _rand(2, 4, 2, 200, 8, seed=3, needle=1.0)
    full = O.prefill(q, k, v, hc)
    rows = np.array([0, 63, 64, 130, 199])
    sub = O.prefill(q, k, v, hc, rows=rows)
    np.testing.assert_allclose(sub["out"], full["out"][:, :, rows], atol=0)
    np.testing.assert_allclose(sub["w_bar"], full["w_bar"][:, :, rows], atol=0)


def test_routing_invariants():
    q, k, v, hc = _rand(1, 8, 2, 512, 16, seed=4, needle=12.0)
    r = O.prefill(q, k, v, hc, alpha=1.5)
    wb, mg, mask = r["w_bar"], r["margin"], r["mask"]
    T = 512
    for t in range(T):
        it = t // 64
        # rows of the first chunk route nowhere; nothing at or after the own chunk
        assert np.all(wb[..., t, it:] == 0.0)
        if it:
            seg = wb[..., t, :it]
            np.testing.assert_allclose(seg.sum(axis=-1), 1.0, atol=1e-12)
            # the mask bit is set exactly where some head has a positive margin
            assert np.array_equal(mask[..., t, :it], mg[..., t, :it] > 0.0)
    assert 0.0 < O.zero_fraction(wb, r["rows"]) < 1.0


def test_gqa_average_of_head_distributions():
    rng = np.random.default_rng(8)
    qg = rng.normal(size=(4, 16))
    summ = rng.normal(size=(10, 16))
    wb, mg, p = O.route_row(qg, summ, 64 * 10 + 5, alpha=1.5, gamma=1.0, scale=0.25)
    for g in range(4):
        np.testing.assert_allclose(p[g], O.entmax15_sorted(0.25 * summ @ qg[g]), atol=1e-12)
    np.testing.assert_allclose(wb, p.mean(0), atol=1e-15)
    # shared support is the union of the heads' supports
    assert np.array_equal(wb > 0, (p > 0).any(axis=0))


def test_gamma_scales_logits():
    rng = np.random.default_rng(2)
    qg = rng.normal(size=(2, 8))
    summ = rng.normal(size=(6, 8))
    a, _, _ = O.route_row(qg, summ, 6 * 64, alpha=1.5, gamma=2.0, scale=0.5)
    b, _, _ = O.route_row(qg, summ, 6 * 64, alpha=1.5, gamma=1.0, scale=1.0)
    np.testing.assert_allclose(a, b, atol=1e-14)


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_decode_equals_prefill_row(alpha):
    B, Hq, Hkv, T, D = 2, 4, 2, 390, 8
    q, k, v, hc = _rand(B, Hq, Hkv, T, D, seed=21, needle=2.0)
    full = O.prefill(q, k, v, hc, alpha=alpha)
    scale = 1 / math.sqrt(D)
    summ = O.chunk_summaries(k, hc, scale)           # frozen summaries of full chunks
    for t in (5, 63, 64, 127, 128, 300, 389):
        seq = np.array([t + 1, t + 1])
        # a cache longer than the sequence: entries past t must not matter
        kc = np.concatenate([k, np.full((B, Hkv, 40, D), 7.0)], axis=2)
        vc = np.concatenate([v, np.full((B, Hkv, 40, D), -7.0)], axis=2)
        kc[:, :, t + 1:] = 7.0
        vc[:, :, t + 1:] = -7.0
        # the summary cache holds only chunks complete by step t
        sc = np.zeros((B, Hkv, kc.shape[2] // 64 + 1, D))
        n = (t + 1) // 64
        sc[:, :, :n] = summ[:, :, :n]
        d = O.decode_step(q[:, :, t], kc, vc, seq, sc, alpha=alpha)
        np.testing.assert_allclose(d["out"], full["out"][:, :, t], atol=1e-12)
        it = t // 64
        np.testing.assert_allclose(d["w_bar"][..., :it], full["w_bar"][:, :, t, :it], atol=1e-15)


# ---------------------------------------------------------------- generator

def test_generator_is_deterministic_and_bf16():
    w = Workload(name="tiny", kind="prefill", B=1, Hq=8, Hkv=2, T=640, D=32, dtype="bf16",
                 seed=123, needle_amp=3.0)
    a = synth.prefill_inputs(w)
    b = synth.prefill_inputs(w, workers=1)
    for key in a:
        assert np.array_equal(a[key], b[key])
        assert np.array_equal(synth.round_bf16(a[key]), a[key]), key
    # queries are marginally ~N(0,1)
    assert abs(a["q"].std() - 1.0) < 0.05
    # needles exist: some chunks of the keys are shifted along their block's query mean
    k0 = synth.prefill_inputs(Workload(name="t0", kind="prefill", B=1, Hq=8, Hkv=2, T=640,
                                       D=32, dtype="bf16", seed=123, needle_amp=0.0))["k"]
    moved = np.abs(a["k"] - k0).reshape(1, 2, 10, 64, 32).max(axis=(3, 4)) > 0.5
    assert moved.any() and not moved.all()
    assert not moved[..., 9].any()          # the last chunk is before no query block


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.00390625, 3.0e38],
                 dtype=np.float32)
    r = synth.round_bf16(x)
    assert r[0] == 1.0
    assert r[1] == 1.0                       # tie -> even (mantissa ...0)
    assert r[2] == 1.0 + 4 * 2 ** -8         # tie -> even (rounds up)
    assert r[3] == -2.5
    bits = synth.bf16_bits(r)
    assert bits.dtype == np.uint16 and bits[0] == 0x3F80


def test_needles_create_sparsity_in_routing():
    w = Workload(name="tiny2", kind="prefill", B=1, Hq=8, Hkv=2, T=1024, D=64, dtype="bf16",
                 seed=5, needle_amp=3.0)
    x = synth.prefill_inputs(w)
    rows = np.arange(64 * 8, 1024, 37)
    r = O.prefill(x["q"], x["k"], x["v"], x["head_cls"], rows=rows)
    frac = O.zero_fraction(r["w_bar"], rows)
    assert frac > 0.3, frac


# ---------------------------------------------------------------------------------------
# Top-k comparison router
# ---------------------------------------------------------------------------------------

def test_topk_router_brute_force():
    """On tiny rows the selected chunks are the k-subset with the largest total group score,
    and k = 1 is the argmax."""
    import itertools
    rng = np.random.default_rng(41)
    G, D = 4, 8
    for trial in range(30):
        it = int(rng.integers(2, 9))
        t = 64 * it + int(rng.integers(0, 64))
        qg = rng.normal(size=(G, D))
        summ = rng.normal(size=(it, D))
        z = (qg @ summ.T).mean(axis=0) * 0.3
        for k in range(1, it + 1):
            w, m = O.route_row_topk(qg, summ, t, k=k, gamma=1.0, scale=0.3)
            sel = set(np.flatnonzero(w > 0))
            best = max(itertools.combinations(range(it), k), key=lambda c: z[list(c)].sum())
            assert sel == set(best) and len(sel) == k
            assert np.all((m >= 0) == (w > 0))
        w, _ = O.route_row_topk(qg, summ, t, k=1, gamma=1.0, scale=0.3)
        assert np.flatnonzero(w) == [np.argmax(z)]


def test_topk_router_keeps_ties_and_short_rows():
    qg = np.ones((2, 4))
    summ = np.array([[1.0, 0, 0, 0], [2.0, 0, 0, 0], [2.0, 0, 0, 0], [0.5, 0, 0, 0]])
    w, _ = O.route_row_topk(qg, summ, 4 * 64, k=1, gamma=1.0, scale=1.0)
    np.testing.assert_array_equal(w, [0, 1, 1, 0])            # both tied maxima
    w, m = O.route_row_topk(qg, summ, 4 * 64 + 5, k=7, gamma=1.0, scale=1.0)
    np.testing.assert_array_equal(w, [1, 1, 1, 1])            # i_t <= k: every chunk


def test_topk_with_every_chunk_is_dense_causal():
    """k at least the number of routed chunks selects everything with no prior: the whole
    prefill equals textbook causal attention."""
    T, D = 300, 8
    q, k, v, hc = _rand(1, 4, 2, T, D, seed=43)
    out = O.prefill(q, k, v, hc, topk=8)["out"]
    for h in range(4):
        ref = O.causal_attention(q[0, h], k[0, h // 2], v[0, h // 2])
        np.testing.assert_allclose(out[0, h], ref, atol=1e-12)


# ---------------------------------------------------------------------------------------
# estimate_diagonal: the own chunk's partial summary joins the entmax normalisation
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("alpha", [1.5, 2.0])
@pytest.mark.parametrize("G", [1, 4])
def test_estimate_diagonal_block_walk_equals_dense_formulation(alpha, G):
    T, D = 300, 8
    q, k, v, hc = _rand(1, 2 * G, 2, T, D, seed=int(alpha * 10) + G + 50, needle=2.0)
    walk = O.prefill(q, k, v, hc, alpha=alpha, estimate_diagonal=True)
    dense = O.prefill_dense_formulation(q, k, v, hc, alpha=alpha, estimate_diagonal=True)
    np.testing.assert_allclose(walk["out"], dense, rtol=0, atol=1e-12)
    plain = O.prefill(q, k, v, hc, alpha=alpha)
    assert np.abs(walk["out"] - plain["out"]).max() > 1e-6      # the correction matters
    np.testing.assert_array_equal(walk["out"][:, :, :64], plain["out"][:, :, :64])  # no routing


def test_estimate_diagonal_weights_leave_room_for_the_diagonal():
    """With the own chunk in the normalisation the routed weights of each head sum to
    1 - p_diagonal, so their GQA mean sums to at most 1, and below 1 when the own chunk
    keeps weight."""
    q, k, v, hc = _rand(1, 8, 2, 500, 8, seed=61, needle=1.0)
    r = O.prefill(q, k, v, hc, estimate_diagonal=True)
    s = r["w_bar"].sum(axis=-1)[:, :, 64:]                     # rows that route
    assert np.all(s <= 1.0 + 1e-12) and np.any(s < 1.0 - 1e-6)
    r0 = O.prefill(q, k, v, hc)
    np.testing.assert_allclose(r0["w_bar"].sum(axis=-1)[:, :, 64:], 1.0, atol=1e-12)


def test_diagonal_summary_with_zero_query_is_the_mean_of_the_keys_so_far():
    rng = np.random.default_rng(62)
    k = rng.normal(size=(200, 6))
    for t in (128, 130, 191):
        dg = O.diagonal_summary(k, np.zeros(6), t, 0.5)
        np.testing.assert_allclose(dg, k[128:t + 1].mean(axis=0), atol=1e-14)
