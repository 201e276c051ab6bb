"""Pins of the oracle's Gumbel-max verification and of the noise table.

Each test checks the oracle against something other than its own formula:
the Gumbel-max theorem (reading-club post on Gumbel coupling: argmax of
logits + Gumbel noise samples from the softmax), the Gumbel distribution's
closed-form moments and CDF, exact fp32 tie cases, and brute force over every
candidate vector of a tiny vocabulary.
"""
import math

import numpy as np
import pytest
from scipy import stats

import oracle
import workloads as wl


def _softmax(z):
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - z.max())
    return e / e.sum()


@pytest.mark.parametrize("logits", [
    [0.0, 0.0],
    [1.5, -0.5],
    [0.3, -1.0, 2.0, 0.1],
    [-2.0, 1.0, 0.5, 0.5, 3.0, -1.0, 0.0, 2.5],
])
def test_gumbel_max_matches_softmax_sampling(logits):
    """Gumbel post, Gumbel-max trick: argmax(l + g) is distributed as softmax(l).
    200k independent noise rows (distinct positions); chi-square p > 1e-3.
    A sign error in -ln(-ln u), a wrong u mapping, a biased hash or a wrong
    argmax all fail this."""
    V = len(logits)
    n = 200_000
    g = wl.gumbel_noise(seed=7, requests=np.zeros(n, dtype=np.int64), positions=np.arange(n), vocab_size=V)
    l32 = np.broadcast_to(np.asarray(logits, dtype=np.float32), (n, V))
    t, _, _ = oracle.gumbel_verify(l32[:, None, :], g[:, None, :], np.full((n, 1), -1))
    counts = np.bincount(t[:, 0], minlength=V)
    expected = n * _softmax(logits)
    p = stats.chisquare(counts, expected).pvalue
    assert p > 1e-3, (counts, expected, p)


def test_noise_is_standard_gumbel():
    """Closed forms of Gumbel(0,1): mean = Euler-Mascheroni gamma, variance
    pi^2/6, CDF exp(-exp(-x)); range fixed by u in [2^-25, 1-2^-25]."""
    g = wl.gumbel_noise(seed=3, requests=np.arange(64), positions=np.full(64, 1000), vocab_size=8192)
    x = g.astype(np.float64).ravel()
    n = x.size
    assert abs(x.mean() - 0.5772156649) < 4 * math.sqrt(math.pi ** 2 / 6 / n)
    assert abs(x.var() - math.pi ** 2 / 6) < 0.02
    assert x.min() >= -2.8530 and x.max() <= 17.330
    ks = stats.kstest(x[:200_000], lambda v: np.exp(-np.exp(-v)))
    assert ks.pvalue > 1e-3


def test_noise_keys_are_independent():
    """Different (request, position) keys give uncorrelated rows; the same key
    gives the same row (noise is prepared in advance and shared by draft and
    target, Gumbel post, coupling paragraph)."""
    a = wl.gumbel_noise(5, [0, 0, 1], [10, 11, 10], 4096)
    b = wl.gumbel_noise(5, [0], [10], 4096)
    assert np.array_equal(a[0], b[0])
    for i, j in [(0, 1), (0, 2), (1, 2)]:
        r = np.corrcoef(a[i], a[j])[0, 1]
        assert abs(r) < 0.06
    c = wl.gumbel_noise(6, [0], [10], 4096)  # another seed
    assert abs(np.corrcoef(a[0], c[0])[0, 1]) < 0.06


def test_brute_force_prefix_rule_tiny():
    """Every candidate vector over V=3, K=3 (27 cases) against every target
    vector (27 cases): the accepted length is the length of the longest common
    prefix, next is the target token at the first mismatch."""
    V, K = 3, 3
    import itertools

    for tgt in itertools.product(range(V), repeat=K):
        logits = np.full((1, K, V), -5.0, dtype=np.float32)
        for j, t in enumerate(tgt):
            logits[0, j, t] = 5.0
        noise = np.zeros((1, K, V), dtype=np.float32)
        for cand in itertools.product(range(V), repeat=K):
            t, a, nx = oracle.gumbel_verify(logits, noise, np.asarray([cand]))
            assert tuple(t[0]) == tgt
            lcp = 0
            while lcp < K and cand[lcp] == tgt[lcp]:
                lcp += 1
            assert a[0] == lcp
            assert nx[0] == (tgt[lcp] if lcp < K else -1)


def test_exact_fp32_ties_pick_lowest_index():
    """Exact ties in s = fl32(l + g) go to the lowest index, -0 equals +0, and
    a NaN never wins; an all-NaN row resolves to index 0."""
    V = 6
    l = np.zeros((1, 4, V), dtype=np.float32)
    g = np.zeros((1, 4, V), dtype=np.float32)
    l[0, 0] = [1, 3, 3, 0, 3, 2]                 # tie 1/2/4 -> 1
    l[0, 1] = [-0.0, 0.0, -1, -1, -1, -1]        # -0 == +0 -> 0
    l[0, 1, 0] = np.float32(-0.0)
    l[0, 2] = [np.nan, 1, np.nan, 5, 5, np.nan]  # NaN never wins, tie -> 3
    l[0, 3] = np.nan
    t, _, _ = oracle.gumbel_verify(l, g, np.zeros((1, 4), dtype=np.int32))
    assert list(t[0]) == [1, 0, 3, 0]


def test_score_is_a_single_fp32_add():
    """s is fl32(logit + g), not the fp64 sum: two entries whose fp64 sums
    differ but whose fp32 sums tie resolve to the lower index."""
    l = np.array([[[1.0, 1.0]]], dtype=np.float32)
    g = np.array([[[2.0 ** -25, 2.0 ** -24 * 0.75]]], dtype=np.float32)
    # fp64: index 1 is larger; fp32: both round to 1.0 -> tie -> index 0
    assert (1.0 + 2.0 ** -24 * 0.75) > (1.0 + 2.0 ** -25)
    t, _, _ = oracle.gumbel_verify(l, g, np.zeros((1, 1), dtype=np.int32))
    assert t[0, 0] == 0


def test_planted_divergence_is_recovered():
    """Candidates equal to the target up to d, then different: accept == d."""
    R, K, V = 32, 8, 512
    l = wl.normal_f32(30, (R, K, V), std=3.0)
    g = wl.gumbel_noise(33, np.repeat(np.arange(R), K), np.tile(np.arange(K) + 100, R), V).reshape(R, K, V)
    t, _, _ = oracle.gumbel_verify(l, g, np.zeros((R, K), dtype=np.int32))
    d = wl.rng(32).integers(0, K + 1, size=R)
    cand = wl.plant_divergence(t, d, V, 32)
    t2, a, nx = oracle.gumbel_verify(l, g, cand)
    assert np.array_equal(t, t2)
    assert np.array_equal(a, d)
    for r in range(R):
        assert nx[r] == (t[r, d[r]] if d[r] < K else -1)


def test_rollback_rule():
    """LLM-42 post, paragraph 3: keep the accepted prefix, fix the first
    divergence, continue; at least one token is committed per round."""
    cand = np.array([[5, 6, 7, 8], [5, 6, 7, 8], [5, 6, 7, 8]])
    ctx = np.array([100, 200, 300])
    acc = np.array([0, 2, 4])
    nxt = np.array([9, 9, -1])
    new_ctx, committed, t0 = oracle.rollback(ctx, acc, nxt, cand)
    assert list(new_ctx) == [101, 203, 304]
    assert committed == [[9], [5, 6, 9], [5, 6, 7, 8]]
    assert list(t0) == [9, 9, 8]


def test_tile_rule_golden():
    """Spec-dec guide, attention-tile paragraph: G * (1 + D) <= tile, so the
    number of drafts is D = tile/G - 1 (the page prints it garbled); its worked
    numbers are G=8 -> 15 and G=32 -> 3 for tile 128."""
    import json
    import os

    path = os.path.join(os.path.dirname(__file__), "golden", "tile_rule.json")
    with open(path) as f:
        fx = json.load(f)
    for case in fx["cases"]:
        tile, G = fx["tile"], case["G"]
        D = tile // G - 1
        assert G * (1 + D) <= tile < G * (2 + D)
        assert D == case["drafts"]


@pytest.mark.parametrize("logits", [[0.3, -1.0, 2.0, 0.1], [1.0, 1.0, 1.0, 1.0]])
def test_gumbel_topk_is_sampling_without_replacement(logits):
    """Gumbel-top-k (the Gumbel post's "top-k for free"): the first two entries
    of the top-2 of l + g are an ordered draw without replacement from the
    softmax, P(a, b) = p_a p_b / (1 - p_a).  200k noise rows; chi-square over
    the 12 ordered pairs, p > 1e-3.  Ascending order, a reused draw, or a second
    entry taken from the wrong distribution all fail."""
    V, n = len(logits), 200_000
    g = wl.gumbel_noise(seed=9, requests=np.zeros(n, dtype=np.int64), positions=np.arange(n), vocab_size=V)
    l32 = np.broadcast_to(np.asarray(logits, dtype=np.float32), (n, V))
    idx, score = oracle.gumbel_topk(l32, g, 2)
    assert (idx[:, 0] != idx[:, 1]).all() and (score[:, 0] >= score[:, 1]).all()
    p = _softmax(logits)
    pairs = [(a, b) for a in range(V) for b in range(V) if a != b]
    expect = np.array([p[a] * p[b] / (1 - p[a]) for a, b in pairs]) * n
    code = idx[:, 0] * V + idx[:, 1]
    obs = np.array([(code == a * V + b).sum() for a, b in pairs])
    assert obs.sum() == n
    _, pval = stats.chisquare(obs, expect)
    assert pval > 1e-3, (obs, expect, pval)


def test_gumbel_topk_order_ties_nan_and_k1():
    """Descending scores, equal scores in index order, NaN after every real
    score (as -inf, in index order); k = 1 is the Gumbel-max target."""
    l = np.array([[3, 1, 3, np.nan, -np.inf, 3, 2, np.nan]], dtype=np.float32)
    g = np.zeros_like(l)
    idx, score = oracle.gumbel_topk(l, g, 8)
    assert list(idx[0]) == [0, 2, 5, 6, 1, 3, 4, 7]
    assert list(score[0, :5]) == [3, 3, 3, 2, 1] and np.isneginf(score[0, 5:]).all()
    allnan = np.full((1, 5), np.nan, np.float32)
    assert list(oracle.gumbel_topk(allnan, np.zeros_like(allnan), 3)[0][0]) == [0, 1, 2]
    R, K, V = 6, 4, 700
    lr = wl.normal_f32(31, (R, K, V), std=2.0)
    gr = wl.gumbel_noise(34, np.repeat(np.arange(R), K), np.tile(np.arange(K), R), V).reshape(R, K, V)
    lr[0, 0, 5] = lr[0, 0, 9] = np.float32(1e9)  # exact tie
    t, _, _ = oracle.gumbel_verify(lr, gr, np.zeros((R, K), np.int32))
    top1, _ = oracle.gumbel_topk(lr, gr, 1)
    assert np.array_equal(top1[..., 0], t) and t[0, 0] == 5
