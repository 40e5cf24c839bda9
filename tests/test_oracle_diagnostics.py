"""Pins of the diagnostic selectors (oracle/diagnostics.py).

The selectors' recalls are ordered by construction (a per-query choice keeps
at least the mass of any shared choice, the best token set at least that of
the best block set, the best block set at least that of any block set), the
full budget keeps everything, the block oracle is checked against brute force
over all block subsets, and a hand-built case shows mean pooling missing a
high-mass token that the token oracle keeps (recall and output error in
closed form).  k-means is pinned to scikit-learn's Lloyd implementation from
the same initial centres, to planted well-separated clusters and their means,
to the monotone inertia of Lloyd's algorithm and to its tie and empty-cluster
rules; the alignment inflation to closed forms.
"""
import itertools
import math

import numpy as np
import pytest

import oracle
from oracle import diagnostics as dg


def _head(N, D, seed):
    r = np.random.default_rng(seed)
    return r.standard_normal((N, D)), r.standard_normal((N, D)), r.standard_normal((N, D))


@pytest.mark.parametrize("N,C,K", [(512, 64, 128), (700, 128, 256), (300, 64, 64)])
def test_recall_ordering(N, C, K):
    q, k, v = _head(N, 32, N + K)
    scale = 1.5 / math.sqrt(32)
    for perm in (np.arange(N), oracle.pddp(q, C)):
        r = dg.diagnose_head(q, k, v, perm, C, K, scale)
        eps = 1e-12
        assert r["per_query_oracle"]["recall"] >= r["token_oracle"]["recall"] - eps
        assert r["token_oracle"]["recall"] >= r["block_oracle"]["recall"] - eps
        assert r["block_oracle"]["recall"] >= r["mean_pooled_block"]["recall"] - eps
        for s in dg.SELECTORS:
            assert 0.0 < r[s]["recall"] <= 1.0 + eps


def test_full_budget_keeps_everything():
    N, C = 256, 64
    q, k, v = _head(N, 16, 3)
    r = dg.diagnose_head(q, k, v, np.arange(N), C, N, 0.25)
    for s in dg.SELECTORS:
        assert abs(r[s]["recall"] - 1.0) < 1e-12
        assert r[s]["rel_l1"] < 1e-12


def test_block_oracle_is_best_block_set_by_brute_force():
    # N = 6 blocks of 64 keys, one query group, 2 blocks kept: the oracle's
    # recall equals the best over all 15 pairs of blocks
    N, C, K = 6 * dg.KV_BLOCK, 32, 2 * dg.KV_BLOCK
    q, k, v = _head(N, 16, 11)
    scale = 0.4
    perm = np.arange(N)
    q1 = q.copy()
    r = dg.diagnose_head(q1, k, v, perm, N, K, scale)      # one group holding every query
    _, lse = oracle.dense_attention(q, k, v, scale)
    p = np.exp(scale * q @ k.T - lse[:, None])
    best = max(p[:, np.r_[a * 64:(a + 1) * 64, b * 64:(b + 1) * 64]].sum() / N
               for a, b in itertools.combinations(range(6), 2))
    assert abs(r["block_oracle"]["recall"] - best) < 1e-12


def test_mean_pooling_misses_a_high_mass_token():
    # three key blocks of 64: block 0 and 2 orthogonal to the queries (score
    # 0), block 1 anti-aligned on average (score -0.5) but holding one key of
    # score 4.  Mean pooling ranks block 1 last and keeps an orthogonal block;
    # the block oracle keeps block 1; the token oracle keeps the strong key and
    # 63 orthogonal ones.  Closed forms with Z = e^4 + 128 + 63 e^-0.5.
    D, N = 8, 3 * dg.KV_BLOCK
    u = np.zeros(D)
    u[0] = 1.0
    q = np.tile(u, (16, 1))
    k = np.zeros((N, D))
    k[:64, 1] = 1.0
    k[64:128] = -0.5 * u
    k[100] = 4.0 * u
    k[128:, 2] = 1.0
    # V one-hot by key class: score-0 keys -> channel 0, the rest of block 1
    # -> channel 1, the strong key -> channel 2.  The dense output of every
    # query is then its class masses (sum 1), and a selection keeping class
    # masses m_c of total m has output m_c / m, so the relative L1 error is
    # sum_c |m_c / m - p_c| (the same for each tie-break among score-0 keys).
    v = np.zeros((N, D))
    v[:, 0] = 1.0
    v[64:128] = np.eye(D)[1]
    v[100] = np.eye(D)[2]
    r = dg.diagnose_head(q, k, v, np.arange(16), 16, 64, 1.0)
    Z = math.exp(4) + 128 + 63 * math.exp(-0.5)
    a, b, c = 1 / Z, math.exp(-0.5) / Z, math.exp(4) / Z      # one key's probability per class
    dense = (128 * a, 63 * b, c)

    def l1(kept):
        m = sum(kept)
        return sum(abs(kc / m - pc) for kc, pc in zip(kept, dense))

    want = {"mean_pooled_block": (64 * a, 0.0, 0.0),        # block 0
            "block_oracle": (0.0, 63 * b, c),               # block 1
            "token_oracle": (63 * a, 0.0, c),               # key 100 + 63 score-0 keys
            "per_query_oracle": (63 * a, 0.0, c)}
    for sel, kept in want.items():
        assert abs(r[sel]["recall"] - sum(kept)) < 1e-12, sel
        assert abs(r[sel]["rel_l1"] - l1(kept)) < 1e-12, sel
    assert abs(r["mean_pooled_block"]["recall"] - 64 / Z) < 1e-12
    assert abs(r["block_oracle"]["recall"] - (math.exp(4) + 63 * math.exp(-0.5)) / Z) < 1e-12
    assert abs(r["token_oracle"]["recall"] - (math.exp(4) + 63) / Z) < 1e-12


# ---- k-means grouping and alignment inflation -----------------------------

def test_kmeans_matches_scikit_learn_lloyd():
    # same initial centres, run to convergence: identical centres and labels
    from sklearn.cluster import KMeans
    r = np.random.default_rng(7)
    x = np.concatenate([r.normal(m, 1.0, (n, 5)) for m, n in ((0, 80), (4, 50), (-4, 70), (8, 30))])
    init = x[r.choice(len(x), 6, replace=False)]
    lab, cen, _ = dg.kmeans(x, init, 100)
    km = KMeans(n_clusters=6, init=init, n_init=1, max_iter=100, tol=0.0, algorithm="lloyd").fit(x)
    np.testing.assert_allclose(cen, km.cluster_centers_, rtol=0, atol=1e-10)
    np.testing.assert_array_equal(lab, km.labels_)


def test_kmeans_recovers_planted_clusters_and_their_means():
    r = np.random.default_rng(3)
    sizes = (40, 17, 90, 5)
    centres = np.array([[0, 0, 0], [50, 0, 0], [0, 50, 0], [0, 0, 50]], dtype=float)
    x = np.concatenate([c + r.uniform(-1, 1, (n, 3)) for c, n in zip(centres, sizes)])
    truth = np.repeat(np.arange(4), sizes)
    init = x[[0, 40, 57, 147]]                     # one member of each cluster
    lab, cen, inertia = dg.kmeans(x, init, 3)
    np.testing.assert_array_equal(lab, truth)
    for j in range(4):
        np.testing.assert_allclose(cen[j], x[truth == j].mean(axis=0), rtol=0, atol=1e-12)
    groups = dg.cluster_groups(lab, 4)
    assert [g.size for g in groups] == list(sizes)
    assert dg.alignment_inflation([g.size for g in groups], 64) == pytest.approx((64 + 64 + 128 + 64) / 152)


def test_kmeans_inertia_never_rises_and_ties_go_to_the_smaller_centre():
    r = np.random.default_rng(11)
    x = r.standard_normal((300, 4))
    _, _, inertia = dg.kmeans(x, x[:12], 25)
    assert np.all(np.diff(inertia) <= 1e-9)
    lab, _, _ = dg.kmeans(np.zeros((1, 2)), np.array([[-1.0, 0.0], [1.0, 0.0]]), 1)
    assert lab[0] == 0
    # an empty cluster keeps its centre
    lab, cen, _ = dg.kmeans(np.array([[0.0], [0.1]]), np.array([[0.0], [100.0]]), 2)
    assert list(lab) == [0, 0] and cen[1, 0] == 100.0


@pytest.mark.parametrize("sizes,tile,want", [([64, 64], 64, 1.0), ([65, 63], 64, 1.5),
                                              ([1] * 10, 8, 8.0), ([128, 1, 127], 128, 384 / 256)])
def test_alignment_inflation_closed_forms(sizes, tile, want):
    assert dg.alignment_inflation(sizes, tile) == pytest.approx(want, rel=1e-15)


def test_budgets_in_one_call_equal_separate_calls_and_kmeans_groups_keep_the_ordering():
    N, C = 384, 64
    q, k, v = _head(N, 16, 21)
    r = np.random.default_rng(22)
    lab, _, _ = dg.kmeans(q, q[r.choice(N, N // C, replace=False)], 10)
    groups = [g for g in dg.cluster_groups(lab, N // C) if g.size]
    both = dg.diagnose_groups(q, k, v, groups, [64, 128], 0.3)
    for K in (64, 128):
        one = dg.diagnose_groups(q, k, v, groups, [K], 0.3)[K]
        for s in dg.SELECTORS:
            assert both[K][s]["recall"] == pytest.approx(one[s]["recall"], rel=1e-13)
            assert both[K][s]["rel_l1"] == pytest.approx(one[s]["rel_l1"], rel=1e-13)
        r_ = both[K]
        assert r_["per_query_oracle"]["recall"] >= r_["token_oracle"]["recall"] - 1e-12
        assert r_["token_oracle"]["recall"] >= r_["block_oracle"]["recall"] - 1e-12
        assert r_["block_oracle"]["recall"] >= r_["mean_pooled_block"]["recall"] - 1e-12


@pytest.mark.parametrize("dup", [False, True])
def test_per_query_oracle_equals_brute_force_masking(dup):
    # every row keeps its K largest probabilities; recall and output error
    # recomputed here from a dense mask and a plain product, several budgets.
    # dup: keys repeated in pairs, so every probability ties with its twin and
    # the rule for a tie at the K-th value (smaller key id kept) decides which
    # value row enters the output (the value rows stay distinct)
    N, C = 300, 64
    q, k, v = _head(N, 8, 31)
    if dup:
        k[1::2] = k[0::2]
    scale = 0.5
    groups = dg.groups_from_perm(np.random.default_rng(32).permutation(N), C)
    Ks = [1, 37, 128, 299, 300]
    got = dg.diagnose_groups(q, k, v, groups, Ks, scale)
    o, lse = oracle.dense_attention(q, k, v, scale)
    p = np.exp(scale * q @ k.T - lse[:, None])
    for K in Ks:
        keep = np.zeros_like(p, dtype=bool)
        for i in range(N):
            keep[i, np.argsort(-p[i], kind="stable")[:K]] = True
        pm = np.where(keep, p, 0.0)
        kept = pm.sum(axis=1)
        assert got[K]["per_query_oracle"]["recall"] == pytest.approx(kept.mean(), rel=1e-12)
        err = np.abs(pm @ v / kept[:, None] - o).sum() / np.abs(o).sum()
        assert got[K]["per_query_oracle"]["rel_l1"] == pytest.approx(err, rel=1e-10, abs=1e-14)


def test_mean_pooling_uses_each_groups_own_mean_query():
    # two groups that prefer different key blocks: group A points at block 0,
    # group B (fewer, shorter queries) at block 1.  Pooling each group's own
    # mean query picks each group's block, as the block oracle does; the mean
    # over all queries would point both groups at block 0
    r = np.random.default_rng(51)
    D, B = 4, dg.KV_BLOCK
    e = np.eye(D)
    k = np.concatenate([3 * e[0] + 0.05 * r.standard_normal((B, D)),
                        3 * e[1] + 0.05 * r.standard_normal((B, D))])
    v = r.standard_normal((2 * B, D))
    q = np.concatenate([2 * e[0] + 0.05 * r.standard_normal((96, D)),
                        1.5 * e[1] + 0.05 * r.standard_normal((32, D))])
    groups = [np.arange(96), np.arange(96, 128)]
    got = dg.diagnose_groups(q, k, v, groups, [B], 1.0)[B]
    assert got["mean_pooled_block"]["recall"] == pytest.approx(got["block_oracle"]["recall"], rel=1e-12)
    assert got["mean_pooled_block"]["rel_l1"] == pytest.approx(got["block_oracle"]["rel_l1"], rel=1e-12)
    assert got["mean_pooled_block"]["recall"] > 0.95


def test_scoring_a_sample_of_groups_averages_over_their_queries():
    # recall is a mean over the queries the given groups hold: scoring the
    # groups one at a time and weighting by group size gives the full result
    N, C = 320, 64
    q, k, v = _head(N, 8, 41)
    groups = dg.groups_from_perm(np.random.default_rng(42).permutation(N), C)
    full = dg.diagnose_groups(q, k, v, groups, [64], 0.4)[64]
    for s in dg.SELECTORS:
        parts = [dg.diagnose_groups(q, k, v, [g], [64], 0.4)[64][s]["recall"] * len(g) for g in groups]
        assert sum(parts) / N == pytest.approx(full[s]["recall"], rel=1e-12)


def test_mean_pooled_blocks_closed_form():
    # keys in 4 blocks of 64 whose means point along e0, e1, -e0 and 2 e1; a
    # query block with mean 3 e1 + e0 scores them 3s, ... so with budget 128
    # (two blocks) the blocks are {1, 3} and with 64 just {3}
    from oracle import diagnostics as dg
    N, D = 256, 4
    k = np.zeros((N, D))
    means = [np.eye(D)[0], np.eye(D)[1], -np.eye(D)[0], 2 * np.eye(D)[1]]
    rng = np.random.default_rng(33)
    for b, m in enumerate(means):
        noise = rng.standard_normal((64, D))
        noise -= noise.mean(axis=0)                    # block mean exactly m
        k[64 * b:64 * (b + 1)] = m + 0.1 * noise
    kbar = dg.block_means(k)
    np.testing.assert_allclose(kbar, np.stack(means), atol=1e-14)
    q = np.tile(np.array([1.0, 3.0, 0.0, 0.0]), (10, 1))
    np.testing.assert_allclose(dg.mean_pooled_scores(q, kbar, np.arange(10), 0.5),
                               0.5 * np.array([1.0, 3.0, -1.0, 6.0]), atol=1e-14)
    assert dg.mean_pooled_blocks(q, kbar, np.arange(10), 128, 0.5).tolist() == [1, 3]
    assert dg.mean_pooled_blocks(q, kbar, np.arange(10), 64, 0.5).tolist() == [3]
    # ties go to the smaller block id
    kt = np.zeros((192, D))
    assert dg.mean_pooled_blocks(q, dg.block_means(kt), np.arange(10), 128, 0.5).tolist() == [0, 1]
