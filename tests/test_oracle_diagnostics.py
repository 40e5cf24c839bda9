"""Pins of the diagnostic selectors (oracle/diagnostics.py).

The selectors' recalls are ordered by construction (a per-query choice keeps
at least the mass of any shared choice, the best token set at least that of
the best block set, the best block set at least that of any block set), the
full budget keeps everything, the block oracle is checked against brute force
over all block subsets, and a hand-built case shows mean pooling missing a
high-mass token that the token oracle keeps (recall and output error in
closed form).
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
