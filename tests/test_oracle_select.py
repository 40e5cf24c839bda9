"""Pins of the oracle's group mass, top-K selection and retained mass.

Ties: brute force over all K-subsets on tiny inputs (the selected set must carry
the largest retained mass), closed forms (masses of a group sum to its size),
hand-made tie cases, and an independent library selection (heapq.nlargest).
"""
import heapq
import itertools
import math

import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed, scale=1.0):
    return scale * np.random.default_rng(seed).standard_normal(shape)


def _setup(n=50, d=8, C=8, seed=0):
    q, k = _rand((n, d), seed, 1.5), _rand((n, d), seed + 1, 1.5)
    scale = 1 / math.sqrt(d)
    _, lse = oracle.dense_attention(q, k, _rand((n, d), seed + 2), scale)
    perm = np.random.default_rng(seed + 3).permutation(n)
    return q, k, lse, perm, C, scale


def test_group_mass_sums_to_group_size():
    q, k, lse, perm, C, scale = _setup(n=50, C=8)   # 6 groups of 8 and one of 2
    mass = oracle.group_mass(q, k, lse, perm, C, scale)
    sizes = [len(g) for g in oracle.groups_from_perm(perm, C)]
    assert sizes == [8] * 6 + [2]
    np.testing.assert_allclose(mass.sum(axis=1), sizes, atol=1e-10)


def test_group_mass_against_torch_softmax():
    q, k, lse, perm, C, scale = _setup(n=40, C=8, seed=10)
    mass = oracle.group_mass(q, k, lse, perm, C, scale)
    p = torch.softmax(scale * torch.from_numpy(q) @ torch.from_numpy(k).T, dim=1).numpy()
    for g, members in enumerate(oracle.groups_from_perm(perm, C)):
        np.testing.assert_allclose(mass[g], p[members].sum(axis=0), atol=1e-13)


def test_singleton_group_mass_is_probability_row():
    q, k, lse, perm, _, scale = _setup(n=12, C=1, seed=20)
    mass = oracle.group_mass(q, k, lse, perm, 1, scale)
    p = oracle.probabilities(q, k, lse, scale)
    np.testing.assert_allclose(mass, p[perm], atol=1e-15)


@pytest.mark.parametrize("mass,K,expected", [
    ([0.5, 0.2, 0.5, 0.2, 0.1], 2, [0, 2]),
    ([0.5, 0.2, 0.5, 0.2, 0.1], 3, [0, 1, 2]),      # 0.2 tie -> smaller id 1
    ([0.5, 0.2, 0.5, 0.2, 0.1], 4, [0, 1, 2, 3]),
    ([0.1, 0.1, 0.1, 0.1], 2, [0, 1]),
    ([0.0, 0.3, 0.0, 0.7, 0.0, 0.0], 3, [0, 1, 3]),
    ([0.25, 0.75], 2, [0, 1]),
    ([0.9], 1, [0]),
])
def test_topk_hand_cases(mass, K, expected):
    assert oracle.topk_indices(np.array(mass), K).tolist() == expected


def test_topk_compares_in_the_given_precision():
    # 1 + 2^-30 and 1 are distinct in float64 but equal in float32
    row64 = np.array([1.0, 1.0 + 2.0 ** -30, 0.5])
    assert oracle.topk_indices(row64, 1).tolist() == [1]
    assert oracle.topk_indices(row64.astype(np.float32), 1).tolist() == [0]


@pytest.mark.parametrize("seed", range(6))
def test_topk_is_optimal_by_brute_force(seed):
    q, k, lse, perm, C, scale = _setup(n=12, d=4, C=4, seed=100 + seed)
    for K in range(1, 6):
        idx, mass = oracle.select(q, k, lse, perm, C, K, scale)
        rho = oracle.retained_mass(mass, idx)
        for g in range(mass.shape[0]):
            best = max(mass[g, list(s)].sum() for s in itertools.combinations(range(12), K))
            assert rho[g] == pytest.approx(best, abs=1e-14)
            assert len(set(idx[g].tolist())) == K
            assert (np.diff(idx[g]) > 0).all()


def test_topk_matches_heapq():
    rng = np.random.default_rng(5)
    row = np.round(rng.random(300), 2)       # many ties
    for K in (1, 7, 150, 299, 300):
        ref = heapq.nlargest(K, range(300), key=lambda j: (row[j], -j))
        assert oracle.topk_indices(row, K).tolist() == sorted(ref)


def test_retained_mass_monotone_and_full():
    q, k, lse, perm, C, scale = _setup(n=48, C=16, seed=30)
    prev = None
    for K in (1, 5, 12, 30, 48):
        idx, mass = oracle.select(q, k, lse, perm, C, K, scale)
        rho = oracle.retained_mass(mass, idx)
        if prev is not None:
            assert (rho >= prev - 1e-15).all()
        prev = rho
    np.testing.assert_allclose(prev, 16.0, atol=1e-10)


def test_select_bh_shapes():
    q = _rand((1, 2, 30, 8), 40)
    k = _rand((1, 2, 30, 8), 41)
    _, lse = oracle.dense_attention_bh(q, k, _rand((1, 2, 30, 8), 42), 0.3)
    perm = np.stack([np.stack([np.arange(30), np.arange(30)[::-1]])])
    idx, mass = oracle.select_bh(q, k, lse, perm, 8, 5, 0.3)
    assert idx.shape == (1, 2, 4, 5) and mass.shape == (1, 2, 4, 30)


# ---- per-query selection statistics: sparse LSE and kept (recalled) mass ----

def test_sparse_lse_and_kept_mass_two_keys():
    # one query, keys with scores 1 and 3 (scale 1): selecting key 0 keeps
    # e/(e + e^3) of the mass, and its sparse LSE is the score itself
    q = np.array([[1.0, 0.0]])
    k = np.array([[1.0, 0.0], [3.0, 0.0]])
    _, lse = oracle.dense_attention(q, k, k, 1.0)
    assert oracle.sparse_lse(q, k, np.array([0]), [np.array([0])], 1, 1.0)[0] == pytest.approx(1.0, abs=1e-15)
    kept = oracle.kept_mass(q, k, lse, np.array([0]), [np.array([0])], 1, 1.0)[0]
    assert kept == pytest.approx(np.e / (np.e + np.e ** 3), rel=1e-14)


def test_sparse_lse_full_budget_is_dense_lse_and_recall_is_one():
    rng = np.random.default_rng(31)
    N, D, C = 70, 8, 16
    q, k = rng.standard_normal((N, D)), rng.standard_normal((N, D))
    perm = rng.permutation(N)
    G = -(-N // C)
    full = [np.arange(N)] * G
    _, lse = oracle.dense_attention(q, k, k, 0.4)
    np.testing.assert_allclose(oracle.sparse_lse(q, k, perm, full, C, 0.4), lse, rtol=0, atol=1e-12)
    np.testing.assert_allclose(oracle.kept_mass(q, k, lse, perm, full, C, 0.4), 1.0, rtol=0, atol=1e-12)


def test_kept_mass_matches_lse_gap_and_group_retained_mass():
    rng = np.random.default_rng(32)
    N, D, C, K = 90, 6, 16, 20
    q, k = rng.standard_normal((N, D)), rng.standard_normal((N, D))
    perm = rng.permutation(N)
    _, lse = oracle.dense_attention(q, k, k, 0.5)
    idx, mass = oracle.select(q, k, lse, perm, C, K, 0.5)
    kept = oracle.kept_mass(q, k, lse, perm, idx, C, 0.5)
    # the same quantity through the sparse normaliser
    np.testing.assert_allclose(kept, np.exp(oracle.sparse_lse(q, k, perm, idx, C, 0.5) - lse), rtol=1e-12)
    # summed over a group it is the group's retained mass
    rho = oracle.retained_mass(mass, idx)
    for g, members in enumerate(oracle.groups_from_perm(perm, C)):
        assert kept[members].sum() == pytest.approx(rho[g], rel=1e-12)
    assert (kept <= 1 + 1e-12).all()
    # per-group budgets of any length, monotone in the budget
    short = [ids[: 5 + g] for g, ids in enumerate(idx)]
    kept_short = oracle.kept_mass(q, k, lse, perm, short, C, 0.5)
    assert (kept_short <= kept + 1e-15).all()
