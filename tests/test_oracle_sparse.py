"""Pins of the oracle's token-sparse attention, residual and anchor/reuse steps.

Special cases with known answers (full budget equals dense attention, a budget
of one returns that token's value), invariance to the order of the selected
ids, the anchor identity sparse + residual = dense, and an independent library
routine (torch's scaled_dot_product_attention on the gathered keys, float64).
"""
import math

import numpy as np
import torch

import oracle


def _rand(shape, seed, scale=1.0):
    return scale * np.random.default_rng(seed).standard_normal(shape)


def _inputs(n=45, d=8, seed=0):
    return _rand((n, d), seed, 1.5), _rand((n, d), seed + 1, 1.5), _rand((n, d), seed + 2)


def test_full_budget_equals_dense():
    q, k, v = _inputs(n=45)
    scale = 1 / math.sqrt(8)
    perm = np.random.default_rng(3).permutation(45)
    G = -(-45 // 8)
    idx = np.broadcast_to(np.arange(45), (G, 45))
    dense, _ = oracle.dense_attention(q, k, v, scale)
    np.testing.assert_allclose(oracle.sparse_attention(q, k, v, perm, idx, 8, scale), dense, atol=1e-12)


def test_budget_one_returns_that_value():
    q, k, v = _inputs(n=30, seed=10)
    perm = np.arange(30)
    idx = np.array([[7], [0], [29], [3]])
    out = oracle.sparse_attention(q, k, v, perm, idx, 8, 0.4)
    for g in range(4):
        np.testing.assert_allclose(out[g * 8:(g + 1) * 8], np.broadcast_to(v[idx[g, 0]], out[g * 8:(g + 1) * 8].shape), atol=1e-15)


def test_order_of_selected_ids_is_irrelevant():
    q, k, v = _inputs(n=40, seed=20)
    rng = np.random.default_rng(21)
    perm = rng.permutation(40)
    idx = np.stack([np.sort(rng.choice(40, 9, replace=False)) for _ in range(5)])
    shuffled = np.stack([rng.permutation(r) for r in idx])
    a = oracle.sparse_attention(q, k, v, perm, idx, 8, 0.3)
    b = oracle.sparse_attention(q, k, v, perm, shuffled, 8, 0.3)
    np.testing.assert_allclose(a, b, atol=1e-14)


def test_sparse_matches_torch_on_gathered_keys():
    q, k, v = _inputs(n=50, d=16, seed=30)
    rng = np.random.default_rng(31)
    perm = rng.permutation(50)
    C, K = 16, 11
    idx = np.stack([np.sort(rng.choice(50, K, replace=False)) for _ in range(4)])
    out = oracle.sparse_attention(q, k, v, perm, idx, C, 0.25)
    for g, members in enumerate(oracle.groups_from_perm(perm, C)):
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[members])[None], torch.from_numpy(k[idx[g]])[None],
            torch.from_numpy(v[idx[g]])[None], scale=0.25)[0].numpy()
        np.testing.assert_allclose(out[members], ref, atol=1e-12)


def test_residual_is_added():
    q, k, v = _inputs(n=20, seed=40)
    perm = np.arange(20)
    idx = np.stack([np.arange(5), np.arange(5, 10), np.arange(10, 15)])
    r = _rand((20, 8), 41)
    a = oracle.sparse_attention(q, k, v, perm, idx, 8, 0.5)
    b = oracle.sparse_attention(q, k, v, perm, idx, 8, 0.5, residual=r)
    np.testing.assert_allclose(b - a, r, atol=1e-14)


def test_anchor_identity_and_reuse():
    q, k, v = _inputs(n=64, d=8, seed=50)
    scale = 1 / math.sqrt(8)
    st = oracle.anchor_step(q, k, v, C=8, K=12, scale=scale)
    np.testing.assert_allclose(st["o_sparse"] + st["residual"], st["out"], atol=1e-12)
    dense, _ = oracle.dense_attention(q, k, v, scale)
    np.testing.assert_array_equal(st["out"], dense)
    # reuse with the anchor's own inputs reproduces the dense output
    again = oracle.reuse_step(q, k, v, st["perm"], st["idx"], st["residual"], 8, scale)
    np.testing.assert_allclose(again, dense, atol=1e-12)
    # at full budget the residual vanishes
    full = oracle.anchor_step(q, k, v, C=8, K=64, scale=scale)
    np.testing.assert_allclose(full["residual"], 0.0, atol=1e-12)


def test_sparse_bh_wrapper():
    q = _rand((1, 2, 24, 8), 60)
    k = _rand((1, 2, 24, 8), 61)
    v = _rand((1, 2, 24, 8), 62)
    perm = np.stack([np.stack([np.arange(24), np.arange(24)[::-1]])])
    idx = np.tile(np.arange(6), (1, 2, 3, 1))
    out = oracle.sparse_attention_bh(q, k, v, perm, idx, 8, 0.3)
    np.testing.assert_array_equal(out[0, 1], oracle.sparse_attention(q[0, 1], k[0, 1], v[0, 1], perm[0, 1], idx[0, 1], 8, 0.3))
