"""Pins of the oracle's dense attention, LSE and probability recovery.

Each test ties ``oracle.dense_attention`` / ``oracle.probabilities`` to
something other than the oracle itself: a hand-derived closed form, softmax
invariants, special cases with known answers, and independent library
routines (scipy's logsumexp, torch's scaled_dot_product_attention in float64
on the CPU).
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle


def _rand(shape, seed, scale=1.0):
    return scale * np.random.default_rng(seed).standard_normal(shape)


def test_two_key_closed_form():
    # scores 0 and ln 3 -> probabilities 1/4, 3/4; lse = ln 4; output 1/4 v0 + 3/4 v1
    q = np.array([[1.0, 0.0]])
    k = np.array([[0.0, 0.0], [math.log(3.0), 0.0]])
    v = np.array([[4.0, -2.0], [0.0, 2.0]])
    out, lse = oracle.dense_attention(q, k, v, 1.0)
    assert lse[0] == pytest.approx(math.log(4.0), abs=1e-15)
    np.testing.assert_allclose(out, [[1.0, 1.0]], atol=1e-15)
    np.testing.assert_allclose(oracle.probabilities(q, k, lse, 1.0), [[0.25, 0.75]], atol=1e-15)


def test_rows_sum_to_one():
    q, k = _rand((37, 16), 1), _rand((53, 16), 2)
    _, lse = oracle.dense_attention(q, k, _rand((53, 16), 3), 0.25)
    p = oracle.probabilities(q, k, lse, 0.25)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12)
    assert (p >= 0).all()


def test_lse_matches_scipy_logsumexp():
    q, k = _rand((40, 32), 4, 3.0), _rand((70, 32), 5, 3.0)
    scale = 1 / math.sqrt(32)
    _, lse = oracle.dense_attention(q, k, _rand((70, 32), 6), scale)
    ref = scipy.special.logsumexp(scale * np.einsum("id,jd->ij", q, k), axis=1)
    np.testing.assert_allclose(lse, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n,m,d", [(1, 1, 8), (17, 33, 64), (600, 700, 128)])
def test_dense_matches_torch_sdpa_fp64(n, m, d):
    q, k, v = _rand((n, d), 7, 2.0), _rand((m, d), 8, 2.0), _rand((m, d), 9)
    scale = 1 / math.sqrt(d)
    out, _ = oracle.dense_attention(q, k, v, scale)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        scale=scale)[0].numpy()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_zero_queries_average_values():
    v = _rand((29, 8), 10)
    out, lse = oracle.dense_attention(np.zeros((5, 8)), _rand((29, 8), 11), v, 0.3)
    np.testing.assert_allclose(out, np.broadcast_to(v.mean(axis=0), out.shape), atol=1e-14)
    np.testing.assert_allclose(lse, math.log(29.0), atol=1e-14)


def test_single_token_returns_its_value():
    v = _rand((1, 8), 12)
    out, _ = oracle.dense_attention(_rand((1, 8), 13), _rand((1, 8), 14), v, 0.5)
    np.testing.assert_allclose(out, v, atol=1e-15)


def test_dominant_key_selects_its_value():
    k = _rand((10, 4), 15)
    q = 200.0 * k[3:4] / np.linalg.norm(k[3])
    k[np.arange(10) != 3] *= 0.01
    v = _rand((10, 4), 16)
    out, _ = oracle.dense_attention(q, k, v, 1.0)
    np.testing.assert_allclose(out[0], v[3], atol=1e-12)


def test_key_shift_moves_lse_not_output():
    # adding c to every key adds scale*q_i.c to row i's scores: softmax unchanged,
    # lse shifted by exactly that amount (catches a max/sum over the wrong axis)
    q, k, v = _rand((9, 6), 17), _rand((15, 6), 18), _rand((15, 6), 19)
    c = _rand((6,), 20)
    o1, l1 = oracle.dense_attention(q, k, v, 0.7)
    o2, l2 = oracle.dense_attention(q, k + c, v, 0.7)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(l2 - l1, 0.7 * q @ c, atol=1e-12)


def test_large_logits_are_stable():
    q, k, v = _rand((8, 16), 21, 40.0), _rand((12, 16), 22, 40.0), _rand((12, 16), 23)
    out, lse = oracle.dense_attention(q, k, v, 1.0)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    p = oracle.probabilities(q, k, lse, 1.0)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12)


def test_row_blocking_is_invisible():
    q, k, v = _rand((1300, 8), 24), _rand((40, 8), 25), _rand((40, 8), 26)
    out, lse = oracle.dense_attention(q, k, v, 0.5)
    for i in (0, 511, 512, 1023, 1299):
        o1, l1 = oracle.dense_attention(q[i:i + 1], k, v, 0.5)
        np.testing.assert_allclose(out[i], o1[0], atol=1e-15)
        assert lse[i] == pytest.approx(l1[0], abs=1e-15)


def test_batched_wrapper_loops_heads():
    q = _rand((2, 3, 20, 8), 27)
    k = _rand((2, 3, 20, 8), 28)
    v = _rand((2, 3, 20, 8), 29)
    out, lse = oracle.dense_attention_bh(q, k, v, 0.3)
    assert out.shape == (2, 3, 20, 8) and lse.shape == (2, 3, 20)
    o, l = oracle.dense_attention(q[1, 2], k[1, 2], v[1, 2], 0.3)
    np.testing.assert_array_equal(out[1, 2], o)
    np.testing.assert_array_equal(lse[1, 2], l)
