"""GPU parity of mcs_dense_attn, mcs_sparse_attn and mcs_residual_update.

Every GPU call goes through the C ABI (via the ctypes binding); the expected
values come from the fp64 oracle on the very same bf16 inputs.  Shapes span
several tiles with ragged tails (N, K not multiples of the 64-key tile, a short
last query group), both head dimensions and both group sizes.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from token_sparse_attention_amd import accounting, synth
from tests.helpers import (assert_output_close, bf16_to_f64, to_dev, to_dev_bf16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mcs():
    from token_sparse_attention_amd import binding
    return binding


def _qkv(B, H, N, D, seed, scale=1.0):
    q = synth.gaussian((B, H, N, D), seed, scale)
    k = synth.gaussian((B, H, N, D), seed + 1, scale)
    v = synth.gaussian((B, H, N, D), seed + 2)
    return q, k, v


@pytest.mark.parametrize("B,H,N,D", [(1, 2, 1000, 128), (2, 1, 333, 64), (1, 1, 37, 128), (1, 3, 1, 64),
                                     (1, 1, 129, 64), (1, 1, 64, 128)])
def test_dense_matches_oracle(mcs, B, H, N, D):
    q, k, v = _qkv(B, H, N, D, seed=N + D, scale=1.5)
    scale = 1 / math.sqrt(D)
    o, lse = mcs.dense_attn(to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), scale, want_lse=True)
    o_nolse = mcs.dense_attn(to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), scale)
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle.dense_attention_bh(synth.to_f64(q), synth.to_f64(k), synth.to_f64(v), scale)
    assert_output_close(bf16_to_f64(o), ref_o, "dense O")
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=0, atol=2e-3)
    # without the LSE the kernel defers its row max (another rounding order)
    assert_output_close(bf16_to_f64(o_nolse), ref_o, "dense O without LSE")


def test_dense_large_logits(mcs):
    # peaked softmax: scores of order 50
    q, k, v = _qkv(1, 1, 300, 64, seed=77, scale=3.0)
    o, lse = mcs.dense_attn(to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), 1.0, want_lse=True)
    ref_o, ref_lse = oracle.dense_attention_bh(synth.to_f64(q), synth.to_f64(k), synth.to_f64(v), 1.0)
    assert_output_close(bf16_to_f64(o), ref_o, "dense O")
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=1e-5, atol=2e-3)


@pytest.mark.parametrize("D", [64, 128])
def test_dense_reference_moves_many_times(mcs, D):
    """Scores climb by ~4.5 (6.5 in log2 units) per 64-key tile, so the
    running reference maximum moves again and again (O and the sums are
    rescaled each time) and the last tile dominates the softmax."""
    q, k, v = synth.growing_scores(1000, D, seed=31, step=1.5)
    o, lse = mcs.dense_attn(to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), 1.0, want_lse=True)
    o32 = mcs.dense_attn(to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), 1.0, out_dtype=torch.float32)
    ref_o, ref_lse = oracle.dense_attention_bh(synth.to_f64(q), synth.to_f64(k), synth.to_f64(v), 1.0)
    assert ref_lse.max() > 60.0          # the regime the test is about
    assert_output_close(o32.cpu().numpy().astype(np.float64), ref_o, "dense O (fp32 out)")
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=1e-5, atol=2e-3)


@pytest.mark.parametrize("ascending", [True, False])
def test_sparse_reference_moves_many_times(mcs, ascending):
    """The same climbing scores through gathered ids: ascending ids make each
    later tile outrank the earlier ones (the reference moves), descending ids
    put the largest scores in the first tile (it never moves)."""
    N, D, C, K = 1000, 128, 128, 400
    q, k, v = synth.growing_scores(N, D, seed=32, step=1.5)
    G = accounting.num_groups(N, C)
    perm = synth.random_perm(1, 1, N, seed=33)
    idx = synth.random_index_sets(1, 1, G, K, N, seed=34)
    if not ascending:
        idx = np.ascontiguousarray(idx[..., ::-1])
    o = mcs.sparse_attn(to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), to_dev(perm), to_dev(idx), C, scale=1.0,
                        out_dtype=torch.float32)
    ref = oracle.sparse_attention_bh(synth.to_f64(q), synth.to_f64(k), synth.to_f64(v), perm, idx, C, 1.0)
    assert_output_close(o.cpu().numpy().astype(np.float64), ref, "sparse O (fp32 out)")


@pytest.mark.parametrize("D", [64, 128])
def test_reference_jumps_past_fp32_range(mcs, D):
    """Each 64-key tile outscores the one before by about 170 in log2 units,
    so exponentials taken against the old reference overflow to inf: the
    kernels without an LSE output must see that in the tile's P sum, move the
    reference and take the tile's exponentials again (dense and sparse)."""
    N, C, K = 400, 128, 300
    q, k, v = synth.growing_scores(N, D, seed=35, step=40.0)
    qf, kf, vf = synth.to_f64(q), synth.to_f64(k), synth.to_f64(v)
    ref_o, ref_lse = oracle.dense_attention_bh(qf, kf, vf, 1.0)
    assert ref_lse.min() > 300.0   # every row ends > 2^128 (in P) above its first tile's scores
    o32 = mcs.dense_attn(to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), 1.0, out_dtype=torch.float32)
    assert_output_close(o32.cpu().numpy().astype(np.float64), ref_o, "dense O (fp32 out)")
    o, lse = mcs.dense_attn(to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), 1.0, want_lse=True)
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=1e-5, atol=2e-3)
    G = accounting.num_groups(N, C)
    perm = synth.random_perm(1, 1, N, seed=36)
    idx = synth.random_index_sets(1, 1, G, K, N, seed=37)
    o = mcs.sparse_attn(to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), to_dev(perm), to_dev(idx), C, scale=1.0,
                        out_dtype=torch.float32)
    ref = oracle.sparse_attention_bh(qf, kf, vf, perm, idx, C, 1.0)
    assert_output_close(o.cpu().numpy().astype(np.float64), ref, "sparse O (fp32 out)")


SPARSE_CASES = [
    # B, H, N, D, C, K
    (1, 2, 1000, 128, 128, 200),
    (1, 1, 1000, 128, 64, 65),
    (2, 1, 700, 64, 64, 257),
    (1, 2, 513, 64, 128, 1),
    (1, 1, 300, 128, 128, 300),
    (1, 1, 50, 64, 64, 7),
]


@pytest.mark.parametrize("B,H,N,D,C,K", SPARSE_CASES)
@pytest.mark.parametrize("with_res", [False, True])
def test_sparse_matches_oracle(mcs, B, H, N, D, C, K, with_res):
    q, k, v = _qkv(B, H, N, D, seed=3 * N + K, scale=1.5)
    G = accounting.num_groups(N, C)
    perm = synth.random_perm(B, H, N, seed=N)
    idx = synth.random_index_sets(B, H, G, K, N, seed=K)
    res = synth.gaussian((B, H, N, D), seed=11, scale=0.1) if with_res else None
    scale = 1 / math.sqrt(D)
    o = mcs.sparse_attn(to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), to_dev(perm), to_dev(idx), C,
                        residual=to_dev_bf16(res) if with_res else None, scale=scale)
    ref = oracle.sparse_attention_bh(synth.to_f64(q), synth.to_f64(k), synth.to_f64(v), perm, idx, C, scale,
                                     residual=synth.to_f64(res) if with_res else None)
    assert_output_close(bf16_to_f64(o), ref, "sparse O")


def test_sparse_unsorted_ids_and_full_budget(mcs):
    B, H, N, D, C = 1, 1, 400, 128, 128
    q, k, v = _qkv(B, H, N, D, seed=5, scale=1.5)
    G = accounting.num_groups(N, C)
    perm = synth.random_perm(B, H, N, seed=6)
    idx = synth.random_index_sets(B, H, G, 150, N, seed=7)
    shuffled = np.ascontiguousarray(idx[..., ::-1])
    dq, dk, dv = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    a = mcs.sparse_attn(dq, dk, dv, to_dev(perm), to_dev(idx), C)
    b = mcs.sparse_attn(dq, dk, dv, to_dev(perm), to_dev(shuffled), C)
    ref = oracle.sparse_attention_bh(synth.to_f64(q), synth.to_f64(k), synth.to_f64(v), perm, idx, C, 1 / math.sqrt(D))
    assert_output_close(bf16_to_f64(a), ref)
    assert_output_close(bf16_to_f64(b), ref)
    # K = N: every group attends to all keys -> dense attention
    full = np.broadcast_to(np.arange(N, dtype=np.int32), (B, H, G, N)).copy()
    o_full = mcs.sparse_attn(dq, dk, dv, to_dev(perm), to_dev(full), C)
    o_dense = mcs.dense_attn(dq, dk, dv)
    ref_dense, _ = oracle.dense_attention_bh(synth.to_f64(q), synth.to_f64(k), synth.to_f64(v), 1 / math.sqrt(D))
    assert_output_close(bf16_to_f64(o_full), ref_dense)
    assert_output_close(bf16_to_f64(o_full), bf16_to_f64(o_dense), "sparse(K=N) vs dense")


def test_residual_update_exact(mcs):
    a = synth.gaussian((3, 1001), seed=21)
    b = synth.gaussian((3, 1001), seed=22, scale=0.5)
    r = mcs.residual_update(to_dev_bf16(a), to_dev_bf16(b))
    # exact: bf16 round-to-nearest-even of the fp32 difference of two bf16 values
    expect = synth.to_bf16_bits((synth.to_f32(a) - synth.to_f32(b)).astype(np.float32))
    got = r.view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got, expect)


@pytest.mark.parametrize("alias", ["o_dense", "o_sparse"])
def test_residual_update_in_place(mcs, alias):
    # 3090 elements: 386 16-byte vectors and a 2-element tail
    a = synth.gaussian((2, 3, 515), seed=23)
    b = synth.gaussian((2, 3, 515), seed=24, scale=0.5)
    expect = synth.to_bf16_bits((synth.to_f32(a) - synth.to_f32(b)).astype(np.float32))
    da, db = to_dev_bf16(a), to_dev_bf16(b)
    out = da if alias == "o_dense" else db
    r = mcs.residual_update(da, db, out=out)
    assert r.data_ptr() == out.data_ptr()
    np.testing.assert_array_equal(r.view(torch.int16).cpu().numpy().view(np.uint16), expect)


@pytest.mark.parametrize("D", [64, 128])
def test_sparse_out_of_range_ids_read_zero_rows(mcs, D):
    # ids past N, far past N (id * row bytes would wrap 32 bits) and negative
    # ids each read a zero key and value row
    B, H, N, C, K = 1, 1, 300, 128, 70
    q, k, v = _qkv(B, H, N, D, seed=41, scale=1.5)
    G = accounting.num_groups(N, C)
    perm = synth.random_perm(B, H, N, seed=42)
    idx = synth.random_index_sets(B, H, G, K, N, seed=43)
    bad = idx.copy()
    wrap = 2 ** 32 // (2 * D)             # id whose row offset wraps to 0 in 32 bits
    bad[0, 0, 0, 5] = N
    bad[0, 0, 0, 6] = wrap + 3
    bad[0, 0, 1, 7] = -1
    bad[0, 0, 2, 9] = 2 ** 31 - 1
    bad[0, 0, 2, 10] = -2 ** 31
    o = mcs.sparse_attn(to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), to_dev(perm), to_dev(bad), C,
                        out_dtype=torch.float32)
    kz = np.concatenate([synth.to_f64(k), np.zeros((B, H, 1, D))], axis=2)
    vz = np.concatenate([synth.to_f64(v), np.zeros((B, H, 1, D))], axis=2)
    mapped = np.where((bad >= 0) & (bad < N), bad, N)
    ref = oracle.sparse_attention_bh(synth.to_f64(q), kz, vz, perm, mapped, C, 1 / math.sqrt(D))
    assert_output_close(o.cpu().numpy(), ref, "sparse O with out-of-range ids")


def test_anchor_identity_on_gpu(mcs):
    # with the anchor's own inputs, sparse + residual reproduces the dense output
    B, H, N, D, C, K = 1, 2, 640, 64, 64, 128
    q, k, v = _qkv(B, H, N, D, seed=31, scale=1.5)
    G = accounting.num_groups(N, C)
    dq, dk, dv = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    perm = to_dev(synth.random_perm(B, H, N, seed=32))
    idx = to_dev(synth.random_index_sets(B, H, G, K, N, seed=33))
    o_dense = mcs.dense_attn(dq, dk, dv)
    o_sp = mcs.sparse_attn(dq, dk, dv, perm, idx, C)
    res = mcs.residual_update(o_dense, o_sp)
    o_reuse = mcs.sparse_attn(dq, dk, dv, perm, idx, C, residual=res)
    diff = (o_reuse.float() - o_dense.float()).abs().max().item()
    assert diff <= 2e-2
