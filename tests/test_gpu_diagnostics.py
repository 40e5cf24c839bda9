"""GPU parity of the selection diagnostics and the block-sparse comparison.

mcs_sparse_attn_ex (per-group key counts, sparse LSE), mcs_select_blocks
(mean-pooled block selection), mcs_query_quality and mcs_row_sums, each
against the fp64 oracle on the same inputs.  Block ids are compared like
token ids: exactly, except where fp32 and fp64 scores order near-equal blocks
differently (every id in the symmetric difference within 1e-5 of the oracle's
K-th score).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import diagnostics as dg
from token_sparse_attention_amd import accounting, synth
from tests.helpers import assert_output_close, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

BLOCK_TIE = 1e-5


@pytest.fixture(scope="module")
def mcs():
    from token_sparse_attention_amd import binding
    return binding


def _qkv(B, H, N, D, seed, scale=1.0):
    return (synth.gaussian((B, H, N, D), seed, scale), synth.gaussian((B, H, N, D), seed + 1, scale),
            synth.gaussian((B, H, N, D), seed + 2))


@pytest.mark.parametrize("D,C", [(128, 128), (64, 64)])
def test_sparse_ex_counts_and_lse_match_oracle(mcs, D, C):
    B, H, N, K = 1, 2, 700, 150
    q, k, v = _qkv(B, H, N, D, seed=51, scale=1.5)
    G = accounting.num_groups(N, C)
    perm = synth.random_perm(B, H, N, seed=52)
    idx = synth.random_index_sets(B, H, G, K, N, seed=53)
    counts = np.random.default_rng(54).integers(1, K + 1, size=(B, H, G)).astype(np.int32)
    counts[0, 0, 0], counts[0, 1, -1] = 1, K                       # both ends of the range
    scale = 1 / math.sqrt(D)
    o, lse = mcs.sparse_attn_ex(to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), to_dev(perm), to_dev(idx), C,
                                kv_count=to_dev(counts), scale=scale, want_lse=True, out_dtype=torch.float32)
    qf, kf, vf = synth.to_f64(q), synth.to_f64(k), synth.to_f64(v)
    for h in range(H):
        sel = [idx[0, h, g, :counts[0, h, g]] for g in range(G)]
        ref_o = oracle.sparse_attention(qf[0, h], kf[0, h], vf[0, h], perm[0, h], sel, C, scale)
        ref_lse = oracle.sparse_lse(qf[0, h], kf[0, h], perm[0, h], sel, C, scale)
        assert_output_close(o[0, h].cpu().numpy(), ref_o, f"head {h} output")
        np.testing.assert_allclose(lse[0, h].cpu().numpy(), ref_lse, rtol=0, atol=2e-3)
    # without counts and lse the extended call is mcs_sparse_attn bit for bit
    a = mcs.sparse_attn_ex(to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), to_dev(perm), to_dev(idx), C, scale=scale)
    b = mcs.sparse_attn(to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), to_dev(perm), to_dev(idx), C, scale=scale)
    assert torch.equal(a, b)


def test_sparse_ex_rejects_residual_with_lse(mcs):
    B, H, N, D, C, K = 1, 1, 128, 64, 64, 64
    q, k, v = _qkv(B, H, N, D, seed=55)
    perm = to_dev(synth.random_perm(B, H, N, seed=56))
    idx = to_dev(synth.random_index_sets(B, H, 2, K, N, seed=57))
    with pytest.raises(mcs.McsError):
        mcs.sparse_attn_ex(to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), perm, idx, C,
                           residual=to_dev_bf16(q), want_lse=True)


def _check_blocks(got_idx, got_count, q, k, perm, C, K, scale, what):
    """GPU block selection of one head against the oracle's mean-pooled selector."""
    N = k.shape[0]
    kbar = dg.block_means(k)
    nblk = K // dg.KV_BLOCK
    tail = N - (kbar.shape[0] - 1) * dg.KV_BLOCK
    for g, rows in enumerate(oracle.groups_from_perm(perm, C)):
        ids = got_idx[g]
        blocks = ids[::dg.KV_BLOCK] // dg.KV_BLOCK
        assert (np.diff(blocks) > 0).all(), f"{what} group {g}: blocks not ascending"
        expect_ids = np.concatenate([b * dg.KV_BLOCK + np.arange(dg.KV_BLOCK) for b in blocks])
        valid = expect_ids < N
        assert got_count[g] == valid.sum(), f"{what} group {g}: count {got_count[g]} != {valid.sum()}"
        np.testing.assert_array_equal(ids[:got_count[g]], expect_ids[valid])
        assert got_count[g] == K - (dg.KV_BLOCK - tail if blocks[-1] == kbar.shape[0] - 1 else 0)
        score = dg.mean_pooled_scores(q, kbar, rows, scale)
        ref = dg.mean_pooled_blocks(q, kbar, rows, K, scale)
        diff = np.setxor1d(blocks, ref)
        if diff.size:
            kth = np.sort(score)[::-1][nblk - 1]
            worst = np.abs(score[diff] - kth).max()
            assert worst <= BLOCK_TIE, f"{what} group {g}: {diff.size} blocks differ, worst {worst:.2e}"


@pytest.mark.parametrize("name,N,heads,K", [("tiny", 1024, 2, 256), ("small", 5000, 2, 1024),
                                            ("asset3d", 4160, 2, 640)])
def test_select_blocks_matches_oracle(mcs, name, N, heads, K):
    w = synth.WORKLOADS[name]
    x = synth.generate(name, heads=[(0, h) for h in range(heads)])
    q, k = (np.ascontiguousarray(x[t][:, :, :N]) for t in "qk")
    scale = 1 / math.sqrt(w.D)
    qf, kf = synth.to_f64(q), synth.to_f64(k)
    perm = np.stack([oracle.pddp(qf[0, h], w.C) for h in range(heads)])[None].astype(np.int32)
    idx, count = mcs.select_blocks(to_dev_bf16(q), to_dev_bf16(k), to_dev(perm), w.C, K, scale)
    idx, count = idx.cpu().numpy(), count.cpu().numpy()
    for h in range(heads):
        _check_blocks(idx[0, h], count[0, h], qf[0, h], kf[0, h], perm[0, h], w.C, K, scale, f"{name} head {h}")


def test_block_sparse_output_matches_oracle(mcs):
    # the block-sparse run: the GPU's own block selection (with a short last
    # block) through the sparse kernel, against the oracle on the same keys
    name, N, K = "small", 3000, 512
    w = synth.WORKLOADS[name]
    x = synth.generate(name, heads=[(0, 0)])
    q, k, v = (np.ascontiguousarray(x[t][:, :, :N]) for t in "qkv")
    scale = 1 / math.sqrt(w.D)
    perm = np.arange(N, dtype=np.int32)[None, None]
    dq, dk, dv = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    idx, count = mcs.select_blocks(dq, dk, to_dev(perm), w.C, K, scale)
    o = mcs.sparse_attn_ex(dq, dk, dv, to_dev(perm), idx, w.C, kv_count=count, scale=scale, out_dtype=torch.float32)
    idx, count = idx.cpu().numpy()[0, 0], count.cpu().numpy()[0, 0]
    assert (count < K).any(), "the short last block should be picked by some group"
    sel = [idx[g, :count[g]] for g in range(idx.shape[0])]
    ref = oracle.sparse_attention(*(synth.to_f64(t)[0, 0] for t in (q, k, v)), perm[0, 0], sel, w.C, scale)
    assert_output_close(o[0, 0].cpu().numpy(), ref, "block-sparse output")


def test_query_quality_and_row_sums(mcs):
    # recall from the two LSEs against the oracle's kept mass; the L1 sums
    # against numpy on the very outputs the kernel read; fp64 row sums
    B, H, N, D, C, K = 1, 2, 900, 128, 128, 256
    q, k, v = _qkv(B, H, N, D, seed=61, scale=1.5)
    G = accounting.num_groups(N, C)
    perm = synth.random_perm(B, H, N, seed=62)
    idx = synth.random_index_sets(B, H, G, K, N, seed=63)
    dq, dk, dv = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    od, lse_d = mcs.dense_attn(dq, dk, dv, want_lse=True, out_dtype=torch.float32)
    osp, lse_s = mcs.sparse_attn_ex(dq, dk, dv, to_dev(perm), to_dev(idx), C, want_lse=True,
                                    out_dtype=torch.float32)
    recall, l1, l1_ref = mcs.query_quality(lse_d, lse_s, od, osp)
    qf, kf = synth.to_f64(q), synth.to_f64(k)
    for h in range(H):
        _, lse = oracle.dense_attention(qf[0, h], kf[0, h], kf[0, h], 1 / math.sqrt(D))
        kept = oracle.kept_mass(qf[0, h], kf[0, h], lse, perm[0, h], idx[0, h], C, 1 / math.sqrt(D))
        np.testing.assert_allclose(recall[0, h].cpu().numpy(), kept, rtol=0, atol=1e-4)
    a, b = od.cpu().numpy().astype(np.float64), osp.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(l1.cpu().numpy(), np.abs(b - a).sum(axis=-1), rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(l1_ref.cpu().numpy(), np.abs(a).sum(axis=-1), rtol=1e-5, atol=1e-6)
    sums = mcs.row_sums(l1.view(B * H, N)).cpu().numpy()
    np.testing.assert_allclose(sums, l1.view(B * H, N).cpu().numpy().astype(np.float64).sum(axis=1), rtol=1e-12)
    x = torch.from_numpy(np.random.default_rng(64).standard_normal((3, 100003)).astype(np.float32)).cuda()
    np.testing.assert_allclose(mcs.row_sums(x).cpu().numpy(), x.cpu().numpy().astype(np.float64).sum(axis=1),
                               rtol=1e-12)


def test_kmeans_planted_clusters_exact(mcs):
    # well-separated clusters of unequal sizes, centres started on one member
    # each: labels, sizes and centres follow the oracle exactly (up to fp32)
    rng = np.random.default_rng(71)
    k, D = 12, 64
    sizes = rng.integers(5, 90, size=k)
    label = np.repeat(np.arange(k), sizes)
    centres = 30.0 * rng.standard_normal((k, D))
    x = synth.to_bf16_bits((centres[label] + 0.2 * rng.standard_normal((label.size, D))).astype(np.float32))
    xf = synth.to_f64(x)
    init = xf[np.cumsum(sizes) - 1].astype(np.float32)          # the last member of every cluster
    ref_lab, ref_c, ref_in = dg.kmeans(xf, init.astype(np.float64), 4)
    lab, c, inertia, sz = mcs.kmeans(to_dev_bf16(x), torch.from_numpy(init).cuda(), 4)
    np.testing.assert_array_equal(lab.cpu().numpy(), ref_lab)
    np.testing.assert_array_equal(sz.cpu().numpy(), np.bincount(ref_lab, minlength=k))
    np.testing.assert_allclose(c.cpu().numpy(), ref_c, rtol=0, atol=1e-4)
    np.testing.assert_allclose(inertia.cpu().numpy(), ref_in, rtol=1e-5)


@pytest.mark.parametrize("name,N,clusters", [("small", 4096, 32), ("asset3d", 3000, 47)])
def test_kmeans_workload_head_matches_oracle(mcs, name, N, clusters):
    w = synth.WORKLOADS[name]
    x = np.ascontiguousarray(synth.generate(name, heads=[(0, 0)])["q"][0, 0, :N])
    xf = synth.to_f64(x)
    rng = np.random.default_rng(72)
    init = xf[rng.choice(N, clusters, replace=False)]
    rounds = 10
    ref_lab, ref_c, ref_in = dg.kmeans(xf, init, rounds)
    lab, c, inertia, sz = mcs.kmeans(to_dev_bf16(x), torch.from_numpy(init.astype(np.float32)).cuda(), rounds)
    lab, sz = lab.cpu().numpy(), sz.cpu().numpy()
    # fp32 distances can settle a near-tie the other way and move a centre by
    # a little: the inertia stays within 1e-4 and almost every label agrees
    np.testing.assert_allclose(inertia.cpu().numpy(), ref_in, rtol=1e-4)
    assert (lab == ref_lab).mean() >= 0.995, (lab != ref_lab).sum()
    np.testing.assert_array_equal(sz, np.bincount(lab, minlength=clusters))
    f_gpu = dg.alignment_inflation(sz[sz > 0], w.C)
    f_ref = dg.alignment_inflation(np.bincount(ref_lab)[np.bincount(ref_lab) > 0], w.C)
    assert abs(f_gpu - f_ref) <= 0.01 * f_ref, (f_gpu, f_ref)


def test_kmeans_empty_cluster_keeps_its_centre(mcs):
    # two identical initial centres: in the first round the second wins no
    # point (ties go to the smaller id) and stays where it started; later
    # rounds follow the oracle (the first centre moves away, so the second
    # then wins the point it sits on)
    rng = np.random.default_rng(73)
    x = synth.to_bf16_bits(rng.standard_normal((300, 128)).astype(np.float32))
    xf = synth.to_f64(x)
    init = np.stack([xf[0], xf[0], xf[1]]).astype(np.float32)
    lab, c, _, sz = mcs.kmeans(to_dev_bf16(x), torch.from_numpy(init).cuda(), 1)
    assert sz.cpu().numpy()[1] == 0 and (lab.cpu().numpy() != 1).all()
    np.testing.assert_array_equal(c.cpu().numpy()[1], init[1])
    ref_lab, ref_c, _ = dg.kmeans(xf, init.astype(np.float64), 3)
    lab, c, _, sz = mcs.kmeans(to_dev_bf16(x), torch.from_numpy(init).cuda(), 3)
    np.testing.assert_array_equal(lab.cpu().numpy(), ref_lab)
    np.testing.assert_allclose(c.cpu().numpy(), ref_c, rtol=0, atol=1e-4)
