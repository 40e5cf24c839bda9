"""GPU parity of mcs_topk (bit-exact) and mcs_select (the index criterion).

mcs_topk is compared decision-for-decision with the oracle's top-K applied to
the same float32 score rows (both sides decide in float32), including rows
with many ties.  mcs_select is compared with the oracle's fp64 selection on
the same groups: the ids may differ only among masses within 1e-6 of the K-th
largest, and the retained mass must agree to 1e-4 relative.  mcs_select (mass
and top-K in one kernel where the row's counts fit in LDS) and
mcs_select_two_pass (mass kernel, then top-K kernel) compute the same fp32
masses and apply the same rule, so their ids must be identical.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from token_sparse_attention_amd import accounting, synth
from tests.helpers import assert_index_sets_match, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mcs():
    from token_sparse_attention_amd import binding
    return binding


@pytest.mark.parametrize("rows,n,K", [(3, 1, 1), (5, 1000, 1), (5, 1000, 1000), (7, 1000, 333),
                                      (4, 5000, 1024), (2, 75600, 15104), (3, 4097, 4096)])
@pytest.mark.parametrize("ties", [False, True])
def test_topk_bit_exact(mcs, rows, n, K, ties):
    scores = synth.mass_rows(rows, n, seed=n + K, ties=ties)
    got = mcs.topk(to_dev(scores), K).cpu().numpy()
    for r in range(rows):
        np.testing.assert_array_equal(got[r], oracle.topk_indices(scores[r], K))


@pytest.mark.parametrize("rows,n,K", [(2, 81920, 40000), (2, 81921, 81921), (2, 51201, 1), (2, 51200, 51200),
                                      (2, 118800, 29696)])
def test_topk_row_sizes(mcs, rows, n, K):
    """Rows at the edges of the on-chip kernel (all slots in registers, the
    first LDS slot partly filled, the largest on-chip row) and past it (the
    streaming kernel), with ties and zeros."""
    scores = synth.mass_rows(rows, n, seed=7 * n + K, ties=True)
    got = mcs.topk(to_dev(scores), K).cpu().numpy()
    for r in range(rows):
        np.testing.assert_array_equal(got[r], oracle.topk_indices(scores[r], K))


@pytest.mark.parametrize("n", [300, 60000, 81920])
def test_topk_zero_rows_take_first_ids(mcs, n):
    """All-zero rows: the K chosen ids are the first K (equal values go to the
    smaller id), whatever the slots past the row end hold."""
    scores = np.zeros((2, n), dtype=np.float32)
    K = n // 2 + 1
    got = mcs.topk(to_dev(scores), K).cpu().numpy()
    for r in range(2):
        np.testing.assert_array_equal(got[r], np.arange(K))


def test_topk_all_equal_and_zero(mcs):
    scores = np.zeros((2, 300), dtype=np.float32)
    scores[1] = 0.25
    got = mcs.topk(to_dev(scores), 100).cpu().numpy()
    np.testing.assert_array_equal(got[0], np.arange(100))
    np.testing.assert_array_equal(got[1], np.arange(100))


def _select_case(mcs, B, H, N, D, C, K, seed, perm_kind="random"):
    q = synth.gaussian((B, H, N, D), seed, 1.5)
    k = synth.gaussian((B, H, N, D), seed + 1, 1.5)
    scale = 1 / math.sqrt(D)
    qf, kf = synth.to_f64(q), synth.to_f64(k)
    if perm_kind == "random":
        perm = synth.random_perm(B, H, N, seed=seed)
    else:
        perm = oracle.pddp_bh(qf, C).astype(np.int32)
    _, lse = oracle.dense_attention_bh(qf, kf, qf, scale)
    ref_idx, ref_mass = oracle.select_bh(qf, kf, lse, perm, C, K, scale)
    args = (to_dev_bf16(q), to_dev_bf16(k), to_dev(lse.astype(np.float32)), to_dev(perm), C, K, scale)
    got = mcs.select(*args)
    assert torch.equal(got, mcs.select_two_pass(*args))
    got = got.cpu().numpy()
    G = accounting.num_groups(N, C)
    assert got.shape == (B, H, G, K)
    for b in range(B):
        for h in range(H):
            assert_index_sets_match(got[b, h], ref_idx[b, h], ref_mass[b, h], K)


@pytest.mark.parametrize("B,H,N,D,C,K", [(1, 2, 1000, 128, 128, 200), (1, 1, 700, 64, 64, 65),
                                         (2, 1, 333, 64, 128, 1), (1, 1, 256, 128, 64, 256),
                                         (1, 1, 50, 64, 64, 7), (1, 2, 100, 128, 128, 100)])
def test_select_matches_oracle(mcs, B, H, N, D, C, K):
    _select_case(mcs, B, H, N, D, C, K, seed=N + K)


def test_select_on_oracle_groups(mcs):
    _select_case(mcs, 1, 1, 1024, 64, 64, 256, seed=5, perm_kind="pddp")


def test_select_small_workspace_chunks_heads(mcs):
    B, H, N, D, C, K = 1, 3, 300, 64, 64, 50
    q = synth.gaussian((B, H, N, D), 40, 1.5)
    k = synth.gaussian((B, H, N, D), 41, 1.5)
    perm = synth.random_perm(B, H, N, seed=42)
    qf, kf = synth.to_f64(q), synth.to_f64(k)
    _, lse = oracle.dense_attention_bh(qf, kf, qf, 0.125)
    dq, dk, dl, dp = to_dev_bf16(q), to_dev_bf16(k), to_dev(lse.astype(np.float32)), to_dev(perm)
    one_head = mcs.select_workspace_bytes(q.shape, C, K, all_heads=False)
    ws = torch.empty(one_head + 100, dtype=torch.uint8, device=dq.device)
    a = mcs.select(dq, dk, dl, dp, C, K, 0.125, workspace=ws)
    b = mcs.select(dq, dk, dl, dp, C, K, 0.125)
    assert torch.equal(a, b)


def test_select_with_gpu_lse(mcs):
    # pass 1 on the GPU feeds pass 2 on the GPU; the oracle runs both passes itself
    B, H, N, D, C, K = 1, 2, 777, 128, 128, 150
    q = synth.gaussian((B, H, N, D), 50, 1.5)
    k = synth.gaussian((B, H, N, D), 51, 1.5)
    v = synth.gaussian((B, H, N, D), 52)
    perm = synth.random_perm(B, H, N, seed=53)
    scale = 1 / math.sqrt(D)
    dq, dk, dv = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    _, lse = mcs.dense_attn(dq, dk, dv, scale, want_lse=True)
    got = mcs.select(dq, dk, lse, to_dev(perm), C, K, scale).cpu().numpy()
    qf, kf = synth.to_f64(q), synth.to_f64(k)
    _, ref_lse = oracle.dense_attention_bh(qf, kf, synth.to_f64(v), scale)
    ref_idx, ref_mass = oracle.select_bh(qf, kf, ref_lse, perm, C, K, scale)
    for h in range(H):
        assert_index_sets_match(got[0, h], ref_idx[0, h], ref_mass[0, h], K)


@pytest.mark.parametrize("N,D,C,K,dup", [(4097, 128, 128, 800, False), (3000, 64, 64, 1500, True),
                                         (3001, 128, 64, 2999, True), (75600, 128, 128, 15104, False),
                                         (131072, 64, 128, 26215, False), (131073, 64, 128, 100, False),
                                         (131071, 64, 128, 5000, False), (65536, 128, 64, 65536, False),
                                         (262144, 128, 128, 4096, False), (262145, 128, 128, 4096, False)])
def test_fused_select_equals_two_pass(mcs, N, D, C, K, dup):
    """One head per case, LSE from the GPU's own dense pass: a large-workload
    head, the largest rows the fused kernel holds for D = 64 (16-byte and
    4-byte reads; the latter leaves no LDS for the gathered third-digit keys,
    so the counting read runs) and for D = 128, one past each (mcs_select takes
    the two-kernel route), K = N, and duplicated keys (equal masses in pairs,
    so the tie rule decides at the K-th key).  Both kernels start each key
    sweep at a tile taken from the clock (rows of more than 32 tiles), so the
    calls sweep in different orders: equal ids also show that the masses do
    not depend on where a sweep starts."""
    q = synth.gaussian((1, 1, N, D), 60 + N, 1.5)
    k = synth.gaussian((1, 1, N, D), 61 + N, 1.5)
    if dup:
        k[:, :, 1::2] = k[:, :, 0:N - 1:2]
    scale = 1 / math.sqrt(D)
    dq, dk = to_dev_bf16(q), to_dev_bf16(k)
    _, lse = mcs.dense_attn(dq, dk, dk, scale, want_lse=True)
    perm = to_dev(synth.random_perm(1, 1, N, seed=N))
    print(f"[fused select] N={N} D={D} C={C} K={K} dup={dup}", flush=True)
    a = mcs.select(dq, dk, lse, perm, C, K, scale)
    b = mcs.select_two_pass(dq, dk, lse, perm, C, K, scale)
    assert torch.equal(a, b)
    ids = a[0, 0]
    assert bool((ids[:, 1:] > ids[:, :-1]).all()) and int(ids.min()) >= 0 and int(ids.max()) < N


@pytest.mark.parametrize("N,D,C,K", [(5000, 128, 128, 1234), (3001, 64, 64, 3000)])
def test_fused_select_all_masses_equal(mcs, N, D, C, K):
    """Identical keys: every key of a group has the same mass, so the K ids are
    the first K.  Every key shares the threshold's leading bits, more than the
    fused kernel gathers, so its counting read runs."""
    q = synth.gaussian((1, 1, N, D), 70, 1.5)
    k = np.repeat(synth.gaussian((1, 1, 1, D), 71, 1.5), N, axis=2)
    scale = 1 / math.sqrt(D)
    dq, dk = to_dev_bf16(q), to_dev_bf16(k)
    _, lse = mcs.dense_attn(dq, dk, dk, scale, want_lse=True)
    perm = to_dev(synth.random_perm(1, 1, N, seed=N))
    print(f"[fused select, equal masses] N={N} D={D} C={C} K={K}", flush=True)
    a = mcs.select(dq, dk, lse, perm, C, K, scale)
    assert torch.equal(a, mcs.select_two_pass(dq, dk, lse, perm, C, K, scale))
    G = accounting.num_groups(N, C)
    np.testing.assert_array_equal(a[0, 0].cpu().numpy(), np.broadcast_to(np.arange(K), (G, K)))
