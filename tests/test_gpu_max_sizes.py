"""Parity at a sequence length well beyond the workloads' (N = 262144, one head).

Rows of 262144 mass values take the streaming top-K, the grouping tree is 12
levels deep, and one head's selection workspace is 4.3 GB; byte offsets and
element counts pass 2^31 in places.  The oracle checks sampled outputs it can
compute one by one: dense rows, the top-K of sampled groups (from the oracle's
own LSE and masses), and whole sparse groups given generator-made ids.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from token_sparse_attention_amd import accounting, synth
from tests.helpers import assert_index_sets_match, assert_output_close, assert_perm, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

N, D, C = 262144, 64, 64


@pytest.fixture(scope="module")
def mcs():
    from token_sparse_attention_amd import binding
    return binding


@pytest.fixture(scope="module")
def inputs():
    print(f"[max sizes] generating N={N}", flush=True)
    x = {t: synth.gaussian((1, 1, N, D), 900 + i, 1.5) for i, t in enumerate("qkv")}
    return {"x": x, "dev": {t: to_dev_bf16(x[t]) for t in "qkv"},
            "f64": {t: synth.to_f64(x[t])[0, 0] for t in "qkv"}}


def test_dense_rows(mcs, inputs):
    scale = 1 / math.sqrt(D)
    d = inputs["dev"]
    o32, lse = mcs.dense_attn(d["q"], d["k"], d["v"], scale, want_lse=True, out_dtype=torch.float32)
    rows = np.unique(np.r_[0, N - 1, np.random.default_rng(1).choice(N, 30, replace=False)])
    q, k, v = (inputs["f64"][t] for t in "qkv")
    ref_o, ref_lse = oracle.dense_attention(q[rows], k, v, scale)
    assert_output_close(o32[0, 0, rows].cpu().numpy(), ref_o, "dense N=262144")
    np.testing.assert_allclose(lse[0, 0, rows].cpu().numpy(), ref_lse, rtol=0, atol=2e-3)


@pytest.mark.parametrize("K", [1024, 65536])
def test_select_streaming_rows(mcs, inputs, K):
    scale = 1 / math.sqrt(D)
    d = inputs["dev"]
    G = accounting.num_groups(N, C)
    perm = synth.random_perm(1, 1, N, seed=K)
    _, lse = mcs.dense_attn(d["q"], d["k"], d["v"], scale, want_lse=True)
    ws = torch.empty(mcs.select_workspace_bytes(d["q"].shape, C, K, all_heads=False), dtype=torch.uint8,
                     device=lse.device)
    got = mcs.select(d["q"], d["k"], lse, to_dev(perm), C, K, scale, workspace=ws)[0, 0].cpu().numpy()
    assert got.shape == (G, K)
    q, k = inputs["f64"]["q"], inputs["f64"]["k"]
    for g in (0, G - 1):
        members = perm[0, 0, g * C:(g + 1) * C]
        _, lse_g = oracle.dense_attention(q[members], k, k, scale)     # only the LSE is used
        mass = oracle.probabilities(q[members], k, lse_g, scale).sum(axis=0)[None]
        ref = oracle.topk_indices(mass[0], K)[None]
        assert_index_sets_match(got[g:g + 1], ref, mass, K, f"N=262144 K={K} group {g}")


def test_sparse_groups(mcs, inputs):
    scale = 1 / math.sqrt(D)
    d = inputs["dev"]
    K = 4096
    G = accounting.num_groups(N, C)
    perm = synth.random_perm(1, 1, N, seed=7)
    idx = synth.stratified_index_sets(1, 1, G, K, N, seed=8)
    o32 = mcs.sparse_attn(d["q"], d["k"], d["v"], to_dev(perm), to_dev(idx), C, scale=scale,
                          out_dtype=torch.float32)[0, 0].cpu().numpy()
    q, k, v = (inputs["f64"][t] for t in "qkv")
    for g in (0, G // 2, G - 1):
        members = perm[0, 0, g * C:(g + 1) * C]
        ref = oracle.sparse_attention(q[members], k, v, np.arange(members.size), idx[0, 0, g:g + 1], C, scale)
        assert_output_close(o32[members], ref, f"sparse N=262144 group {g}")


def test_group_is_a_partition_into_groups_of_c(mcs, inputs):
    perm = mcs.group(inputs["dev"]["q"], C).cpu().numpy()
    assert_perm(perm)
