"""The anchor and reuse steps captured in a HIP graph replay exactly.

The library only enqueues kernels on the caller's stream: it allocates,
frees, copies, sets and synchronises nothing, so a whole layer-step can be
captured once and replayed (a serving loop's usual shape).  The test captures
an anchor step followed by a reuse step, replays the graph several times with
unrelated eager work and synchronisations between the replays, and checks
every replay bit for bit against the same calls made eagerly (every kernel is
deterministic).
"""
import math

import pytest
import torch

from token_sparse_attention_amd import synth
from tests.helpers import to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mcs():
    from token_sparse_attention_amd import binding
    return binding


@pytest.mark.parametrize("N,D,C,K", [(1000, 128, 128, 256), (777, 64, 64, 130)])
def test_anchor_and_reuse_steps_replay_from_a_graph(mcs, N, D, C, K):
    B, H = 1, 2
    scale = 1 / math.sqrt(D)
    q, k, v = (to_dev_bf16(synth.gaussian((B, H, N, D), N + s, 1.5)) for s in range(3))
    q2, k2, v2 = (to_dev_bf16(synth.gaussian((B, H, N, D), N + 10 + s, 1.5)) for s in range(3))

    ref = mcs.anchor_step(q, k, v, C, K, scale)
    ref_out = mcs.reuse_step(q2, k2, v2, ref["perm"], ref["kv_idx"], ref["residual"], C, scale)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()                     # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                  # warm-up outside the capture
        st = mcs.anchor_step(q, k, v, C, K, scale)
        mcs.reuse_step(q2, k2, v2, st["perm"], st["kv_idx"], st["residual"], C, scale)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = mcs.anchor_step(q, k, v, C, K, scale)
        out = mcs.reuse_step(q2, k2, v2, st["perm"], st["kv_idx"], st["residual"], C, scale)

    for rep in range(3):
        other = mcs.dense_attn(q2, k2, v2, scale)  # eager work between replays
        for t in (st["perm"], st["kv_idx"], st["residual"], st["out"], out):
            t.fill_(0)                             # stale results cannot pass
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st["perm"], ref["perm"]), rep
        assert torch.equal(st["kv_idx"], ref["kv_idx"]), rep
        assert torch.equal(st["lse"], ref["lse"]), rep
        assert torch.equal(st["out"], ref["out"]), rep
        assert torch.equal(st["residual"], ref["residual"]), rep
        assert torch.equal(out, ref_out), rep
        del other
