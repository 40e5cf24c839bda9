"""GPU checks of the per-layer anchor cache: offloaded entries come back
bit-exact through the prefetch slots, in any order and after being replaced,
and a multi-layer reuse step gives the same outputs with offloaded and with
resident entries."""
import math

import pytest
import torch

from token_sparse_attention_amd import accounting, synth
from token_sparse_attention_amd.cache import AnchorCache
from tests.helpers import to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def _entry(B, H, N, D, C, K, seed):
    G = accounting.num_groups(N, C)
    perm = to_dev(synth.random_perm(B, H, N, seed=seed))
    idx = to_dev(synth.random_index_sets(B, H, G, K, N, seed=seed + 1))
    res = to_dev_bf16(synth.gaussian((B, H, N, D), seed + 2))
    return perm, idx, res


@pytest.mark.parametrize("offload", [False, True])
def test_entries_round_trip(offload):
    L = 5
    cache = AnchorCache(L, offload=offload)
    ref = [_entry(1, 2, 700, 64, 64, 100, 10 * l) for l in range(L)]
    for l, e in enumerate(ref):
        cache.put(l, *e)
    # in order, twice around, then out of order
    order = list(range(L)) * 2 + [3, 1, 4, 4, 0, 2]
    for l in order:
        got = cache.get(l)
        for a, b in zip(got.tensors(), ref[l]):
            assert torch.equal(a, b), f"layer {l}"
    # a replaced entry is seen by the next get
    new = _entry(1, 2, 700, 64, 64, 100, 999)
    cache.put(2, *new)
    for l in [1, 2, 3, 2]:
        got = cache.get(l)
        want = new if l == 2 else ref[l]
        for a, b in zip(got.tensors(), want):
            assert torch.equal(a, b), f"layer {l} after replacement"


def test_reuse_step_offloaded_equals_resident():
    from token_sparse_attention_amd import binding
    L, B, H, N, D, C, K = 4, 1, 2, 1000, 128, 128, 256
    scale = 1 / math.sqrt(D)
    q = [to_dev_bf16(synth.gaussian((B, H, N, D), 100 + 3 * l)) for l in range(L)]
    k = [to_dev_bf16(synth.gaussian((B, H, N, D), 101 + 3 * l)) for l in range(L)]
    v = [to_dev_bf16(synth.gaussian((B, H, N, D), 102 + 3 * l)) for l in range(L)]
    entries = [_entry(B, H, N, D, C, K, 50 + 7 * l) for l in range(L)]
    outs = {}
    for offload in (False, True):
        cache = AnchorCache(L, offload=offload)
        for l, e in enumerate(entries):
            cache.put(l, *e)
        res = []
        for _ in range(2):                       # two reuse steps
            for l in range(L):
                e = cache.get(l)
                res.append(binding.sparse_attn(q[l], k[l], v[l], e.perm, e.kv_idx, C, residual=e.residual,
                                               scale=scale))
        torch.cuda.synchronize()
        outs[offload] = res
    for a, b in zip(outs[False], outs[True]):
        assert torch.equal(a, b)
