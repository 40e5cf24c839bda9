"""mcs_group_noalloc (the allocation-free grouping call) against mcs_group.

Both run the same kernels on the same head data, so the permutations must be
identical.  Two calls in a row, the second with a smaller input, so the
second finds the first one's contents in the shared scratch.  The first call
has more heads than the scratch holds at once (two chunks).
"""
import ctypes

import numpy as np
import pytest
import torch

from token_sparse_attention_amd import synth
from tests.helpers import assert_perm, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mcs():
    from token_sparse_attention_amd import binding
    return binding


def _video_heads(H, N):
    x = synth.generate("large", heads=[(0, h) for h in range(H)])
    return np.ascontiguousarray(x["q"][:, :, :N])


def test_noalloc_matches_group_on_two_calls(mcs):
    cases = [("large", 16, 75600, 128), ("asset3d", 3, 5000, 64)]
    for name, H, N, C in cases:
        print(f"[noalloc] {name} H={H} N={N} C={C}", flush=True)
        if name == "large":
            q = to_dev_bf16(_video_heads(H, N))
        else:
            x = synth.generate(name, heads=[(0, h) for h in range(H)])
            q = to_dev_bf16(np.ascontiguousarray(x["q"][:, :, :N]))
        ref = mcs.group(q, C)
        got = mcs.group_noalloc(q, C)
        torch.cuda.synchronize()
        assert_perm(got.cpu().numpy())
        assert torch.equal(got, ref), f"{name}: noalloc grouping differs from mcs_group"


def test_noalloc_rejects_a_head_larger_than_the_scratch(mcs):
    # N = 8388607, D = 128: one head's workspace exceeds 64 MiB; the call is
    # rejected on the host before any pointer is touched
    d = mcs.Dims(1, 1, 8388607, 128)
    st = mcs._lib.mcs_group_noalloc(ctypes.c_void_p(0x10000), ctypes.c_void_p(0x20000), d, 128, 0, None)
    assert st == 8, mcs._lib.mcs_last_error()      # MCS_E_WORKSPACE
    assert b"scratch" in mcs._lib.mcs_last_error()
