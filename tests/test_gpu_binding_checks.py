"""The Python binding refuses tensors whose shape, dtype or device does not
match what the kernels address from the dimensions alone, before anything is
enqueued (the C ABI takes bare pointers and cannot check extents)."""
import pytest
import torch

pytestmark = pytest.mark.gpu

B, H, N, D, C, K = 1, 2, 300, 64, 64, 40
G = -(-N // C)


@pytest.fixture(scope="module")
def mcs():
    from token_sparse_attention_amd import binding
    return binding


@pytest.fixture(scope="module")
def t():
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(0)
    q, k, v = (torch.randn((B, H, N, D), generator=g).to(torch.bfloat16).to(dev) for _ in range(3))
    perm = torch.arange(N, dtype=torch.int32).repeat(B, H, 1).contiguous().to(dev)
    lse = torch.zeros((B, H, N), dtype=torch.float32, device=dev)
    idx = torch.arange(K, dtype=torch.int32).repeat(B, H, G, 1).contiguous().to(dev)
    return dict(q=q, k=k, v=v, perm=perm, lse=lse, idx=idx, dev=dev)


def test_dense_checks(mcs, t):
    q, k, v = t["q"], t["k"], t["v"]
    with pytest.raises(ValueError, match="lse"):
        mcs.dense_attn(q, k, v, want_lse=True, lse=torch.empty((B, H, N - 1), dtype=torch.float32, device=t["dev"]))
    with pytest.raises(ValueError, match="out"):
        mcs.dense_attn(q, k, v, out=torch.empty((B, H, N, D - 1), dtype=torch.bfloat16, device=t["dev"]))
    with pytest.raises(ValueError, match="k"):
        mcs.dense_attn(q, k[:, :, :N - 1].contiguous(), v)
    with pytest.raises(ValueError, match="contiguous"):
        mcs.dense_attn(q, k.transpose(2, 3).contiguous().transpose(2, 3), v)


def test_sparse_checks(mcs, t):
    q, k, v, perm, idx = t["q"], t["k"], t["v"], t["perm"], t["idx"]
    with pytest.raises(ValueError, match="perm"):
        mcs.sparse_attn(q, k, v, perm[:, :, :N - 1].contiguous(), idx, C)
    with pytest.raises(ValueError, match="residual"):
        mcs.sparse_attn(q, k, v, perm, idx, C, residual=torch.zeros((B, H, N - 1, D), dtype=torch.bfloat16,
                                                                    device=t["dev"]))
    with pytest.raises(ValueError, match="kv_idx"):
        mcs.sparse_attn(q, k, v, perm, idx[:, :, :G - 1].contiguous(), C)
    with pytest.raises(TypeError, match="perm"):
        mcs.sparse_attn(q, k, v, perm.long(), idx, C)


def test_select_checks(mcs, t):
    q, k, perm, lse = t["q"], t["k"], t["perm"], t["lse"]
    with pytest.raises(ValueError, match="lse"):
        mcs.select(q, k, lse[:, :1].contiguous(), perm, C, K)
    with pytest.raises(ValueError, match="out"):
        mcs.select(q, k, lse, perm, C, K, out=torch.empty((B, H, G, K - 1), dtype=torch.int32, device=t["dev"]))
    with pytest.raises(TypeError, match="workspace"):
        mcs.select(q, k, lse, perm, C, K, workspace=torch.empty(1 << 20, dtype=torch.float32, device=t["dev"]))
    with pytest.raises(ValueError, match="perm"):
        mcs.select_two_pass(q, k, lse, perm[:, :, :N - 1].contiguous(), C, K)


def test_group_topk_residual_checks(mcs, t):
    q = t["q"]
    with pytest.raises(ValueError, match="out"):
        mcs.group(q, C, out=torch.empty((B, H, N + 1), dtype=torch.int32, device=t["dev"]))
    with pytest.raises(ValueError, match="out"):
        mcs.topk(torch.zeros((3, 100), dtype=torch.float32, device=t["dev"]), 10,
                 out=torch.empty((3, 9), dtype=torch.int32, device=t["dev"]))
    with pytest.raises(ValueError, match="o_sparse"):
        mcs.residual_update(q, q[:, :, :N - 1].contiguous())
