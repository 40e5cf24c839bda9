"""Shared helpers of the GPU parity tests (host-side conversions and criteria)."""
import numpy as np
import torch

# Output criterion: bf16 in, fp32 accumulate; max-abs 2e-2 and relative L2 1e-2.
OUT_MAX_ABS = 2e-2
OUT_REL_L2 = 1e-2
# Index criterion: members of the symmetric difference must lie within this
# absolute distance (in summed-probability units) of the K-th largest mass,
# and the retained mass must match to this relative tolerance.
TIE_ABS = 1e-6
RHO_REL = 1e-4


def dev():
    return torch.device("cuda:0")


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def to_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev())


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def assert_output_close(got: np.ndarray, ref: np.ndarray, what: str = "output"):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    err = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    assert err.max() <= OUT_MAX_ABS, f"{what}: max abs err {err.max():.3e} (rel L2 {rel:.3e})"
    assert rel <= OUT_REL_L2, f"{what}: rel L2 err {rel:.3e} (max abs {err.max():.3e})"


def assert_index_sets_match(got_idx: np.ndarray, ref_idx: np.ndarray, ref_mass: np.ndarray, K: int,
                            what: str = "kv_idx"):
    """got_idx/ref_idx [G, K], ref_mass [G, N] fp64 masses of the oracle."""
    n = ref_mass.shape[1]
    for g in range(ref_idx.shape[0]):
        a = got_idx[g]
        assert a.shape == (K,)
        assert (a >= 0).all() and (a < n).all(), f"{what}[{g}] out of range"
        assert (np.diff(a) > 0).all(), f"{what}[{g}] not strictly ascending"
        kth = np.sort(ref_mass[g])[::-1][K - 1]
        diff = np.setxor1d(a, ref_idx[g])
        if diff.size:
            worst = np.abs(ref_mass[g, diff] - kth).max()
            assert worst <= TIE_ABS, f"{what}[{g}]: {diff.size} ids differ, worst |M - M_K| = {worst:.3e}"
        rho_got = ref_mass[g, a].sum()
        rho_ref = ref_mass[g, ref_idx[g]].sum()
        assert abs(rho_got - rho_ref) <= RHO_REL * rho_ref, f"{what}[{g}]: retained mass {rho_got} vs {rho_ref}"


def within_group_variance(q: np.ndarray, perm: np.ndarray, C: int) -> float:
    """Property of a grouping: mean squared distance of each query to its group mean."""
    total = 0.0
    n = q.shape[0]
    for g0 in range(0, n, C):
        x = q[perm[g0:g0 + C]]
        total += float(((x - x.mean(axis=0)) ** 2).sum())
    return total / n


def assert_perm(perm: np.ndarray):
    n = perm.shape[-1]
    for row in perm.reshape(-1, n):
        assert np.array_equal(np.sort(row), np.arange(n)), "not a permutation"
