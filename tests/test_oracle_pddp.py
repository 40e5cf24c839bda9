"""Pins of the oracle's median-split PDDP grouping.

Exact group sizes for many (N, C) including non-power-of-two group counts;
closed forms (collinear queries split into consecutive chunks of their sorted
coordinate; well-separated clusters of exactly C points are recovered);
agreement of the principal direction with an SVD and with long power
iteration; refinement and variance monotonicity; the query-id tie rule.
"""
import numpy as np
import pytest

import oracle


def _rand(shape, seed, scale=1.0):
    return scale * np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("N,C", [(1, 4), (3, 4), (4, 4), (5, 4), (64, 8), (100, 8), (129, 8),
                                 (591 * 4 - 3, 4), (768 * 2, 2)])
def test_group_sizes_and_permutation(N, C):
    q = _rand((N, 3), N)
    perm = oracle.pddp(q, C)
    assert sorted(perm.tolist()) == list(range(N))
    sizes = [len(g) for g in oracle.groups_from_perm(perm, C)]
    G = -(-N // C)
    assert sizes[:-1] == [C] * (G - 1)
    assert sizes[-1] == N - (G - 1) * C


def test_principal_direction_matches_svd():
    x = _rand((300, 6), 1) * np.array([5.0, 2.0, 1.0, 0.5, 0.3, 0.1]) + 3.0
    mu, v = oracle.principal_direction(x)
    _, _, vt = np.linalg.svd(x - x.mean(axis=0), full_matrices=False)
    assert abs(abs(v @ vt[0]) - 1.0) < 1e-12
    np.testing.assert_allclose(mu, x.mean(axis=0), atol=1e-14)
    i = int(np.argmax(np.abs(v)))
    assert v[i] > 0


def test_power_iteration_agrees_with_eigh_when_gap_is_large():
    rng = np.random.default_rng(2)
    basis, _ = np.linalg.qr(rng.standard_normal((16, 16)))
    x = (rng.standard_normal((2000, 16)) * np.r_[3.0, np.linspace(2.0, 0.5, 15)]) @ basis.T
    lam = np.linalg.eigvalsh(np.cov(x.T, bias=True))
    assert lam[-1] / lam[-2] > 1.5
    _, v_e = oracle.principal_direction(x, mode="eigh")
    _, v_p = oracle.principal_direction(x, mode="power", power_iters=200)
    assert abs(v_e @ v_p) > 1 - 1e-8
    np.testing.assert_allclose(v_e, v_p, atol=1e-4)    # same canonical sign


@pytest.mark.parametrize("N,C", [(64, 8), (100, 8), (37, 4)])
def test_collinear_queries_give_sorted_chunks(N, C):
    rng = np.random.default_rng(N)
    u = rng.standard_normal(5)
    u[np.argmax(np.abs(u))] = abs(u).max() + 1.0       # canonical sign is +u
    t = rng.permutation(N).astype(float)
    q = t[:, None] * u[None, :] + rng.standard_normal(5)
    perm = oracle.pddp(q, C)
    order = np.argsort(t)
    for g, members in enumerate(oracle.groups_from_perm(perm, C)):
        assert set(members.tolist()) == set(order[g * C:(g + 1) * C].tolist())


def test_separated_clusters_are_recovered():
    rng = np.random.default_rng(7)
    C, L, D = 8, 3, 6
    centres = 100.0 * rng.standard_normal((2 ** L, D))
    label = rng.permutation(np.repeat(np.arange(2 ** L), C))
    q = centres[label] + rng.standard_normal((2 ** L * C, D))
    perm = oracle.pddp(q, C)
    for members in oracle.groups_from_perm(perm, C):
        assert len(set(label[members].tolist())) == 1


def test_refinement_and_variance_monotone():
    q = _rand((256, 5), 9) * np.array([4.0, 3.0, 2.0, 1.0, 0.5])
    total = oracle.within_group_variance(q, np.arange(256), 256)
    prev_w, prev_groups = total, None
    for C in (128, 64, 32, 16, 8):
        perm = oracle.pddp(q, C)
        w = oracle.within_group_variance(q, perm, C)
        assert w <= prev_w + 1e-12
        if prev_groups is not None:
            # N = 2^L * C: the C-grouping splits each 2C-group in two
            for members in oracle.groups_from_perm(perm, C):
                assert any(set(members.tolist()) <= s for s in prev_groups)
        prev_w = w
        prev_groups = [set(m.tolist()) for m in oracle.groups_from_perm(perm, C)]
    assert prev_w < total


def _known_covariance_points(n, lam, rot):
    """n points with mean 0 and covariance exactly rot @ diag(lam) @ rot.T:
    orthonormal columns scaled by sqrt(n * lam), rotated."""
    z, _ = np.linalg.qr(np.random.default_rng(5).standard_normal((n, len(lam))))
    z -= z.mean(axis=0)                        # still orthogonal columns after re-orthonormalising
    z, _ = np.linalg.qr(z)
    return (z * np.sqrt(n * np.asarray(lam))) @ rot.T, z


def test_default_direction_is_the_exact_eigenvector():
    # Covariance rot diag(1, 0.97, 0.3) rot^T by construction: the principal
    # direction is rot[:, 0] (closed form), so the root splits the points by
    # their first coordinate z[:, 0] in the eigenbasis.  Two leading variances
    # 3% apart: 32 power steps from the largest-diagonal column stay far from
    # rot[:, 0] and split differently, so this pins the default to the exact
    # eigenvector and not to any fixed number of power steps.
    c, s_ = np.cos(0.7), np.sin(0.7)
    rot = np.array([[c, -s_, 0.0], [s_, c, 0.0], [0.0, 0.0, 1.0]]) @ \
        np.array([[1.0, 0.0, 0.0], [0.0, np.cos(0.4), -np.sin(0.4)], [0.0, np.sin(0.4), np.cos(0.4)]])
    q, z = _known_covariance_points(256, [1.0, 0.97, 0.3], rot)
    np.testing.assert_allclose(np.cov(q.T, bias=True), rot @ np.diag([1.0, 0.97, 0.3]) @ rot.T, atol=1e-12)
    u = rot[:, 0] if rot[np.argmax(np.abs(rot[:, 0])), 0] > 0 else -rot[:, 0]
    _, v = oracle.principal_direction(q)
    np.testing.assert_allclose(v, u, atol=1e-10)
    proj = q @ u
    left = set(np.argsort(proj, kind="stable")[:128].tolist())
    perm = oracle.pddp(q, 32)
    assert set(perm[:128].tolist()) == left
    # a fixed number of power steps is a different (unconverged) reading here
    perm_p = oracle.pddp(q, 32, mode="power", power_iters=32)
    assert set(perm_p[:128].tolist()) != left
    for mode in ("eigh", "power"):
        assert sorted(oracle.pddp(q, 16, mode=mode).tolist()) == list(range(256))


def test_power_mode_with_many_steps_matches_eigh_grouping():
    q = _rand((512, 5), 22) * np.array([5.0, 3.0, 2.0, 1.0, 0.5])
    a = oracle.pddp(q, 32, mode="eigh")
    b = oracle.pddp(q, 32, mode="power", power_iters=500)
    ga = {frozenset(g.tolist()) for g in oracle.groups_from_perm(a, 32)}
    gb = {frozenset(g.tolist()) for g in oracle.groups_from_perm(b, 32)}
    assert ga == gb


def test_identical_queries_split_by_query_id():
    q = np.ones((40, 4))
    perm = oracle.pddp(q, 8)
    np.testing.assert_array_equal(perm, np.arange(40))


def test_within_group_variance_closed_form():
    q = np.array([[0.0], [2.0], [10.0], [14.0]])
    # groups {0,2} and {10,14}: squared deviations 1+1 and 4+4, over N=4
    assert oracle.within_group_variance(q, np.array([0, 1, 2, 3]), 2) == pytest.approx(2.5)
    assert oracle.within_group_variance(q, np.array([0, 2, 1, 3]), 2) == pytest.approx((25 + 25 + 36 + 36) / 4)


def test_eigh_split_beats_random_split():
    q = _rand((512, 8), 11) * np.linspace(3, 0.5, 8)
    w = oracle.within_group_variance(q, oracle.pddp(q, 32), 32)
    w_rand = oracle.within_group_variance(q, np.random.default_rng(12).permutation(512), 32)
    assert w < 0.8 * w_rand


def test_pddp_bh_shape():
    q = _rand((1, 3, 50, 4), 13)
    perm = oracle.pddp_bh(q, 8)
    assert perm.shape == (1, 3, 50)
    np.testing.assert_array_equal(perm[0, 2], oracle.pddp(q[0, 2], 8))


def test_odd_group_count_splits_at_floor_half():
    # N = 3C with C = 2.  A and B sit at the mean height, so x and y are
    # uncorrelated and the root's principal direction is exactly x: the split
    # at rank C*floor(3/2) = 2 puts {A, B} left and {C, D, E, F} right, and the
    # right node spreads along y and splits into {C, E} and {D, F}.  A split at
    # C*ceil(3/2) = 4 would put {A, B, C, D} left (split along x into {A, B},
    # {C, D}) and leave {E, F}.
    pts = np.array([[0.0, 1.5], [1.0, 1.5], [10.0, 0.0], [10.0, 3.0], [10.2, 0.0], [10.2, 3.0]])
    perm = oracle.pddp(pts, 2)
    groups = [set(g.tolist()) for g in oracle.groups_from_perm(perm, 2)]
    assert groups == [{0, 1}, {2, 4}, {3, 5}]


@pytest.mark.parametrize("steps", [1, 7, 32])
def test_power_iteration_closed_form_after_t_steps(steps):
    # four points +-sqrt(2) u1, +-sqrt(1.8) u2 with u1 = (1, 1)/sqrt2, u2 =
    # (1, -1)/sqrt2: mean 0, covariance eigenvalues 1 (u1) and 0.9 (u2), i.e.
    # [[0.95, 0.05], [0.05, 0.95]].  The start column is column 0 (equal
    # diagonals: the first), (0.95, 0.05) = (u1 + 0.9 u2)/sqrt2, so after t
    # steps the direction is proportional to u1 + 0.9^(t+1) u2.
    u1 = np.array([1.0, 1.0]) / np.sqrt(2)
    u2 = np.array([1.0, -1.0]) / np.sqrt(2)
    pts = np.stack([np.sqrt(2) * u1, -np.sqrt(2) * u1, np.sqrt(1.8) * u2, -np.sqrt(1.8) * u2])
    mu, vec = oracle.principal_direction(pts, mode="power", power_iters=steps)
    want = u1 + 0.9 ** (steps + 1) * u2
    want /= np.linalg.norm(want)
    np.testing.assert_allclose(mu, 0.0, atol=1e-15)
    np.testing.assert_allclose(vec, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("steps", [1, 5, 20])
def test_power_iteration_closed_form_unequal_diagonal(steps):
    # points +-sqrt(2) u1, +-sqrt(1.8) u2 with u1 = (cos 30, sin 30), u2 =
    # (-sin 30, cos 30): covariance u1 u1^T + 0.9 u2 u2^T, diagonal (0.975,
    # 0.925), so the start is column 0 = C e0 = cos30 u1 - 0.9 sin30 u2 and t
    # steps give a direction proportional to u1 - 0.9^(t+1) tan30 u2 (the
    # other column would give u1 + 0.9^(t+1) cot30 u2)
    th = np.pi / 6
    u1 = np.array([np.cos(th), np.sin(th)])
    u2 = np.array([-np.sin(th), np.cos(th)])
    pts = np.stack([np.sqrt(2) * u1, -np.sqrt(2) * u1, np.sqrt(1.8) * u2, -np.sqrt(1.8) * u2])
    _, vec = oracle.principal_direction(pts, mode="power", power_iters=steps)
    want = u1 - 0.9 ** (steps + 1) * np.tan(th) * u2
    want /= np.linalg.norm(want)
    want = want if want[np.argmax(np.abs(want))] > 0 else -want
    np.testing.assert_allclose(vec, want, rtol=0, atol=1e-12)
