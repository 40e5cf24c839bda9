"""Plain, slow fp64 CPU oracle for the MC-Sparse token-sparse attention hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The HIP
library never links, imports or executes anything here, and this module imports
nothing from the HIP path (it needs numpy only).

What it computes is read from the web pages about the paper "MC-Sparse:
Deconstructing and Closing the Dense-Sparse Attention Gap in Diffusion
Transformers" (arXiv 2610.06801).  Citations name the page by its site and the
section on it:

  [ai.info]      AI summary page; sections "Key Contributions", "Main Findings",
                 "Methodology in Plain English".
  [wispaper.ai]  explainer page; sections "Mean-pooled block scoring misses
                 high-mass tokens", "Token-level selection needs tile-aligned
                 query groups", "Reused exact selection beats recomputed mean
                 pooling", "Residual correction recovers the discarded tail".
  [agihunt.info] Chinese summary page; the method paragraphs before the main
                 results table.

Conventions (all arrays are numpy, all arithmetic is float64):
  * One attention head at a time: q, k, v are [N, D]; ``*_bh`` wrappers loop
    over the leading [B, H] axes of [B, H, N, D] arrays.
  * Inputs are whatever the caller passes (the tests pass the exact bf16 values
    the GPU sees, upcast to float64).
  * A query group is a set of query rows.  ``perm`` is a permutation of
    0..N-1; group g is perm[g*C : min((g+1)*C, N)], G = ceil(N / C).
  * ``idx`` holds, per group, the K selected KV token ids (ascending).

Readings of points the pages leave open:
  R1 softmax scale tau = 1/sqrt(D) is passed in by the caller;
  R2 no mask: every query sees all N keys (bidirectional DiT attention);
  R3 top-K ties: larger mass first, equal mass -> smaller KV id; output ascending;
  R4 sparse softmax renormalises over the selected set;
  R5 PDDP split at rank C*floor(g/2) of the projection order, with g =
     ceil(n/C) groups in the node; the exact split is the median when g is
     even and n = g*C; the remainder group ends up rightmost;
  R6 principal direction sign: largest-|.| component positive (ties -> lowest id);
  R6b equal projections are ordered by query id;
  R7 the residual is O_dense - O_sparse formed at the anchor with the anchor's
     own Q, K, V and the freshly built groups and indices;
  R8 the principal direction of a PDDP node is what the term means: the
     eigenvector of the largest eigenvalue of the node's covariance (exact,
     from numpy's symmetric eigensolver, the default).  The pages compute it
     by batched power iteration (ai.info "Key Contributions") but give no step
     count or start, so a fixed number of power steps is no definition of it;
     mode="power" runs such steps from the covariance column of largest
     diagonal, as a mirror of the iteration for tests.

Pins (what ties each function to something other than itself) live in
``tests/test_oracle_*.py``; every function below is pinned there.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "attention_scores", "dense_attention", "probabilities", "groups_from_perm",
    "group_mass", "topk_indices", "select", "retained_mass", "sparse_attention",
    "residual", "anchor_step", "reuse_step", "principal_direction", "pddp", "sparse_lse", "kept_mass",
    "within_group_variance", "dense_attention_bh", "sparse_attention_bh",
    "select_bh", "pddp_bh", "default_scale",
]

# Rows of the score matrix are independent, so the row-wise definitions below
# walk the queries in blocks of this many rows purely to bound memory (an N x N
# float64 matrix at N = 75600 would be 46 GB).
ROW_BLOCK = 512


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# Dense attention with row log-sum-exp
# [ai.info "Methodology in Plain English": pass one of the selector yields the
#  attention output together with one log-sum-exp per query row]
# ---------------------------------------------------------------------------

def attention_scores(q, k, scale: float) -> np.ndarray:
    """s_ij = scale * q_i . k_j for all i, j (R1, R2: no mask)."""
    return float(scale) * (_f64(q) @ _f64(k).T)


def dense_attention(q, k, v, scale: float):
    """Exact softmax attention of one head and its natural-log row LSE.

    For each query row i:  m_i = max_j s_ij,
    lse_i = m_i + ln sum_j exp(s_ij - m_i),  P_ij = exp(s_ij - lse_i),
    O_i = sum_j P_ij v_j.   Returns (O [N, D], lse [N]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    n = q.shape[0]
    out = np.empty((n, v.shape[1]))
    lse = np.empty(n)
    for r0 in range(0, n, ROW_BLOCK):
        s = attention_scores(q[r0:r0 + ROW_BLOCK], k, scale)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=1, keepdims=True)
        lse[r0:r0 + ROW_BLOCK] = (m + np.log(z))[:, 0]
        out[r0:r0 + ROW_BLOCK] = (e / z) @ v
    return out, lse


def probabilities(q, k, lse, scale: float) -> np.ndarray:
    """Recovered attention probabilities P_ij = exp(s_ij - lse_i).

    [ai.info "Methodology in Plain English": the second pass recomputes the QK
     scores to recover the probabilities from the first pass's LSE]
    """
    return np.exp(attention_scores(q, k, scale) - _f64(lse)[:, None])


# ---------------------------------------------------------------------------
# Group-wise aggregation and top-K selection
# [ai.info "Methodology in Plain English" (two-pass selection with group-wise
#  aggregation and top-K); agihunt.info method paragraphs (the objective is the
#  largest summed attention weight of the group over a budget of K KV tokens);
#  wispaper.ai "Token-level selection needs tile-aligned query groups"]
# ---------------------------------------------------------------------------

def groups_from_perm(perm, C: int) -> list[np.ndarray]:
    """Split a permutation into G = ceil(N/C) consecutive groups of C ids."""
    perm = np.asarray(perm, dtype=np.int64)
    n = perm.shape[0]
    return [perm[g * C:min((g + 1) * C, n)] for g in range(-(-n // C))]


def group_mass(q, k, lse, perm, C: int, scale: float) -> np.ndarray:
    """M[g, j] = sum over queries i of group g of P_ij.  Shape [G, N]."""
    q, k, lse = _f64(q), _f64(k), _f64(lse)
    groups = groups_from_perm(perm, C)
    mass = np.empty((len(groups), k.shape[0]))
    for g, members in enumerate(groups):
        mass[g] = probabilities(q[members], k, lse[members], scale).sum(axis=0)
    return mass


def topk_indices(mass_row, K: int) -> np.ndarray:
    """The K ids j of largest mass_row[j] (R3), returned ascending.

    Ordering key is (-mass, j): larger mass first, ties to the smaller id.  The
    arithmetic type of the comparison is that of ``mass_row`` (float64 masses
    from this oracle, or float32 masses when a test compares a given float32
    score array decision-for-decision).
    """
    mass_row = np.asarray(mass_row)
    j = np.arange(mass_row.shape[0])
    order = np.lexsort((j, -mass_row))
    return np.sort(order[:K]).astype(np.int64)


def select(q, k, lse, perm, C: int, K: int, scale: float):
    """Exact selection for one head: (idx [G, K] ascending, mass [G, N])."""
    mass = group_mass(q, k, lse, perm, C, scale)
    idx = np.stack([topk_indices(row, K) for row in mass])
    return idx, mass


def retained_mass(mass, idx) -> np.ndarray:
    """rho_g = sum of M[g, j] over the selected ids of group g."""
    mass = _f64(mass)
    return np.array([mass[g, np.asarray(idx[g])].sum() for g in range(mass.shape[0])])


# ---------------------------------------------------------------------------
# Token-sparse attention and the residual
# [wispaper.ai "Token-level selection needs tile-aligned query groups": each
#  group of C queries shares one selection of individually gathered KV tokens;
#  wispaper.ai "Residual correction recovers the discarded tail": the anchor
#  records dense minus sparse output and reuse steps add it back]
# ---------------------------------------------------------------------------

def sparse_attention(q, k, v, perm, idx, C: int, scale: float, residual=None):
    """O_i = sum_{j in idx_g} softmax_j(s_ij over idx_g) v_j for i in group g (R4).

    ``residual`` (same shape as the output, indexed by query id) is added when
    given: the reuse-step output.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    out = np.zeros((q.shape[0], v.shape[1]))
    for g, members in enumerate(groups_from_perm(perm, C)):
        sel = np.asarray(idx[g], dtype=np.int64)
        s = attention_scores(q[members], k[sel], scale)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        out[members] = (e / e.sum(axis=1, keepdims=True)) @ v[sel]
    if residual is not None:
        out = out + _f64(residual)
    return out


def sparse_lse(q, k, perm, idx, C: int, scale: float) -> np.ndarray:
    """Per query i of group g: ln sum_{j in idx_g} exp(s_ij), the normaliser
    of the sparse softmax over the selected keys (natural log).  idx[g] may
    have any length (a per-group budget)."""
    q, k = _f64(q), _f64(k)
    out = np.empty(q.shape[0])
    for g, members in enumerate(groups_from_perm(perm, C)):
        s = attention_scores(q[members], k[np.asarray(idx[g], dtype=np.int64)], scale)
        m = s.max(axis=1)
        out[members] = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    return out


def kept_mass(q, k, lse, perm, idx, C: int, scale: float) -> np.ndarray:
    """Per query i of group g: sum_{j in idx_g} P_ij, the dense attention mass
    the selection keeps (the attention recall of one query; ai.info "Main
    Findings" and "Methodology in Plain English")."""
    q, k, lse = _f64(q), _f64(k), _f64(lse)
    out = np.empty(q.shape[0])
    for g, members in enumerate(groups_from_perm(perm, C)):
        sel = np.asarray(idx[g], dtype=np.int64)
        out[members] = probabilities(q[members], k[sel], lse[members], scale).sum(axis=1)
    return out


def residual(o_dense, o_sparse) -> np.ndarray:
    """R = O_dense - O_sparse (R7)."""
    return _f64(o_dense) - _f64(o_sparse)


def anchor_step(q, k, v, C: int, K: int, scale: float, pddp_mode: str = "eigh",
                power_iters: int = 32):
    """One anchor step of one head, in the pages' order.

    Groups (PDDP), dense attention + LSE (pass 1), group mass + top-K (pass 2),
    sparse attention with the fresh metadata, residual.  The step's output is
    the dense output (the anchor closes a dense segment).
    [ai.info "Methodology in Plain English"; wispaper.ai "Reused exact
     selection beats recomputed mean pooling"]
    """
    perm = pddp(q, C, mode=pddp_mode, power_iters=power_iters)
    o_dense, lse = dense_attention(q, k, v, scale)
    idx, mass = select(q, k, lse, perm, C, K, scale)
    o_sp = sparse_attention(q, k, v, perm, idx, C, scale)
    return {"out": o_dense, "perm": perm, "lse": lse, "idx": idx, "mass": mass,
            "o_sparse": o_sp, "residual": residual(o_dense, o_sp)}


def reuse_step(q, k, v, perm, idx, res, C: int, scale: float) -> np.ndarray:
    """Reuse step: sparse attention on the current Q, K, V plus the cached residual."""
    return sparse_attention(q, k, v, perm, idx, C, scale, residual=res)


# ---------------------------------------------------------------------------
# Median-split PDDP grouping
# [ai.info "Key Contributions" and "Methodology in Plain English"; wispaper.ai
#  "Token-level selection needs tile-aligned query groups": recursively project
#  each group on its principal direction and split the ordered queries at the
#  median until every group holds exactly C queries; agihunt.info method
#  paragraphs]
# ---------------------------------------------------------------------------

def _canonical_sign(vec: np.ndarray) -> np.ndarray:
    """R6: make the largest-magnitude component positive (first one on ties)."""
    i = int(np.argmax(np.abs(vec)))
    return -vec if vec[i] < 0 else vec


def principal_direction(x, mode: str = "eigh", power_iters: int = 16):
    """Mean and unit principal direction of the rows of x.

    The covariance is (1/n) sum (x_i - mu)(x_i - mu)^T.  ``eigh`` takes the
    eigenvector of its largest eigenvalue.  ``power`` runs a fixed number of
    power-iteration steps instead (the batched power iteration the pages name),
    started from the covariance column with the largest diagonal entry (first
    on ties) and normalised after every step.
    """
    x = _f64(x)
    mu = x.mean(axis=0)
    xc = x - mu
    cov = xc.T @ xc / x.shape[0]
    if mode == "eigh":
        _, vecs = np.linalg.eigh(cov)
        vec = vecs[:, -1]
    elif mode == "power":
        vec = cov[:, int(np.argmax(np.diag(cov)))].copy()
        nrm = np.linalg.norm(vec)
        vec = vec / nrm if nrm > 0 else np.eye(cov.shape[0])[0]
        for _ in range(power_iters):
            w = cov @ vec
            nrm = np.linalg.norm(w)
            if nrm == 0:
                break
            vec = w / nrm
    else:
        raise ValueError(f"unknown mode {mode!r}")
    return mu, _canonical_sign(vec)


def pddp(q, C: int, mode: str = "eigh", power_iters: int = 32) -> np.ndarray:
    """Median-split PDDP of one head's queries into exactly-C groups.

    Node with ids I (n = |I|, g = ceil(n/C) groups): a leaf when g == 1;
    otherwise order I by (projection on the node's principal direction, query
    id (R6b)), left child = first C*floor(g/2) ids, right child = the rest (R5).
    Leaves are emitted left-first, so perm[g*C:(g+1)*C] is group g.  The
    direction is the exact top eigenvector by default (R8); mode="power"
    takes power_iters power steps instead.
    Returns perm [N].
    """
    q = _f64(q)
    leaves: list[np.ndarray] = []

    def split(ids: np.ndarray) -> None:
        n = ids.shape[0]
        g = -(-n // C)
        if g <= 1:
            leaves.append(ids)
            return
        mu, vec = principal_direction(q[ids], mode=mode, power_iters=power_iters)
        proj = (q[ids] - mu) @ vec
        order = np.lexsort((ids, proj))      # by projection, then query id
        r = C * (g // 2)
        split(ids[order[:r]])
        split(ids[order[r:]])

    split(np.arange(q.shape[0], dtype=np.int64))
    return np.concatenate(leaves)


def within_group_variance(q, perm, C: int) -> float:
    """W = (1/N) sum_g sum_{i in g} |q_i - mean_g|^2 for the groups of perm."""
    q = _f64(q)
    total = 0.0
    for members in groups_from_perm(perm, C):
        x = q[members]
        total += float(((x - x.mean(axis=0)) ** 2).sum())
    return total / q.shape[0]


# ---------------------------------------------------------------------------
# [B, H, ...] wrappers (heads are independent)
# ---------------------------------------------------------------------------

def _heads(x):
    x = np.asarray(x)
    return x.reshape((-1,) + x.shape[2:]), x.shape[:2]


def dense_attention_bh(q, k, v, scale: float):
    qs, bh = _heads(q)
    ks, _ = _heads(k)
    vs, _ = _heads(v)
    outs, lses = zip(*(dense_attention(qs[i], ks[i], vs[i], scale) for i in range(qs.shape[0])))
    return np.stack(outs).reshape(bh + outs[0].shape), np.stack(lses).reshape(bh + lses[0].shape)


def sparse_attention_bh(q, k, v, perm, idx, C: int, scale: float, residual=None):
    qs, bh = _heads(q)
    ks, _ = _heads(k)
    vs, _ = _heads(v)
    ps, _ = _heads(perm)
    ix, _ = _heads(idx)
    rs = _heads(residual)[0] if residual is not None else None
    outs = [sparse_attention(qs[i], ks[i], vs[i], ps[i], ix[i], C, scale,
                             None if rs is None else rs[i]) for i in range(qs.shape[0])]
    return np.stack(outs).reshape(bh + outs[0].shape)


def select_bh(q, k, lse, perm, C: int, K: int, scale: float):
    qs, bh = _heads(q)
    ks, _ = _heads(k)
    ls, _ = _heads(lse)
    ps, _ = _heads(perm)
    res = [select(qs[i], ks[i], ls[i], ps[i], C, K, scale) for i in range(qs.shape[0])]
    idx = np.stack([r[0] for r in res]).reshape(bh + res[0][0].shape)
    mass = np.stack([r[1] for r in res]).reshape(bh + res[0][1].shape)
    return idx, mass


def pddp_bh(q, C: int, mode: str = "eigh", power_iters: int = 32) -> np.ndarray:
    qs, bh = _heads(q)
    perms = [pddp(qs[i], C, mode=mode, power_iters=power_iters) for i in range(qs.shape[0])]
    return np.stack(perms).reshape(bh + perms[0].shape)


def default_scale(D: int) -> float:
    """R1: tau = 1/sqrt(D)."""
    return 1.0 / math.sqrt(D)
