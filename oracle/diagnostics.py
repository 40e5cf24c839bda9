"""Diagnostic selectors and groupings of the pages, in plain fp64 numpy.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle``: only tests/ and the
script ``oracle/diagnose.py`` use it; it imports nothing from the HIP path.

The ai.info page ("Methodology in Plain English", the diagnostic question) and
the wispaper.ai explainer ("Mean-pooled block scoring misses high-mass
tokens", "Token-level selection needs tile-aligned query groups") compare
selectors that keep, at a fixed budget, the highest-attention-mass
interactions of a dense attention map:

  block oracle      whole KV blocks per query block, chosen by exact mass;
  token oracle      individual KV tokens, one selection shared by a query block
                    (with PDDP query groups this is MC-Sparse's exact selection);
  per-query oracle  every query picks its own KV tokens;
  mean-pooled BSA   KV blocks chosen by the mean-pooled query-block / key-block
                    score (no dense map needed; the selection of standard
                    block-sparse attention);

and score them by attention recall (the dense attention mass the selection
keeps, averaged over queries) and by the relative L1 error of the output when
attention is renormalised over the selected keys (ai.info "Main Findings":
token granularity improves both at matched density).

The same pages set PDDP against k-means grouping: k-means gives clusters of
unequal size, and padding every cluster to whole tiles makes the interactions
actually computed exceed the nominal budget (ai.info "Main Findings", the
alignment inflation factor of k-means for blocks and for tokens; wispaper.ai
"Token-level selection needs tile-aligned query groups"; the agihunt.info
method paragraphs).  ``kmeans`` and ``alignment_inflation`` measure that.

Readings of what the pages leave open:
  D1 KV blocks are 64 consecutive keys (the kernels' key tile); the last one
     may be short;
  D2 a query block is one query group: C consecutive queries ("contiguous"),
     a PDDP group, or a k-means cluster of any size;
  D3 the budget is K = 128*floor(s*N/128) keys per query block (or per query),
     i.e. K/64 KV blocks for the block selectors;
  D4 recall = mean_i sum_{j in S(i)} P_ij; output error = sum |O_S - O| /
     sum |O| over all queries and channels, O_S renormalised over S(i), no
     residual;
  D5 mean-pooled score of KV block b for query block g: scale * mean(q_g) .
     mean(k_b); ties in every ranking go to the smaller id;
  D6 k-means is Lloyd's algorithm (squared Euclidean distance, assignment to
     the nearest centre with ties to the smaller centre id, centre = mean of
     its members, an empty cluster keeps its centre) for a fixed number of
     rounds from given initial centres; queries form ceil(N/C) clusters
     (as many as PDDP groups), keys ceil(N/64) clusters;
  D7 alignment inflation = the rows actually computed when every cluster is
     padded to whole tiles, over the real rows: sum_c ceil(n_c/T)*T / N.  Token
     selection pads only the query clusters (T = C); block selection over
     k-means key clusters also pads the key clusters (T = 64), so its factor is
     the product of the query and key factors (every key cluster equally
     likely to be chosen).
"""
from __future__ import annotations

from collections.abc import Sequence

import numpy as np

from .mcs_oracle import _f64, dense_attention, groups_from_perm, topk_indices

KV_BLOCK = 64

SELECTORS = ("mean_pooled_block", "block_oracle", "token_oracle", "per_query_oracle")


def _top_ids(score, n: int) -> np.ndarray:
    """The n ids of largest score (ties -> smaller id), ascending."""
    return topk_indices(score, n)


def _block_keys(blocks: np.ndarray, N: int) -> np.ndarray:
    keys = (blocks[:, None] * KV_BLOCK + np.arange(KV_BLOCK)[None, :]).ravel()
    return np.sort(keys[keys < N])


def block_sums(x: np.ndarray, N: int) -> np.ndarray:
    """Sums of x over KV blocks of KV_BLOCK consecutive keys (last one short)."""
    nb = -(-N // KV_BLOCK)
    pad = np.zeros(nb * KV_BLOCK)
    pad[:N] = x
    return pad.reshape(nb, KV_BLOCK).sum(axis=1)


def block_means(k) -> np.ndarray:
    """Mean key of every KV block (D1: KV_BLOCK consecutive keys, last one short)."""
    k = _f64(k)
    N = k.shape[0]
    return np.stack([k[b * KV_BLOCK:min(N, (b + 1) * KV_BLOCK)].mean(axis=0) for b in range(-(-N // KV_BLOCK))])


def mean_pooled_scores(q, kbar, rows, scale: float) -> np.ndarray:
    """D5: score of every KV block for the query block `rows`:
    scale * mean(q_rows) . mean(k_block)."""
    return scale * (kbar @ _f64(q)[rows].mean(axis=0))


def mean_pooled_blocks(q, kbar, rows, K: int, scale: float) -> np.ndarray:
    """The KV blocks mean-pooled block selection keeps for the query block
    `rows` at budget K (max(1, K // KV_BLOCK) blocks, D3, ties to the smaller
    block id), ascending."""
    return _top_ids(mean_pooled_scores(q, kbar, rows, scale), max(1, K // KV_BLOCK))


def diagnose_groups(q, k, v, groups: Sequence[np.ndarray], Ks: Sequence[int], scale: float) -> dict:
    """Recall and output error of the four selectors for one head.

    q: [Nq, D]; k, v: [N, D]; groups: the query blocks to score (disjoint
    arrays of query rows, any sizes; the statistics are over the queries they
    hold, so a sample of a grouping's blocks gives a sample estimate); Ks:
    budgets (keys per query block or per query; a multiple of KV_BLOCK for the
    block selectors).  Returns {K: {selector: {"recall": ..., "rel_l1": ...}}}.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    N = k.shape[0]
    groups = [np.asarray(g) for g in groups if len(g)]
    held = np.concatenate(groups)
    Nq = held.size
    o_held, lse_held = dense_attention(q[held], k, v, scale)
    o_dense = np.zeros((q.shape[0], v.shape[1]))
    lse = np.zeros(q.shape[0])
    o_dense[held], lse[held] = o_held, lse_held
    kbar = block_means(k)
    rec = {K: {s: 0.0 for s in SELECTORS} for K in Ks}
    err = {K: {s: 0.0 for s in SELECTORS} for K in Ks}
    for rows in groups:
        s = scale * (q[rows] @ k.T)
        p = np.exp(s - lse[rows][:, None])                 # exact probabilities [n, N]
        mass = p.sum(axis=0)                               # group mass per key
        pooled = mean_pooled_scores(q, kbar, rows, scale)  # mean-pooled block scores
        bmass = block_sums(mass, N)
        for K in Ks:
            nblk = max(1, K // KV_BLOCK)
            sets = {
                "mean_pooled_block": _block_keys(_top_ids(pooled, nblk), N),
                "block_oracle": _block_keys(_top_ids(bmass, nblk), N),
                "token_oracle": _top_ids(mass, K),
            }
            for name, ids in sets.items():
                ps = p[:, ids]
                kept = ps.sum(axis=1)
                rec[K][name] += kept.sum()
                err[K][name] += np.abs((ps @ v[ids]) / kept[:, None] - o_dense[rows]).sum()
        # per-query oracle: every row keeps its own K largest probabilities, a
        # tie at the K-th value going to the smaller key id.  One partition
        # per row gives the K-th largest value t of every budget; the kept set
        # is {p > t} plus the first (K - #{p > t}) keys with p == t.
        budgets = sorted(set(min(K, N) for K in Ks))
        for r0 in range(0, rows.size, 64):
            pr = p[r0:r0 + 64]
            ref = o_dense[rows[r0:r0 + 64]]
            part = -np.partition(-pr, [K - 1 for K in budgets], axis=1)
            for K in budgets:
                t = part[:, K - 1][:, None]
                gt = pr > t
                eq = pr == t
                need = K - gt.sum(axis=1, keepdims=True)
                keep = gt | (eq & (np.cumsum(eq, axis=1) <= need))
                pm = np.where(keep, pr, 0.0)
                kept = pm.sum(axis=1)
                for Kq in (Kq for Kq in Ks if min(Kq, N) == K):
                    rec[Kq]["per_query_oracle"] += kept.sum()
                    err[Kq]["per_query_oracle"] += np.abs((pm @ v) / kept[:, None] - ref).sum()
    total = np.abs(o_held).sum()
    return {K: {s: {"recall": rec[K][s] / Nq, "rel_l1": err[K][s] / total} for s in SELECTORS}
            for K in Ks}


def diagnose_head(q, k, v, perm, C: int, K: int, scale: float) -> dict:
    """diagnose_groups for the query blocks perm[g*C:(g+1)*C] and one budget K.

    Returns {selector: {"recall": ..., "rel_l1": ...}}.
    """
    return diagnose_groups(q, k, v, groups_from_perm(perm, C), [K], scale)[K]


def kmeans(x, init, rounds: int):
    """Lloyd's k-means (reading D6) from the given initial centres.

    x: [n, D] points; init: [k, D] initial centres; rounds: assignment/update
    rounds.  Returns (labels [n] int, centres [k, D], inertia per round [rounds]).
    """
    x = _f64(x)
    c = _f64(init).copy()
    k = c.shape[0]
    xx = (x * x).sum(axis=1)
    inertia = []
    labels = np.zeros(x.shape[0], dtype=np.int64)
    for _ in range(rounds):
        d = xx[:, None] - 2.0 * (x @ c.T) + (c * c).sum(axis=1)[None, :]
        labels = np.argmin(d, axis=1)                      # first minimum: smaller centre id
        inertia.append(float(((x - c[labels]) ** 2).sum()))
        counts = np.bincount(labels, minlength=k)
        sums = np.zeros_like(c)
        np.add.at(sums, labels, x)
        nz = counts > 0
        c[nz] = sums[nz] / counts[nz][:, None]
    return labels, c, np.array(inertia)


def cluster_groups(labels, k: int) -> list[np.ndarray]:
    """Member rows of each of the k clusters (ascending), empty ones included."""
    order = np.argsort(labels, kind="stable")
    bounds = np.searchsorted(labels[order], np.arange(k + 1))
    return [order[bounds[j]:bounds[j + 1]] for j in range(k)]


def alignment_inflation(sizes, tile: int) -> float:
    """Rows computed when every cluster is padded to whole tiles, over the real
    rows (reading D7): sum ceil(n/tile)*tile / sum n."""
    sizes = np.asarray(sizes, dtype=np.int64)
    return float((-(-sizes // tile) * tile).sum() / sizes.sum())
