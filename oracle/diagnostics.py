"""Diagnostic selectors of the pages, in plain fp64 numpy (test infrastructure).

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

Readings of what the pages leave open (listed in the design notes as well):
  D1 KV blocks are 64 consecutive keys (the kernels' key tile); the last one
     may be short;
  D2 a query block is a query group of C queries: C consecutive queries
     ("contiguous"), or a PDDP group;
  D3 the budget is K = 128*floor(s*N/128) keys per query block (or per query),
     i.e. K/64 KV blocks for the block selectors;
  D4 recall = mean_i sum_{j in S(i)} P_ij; output error = sum |O_S - O| /
     sum |O| over all queries and channels, O_S renormalised over S(i), no
     residual;
  D5 mean-pooled score of KV block b for query block g: scale * mean(q_g) .
     mean(k_b); ties in every ranking go to the smaller id.
"""
from __future__ import annotations

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


def diagnose_head(q, k, v, perm, C: int, K: int, scale: float) -> dict:
    """Recall and output error of the four selectors for one head.

    q: [Nq, D]; k, v: [N, D]; perm: the query grouping (group g =
    perm[g*C:(g+1)*C]);
    K: keys per query block (a multiple of KV_BLOCK for the block selectors).
    Returns {selector: {"recall": ..., "rel_l1": ...}}.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    Nq, N = q.shape[0], k.shape[0]
    o_dense, lse = dense_attention(q, k, v, scale)
    nblk = max(1, K // KV_BLOCK)
    kbar = np.stack([k[b * KV_BLOCK:min(N, (b + 1) * KV_BLOCK)].mean(axis=0)
                     for b in range(-(-N // KV_BLOCK))])
    rec = {s: 0.0 for s in SELECTORS}
    err = {s: 0.0 for s in SELECTORS}
    for rows in groups_from_perm(perm, C):
        s = scale * (q[rows] @ k.T)
        p = np.exp(s - lse[rows][:, None])                 # exact probabilities [n, N]
        mass = p.sum(axis=0)                               # group mass per key
        sets = {
            "mean_pooled_block": _block_keys(_top_ids(scale * (kbar @ q[rows].mean(axis=0)), nblk), N),
            "block_oracle": _block_keys(_top_ids(block_sums(mass, N), nblk), N),
            "token_oracle": _top_ids(mass, K),
        }
        for name, ids in sets.items():
            ps = p[:, ids]
            kept = ps.sum(axis=1)
            rec[name] += kept.sum()
            o = (ps @ v[ids]) / kept[:, None]
            err[name] += np.abs(o - o_dense[rows]).sum()
        # per-query oracle: every row its own K largest probabilities (a tie at
        # the K-th value may be broken either way: the kept mass is the same)
        if K >= N:
            pm = p
        else:
            top = np.argpartition(-p, K - 1, axis=1)[:, :K]
            pm = np.zeros_like(p)
            np.put_along_axis(pm, top, np.take_along_axis(p, top, axis=1), axis=1)
        kept = pm.sum(axis=1)
        rec["per_query_oracle"] += kept.sum()
        err["per_query_oracle"] += np.abs((pm @ v) / kept[:, None] - o_dense[rows]).sum()
    total = np.abs(o_dense).sum()
    return {s: {"recall": rec[s] / Nq, "rel_l1": err[s] / total} for s in SELECTORS}
