"""Planted mistakes in the oracle, for checking that its pins catch them.

Each mutant replaces one exact piece of the oracle's source with a plausible
slip (a dropped term, a wrong sign, a wrong operand or index, a wrong rule).
tests/conftest.py applies the mutant named by the environment variable
MCS_ORACLE_MUTANT before any test imports the oracle, by loading the mutated
source in place of the oracle module; tests/test_oracle_mutations.py runs the
oracle's pin tests once per mutant and requires every run to fail.  The oracle
files themselves are never changed.
"""
from __future__ import annotations

import importlib.util
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MCS = "oracle/mcs_oracle.py"
DIAG = "oracle/diagnostics.py"

# name -> (file, original text, mutated text)
MUTANTS = {
    "scores_drop_scale": (MCS, "return float(scale) * (_f64(q) @ _f64(k).T)", "return (_f64(q) @ _f64(k).T)"),
    "lse_drop_max": (MCS, "lse[r0:r0 + ROW_BLOCK] = (m + np.log(z))[:, 0]",
                     "lse[r0:r0 + ROW_BLOCK] = (np.log(z))[:, 0]"),
    "dense_unnormalised": (MCS, "out[r0:r0 + ROW_BLOCK] = (e / z) @ v", "out[r0:r0 + ROW_BLOCK] = e @ v"),
    "probabilities_sign": (MCS, "np.exp(attention_scores(q, k, scale) - _f64(lse)[:, None])",
                           "np.exp(attention_scores(q, k, scale) + _f64(lse)[:, None])"),
    "mass_mean_not_sum": (MCS, "probabilities(q[members], k, lse[members], scale).sum(axis=0)",
                          "probabilities(q[members], k, lse[members], scale).mean(axis=0)"),
    "topk_ties_to_larger_id": (MCS, "order = np.lexsort((j, -mass_row))", "order = np.lexsort((-j, -mass_row))"),
    "topk_skips_the_largest": (MCS, "return np.sort(order[:K]).astype(np.int64)",
                               "return np.sort(order[1:K + 1]).astype(np.int64)"),
    "topk_not_ascending": (MCS, "return np.sort(order[:K]).astype(np.int64)", "return order[:K].astype(np.int64)"),
    "sparse_not_renormalised": (MCS, "out[members] = (e / e.sum(axis=1, keepdims=True)) @ v[sel]",
                                "out[members] = e @ v[sel]"),
    "sparse_keys_as_values": (MCS, "out[members] = (e / e.sum(axis=1, keepdims=True)) @ v[sel]",
                              "out[members] = (e / e.sum(axis=1, keepdims=True)) @ k[sel]"),
    "residual_sign": (MCS, "return _f64(o_dense) - _f64(o_sparse)", "return _f64(o_sparse) - _f64(o_dense)"),
    "covariance_not_centred": (MCS, "    xc = x - mu\n", "    xc = x\n"),
    "sign_rule_flipped": (MCS, "return -vec if vec[i] < 0 else vec", "return -vec if vec[i] > 0 else vec"),
    "power_start_smallest_diagonal": (MCS, "vec = cov[:, int(np.argmax(np.diag(cov)))].copy()",
                                      "vec = cov[:, int(np.argmin(np.diag(cov)))].copy()"),
    "split_rank_ceil": (MCS, "r = C * (g // 2)", "r = C * (-(-g // 2))"),
    "split_order_descending": (MCS, "order = np.lexsort((ids, proj))", "order = np.lexsort((ids, -proj))"),
    "variance_over_groups": (MCS, "    return total / q.shape[0]\n", "    return total / len(groups_from_perm(perm, C))\n"),
    "power_one_step_short": (MCS, "for _ in range(power_iters):", "for _ in range(power_iters - 1):"),
    "groups_drop_ragged_tail": (MCS, "return [perm[g * C:min((g + 1) * C, n)] for g in range(-(-n // C))]",
                                "return [perm[g * C:min((g + 1) * C, n)] for g in range(n // C)]"),
    "mean_pooling_uses_max": (DIAG, "k[b * KV_BLOCK:min(N, (b + 1) * KV_BLOCK)].mean(axis=0)",
                              "k[b * KV_BLOCK:min(N, (b + 1) * KV_BLOCK)].max(axis=0)"),
    "recall_not_averaged": (DIAG, '{"recall": rec[K][s] / Nq,', '{"recall": rec[K][s],'),
    "reuse_subtracts_residual": (MCS, "out = out + _f64(residual)", "out = out - _f64(residual)"),
    "lse_log2": (MCS, "lse[r0:r0 + ROW_BLOCK] = (m + np.log(z))[:, 0]",
                 "lse[r0:r0 + ROW_BLOCK] = (m + np.log2(z))[:, 0]"),
    "pddp_default_power": (MCS, 'def pddp(q, C: int, mode: str = "eigh"', 'def pddp(q, C: int, mode: str = "power"'),
    "retained_mass_first_ids": (MCS, "mass[g, np.asarray(idx[g])].sum()", "mass[g, :len(idx[g])].sum()"),
    "block_keys_off_by_one": (DIAG, "keys = (blocks[:, None] * KV_BLOCK + np.arange(KV_BLOCK)[None, :]).ravel()",
                              "keys = (blocks[:, None] * KV_BLOCK + 1 + np.arange(KV_BLOCK)[None, :]).ravel()"),
    "kmeans_centre_is_sum": (DIAG, "c[nz] = sums[nz] / counts[nz][:, None]", "c[nz] = sums[nz]"),
    "inflation_over_clusters": (DIAG, "return float((-(-sizes // tile) * tile).sum() / sizes.sum())",
                                "return float((-(-sizes // tile) * tile).sum() / sizes.size)"),
    "topk_smallest_mass": (MCS, "order = np.lexsort((j, -mass_row))", "order = np.lexsort((j, mass_row))"),
    "perquery_keeps_one_less": (DIAG, "need = K - gt.sum(axis=1, keepdims=True)",
                                "need = K - 1 - gt.sum(axis=1, keepdims=True)"),
    "token_oracle_smallest_mass": (DIAG, '"token_oracle": _top_ids(mass, K),', '"token_oracle": _top_ids(-mass, K),'),
    "kmeans_farthest_centre": (DIAG, "labels = np.argmin(d, axis=1)", "labels = np.argmax(d, axis=1)"),
    "inflation_rounds_down": (DIAG, "(-(-sizes // tile) * tile)", "((sizes // tile) * tile)"),
    "pddp_ties_to_larger_id": (MCS, "order = np.lexsort((ids, proj))", "order = np.lexsort((-ids, proj))"),
    "pddp_right_child_first": (MCS, "        split(ids[order[:r]])\n        split(ids[order[r:]])\n",
                               "        split(ids[order[r:]])\n        split(ids[order[:r]])\n"),
    "variance_global_mean": (MCS, "total += float(((x - x.mean(axis=0)) ** 2).sum())",
                             "total += float(((x - q.mean(axis=0)) ** 2).sum())"),
    "dense_keys_as_values": (MCS, "out[r0:r0 + ROW_BLOCK] = (e / z) @ v", "out[r0:r0 + ROW_BLOCK] = (e / z) @ k"),
    "mass_lse_unpermuted": (MCS, "probabilities(q[members], k, lse[members], scale).sum(axis=0)",
                            "probabilities(q[members], k, lse[:len(members)], scale).sum(axis=0)"),
    "sparse_queries_unpermuted": (MCS, "s = attention_scores(q[members], k[sel], scale)",
                                  "s = attention_scores(q[:len(members)], k[sel], scale)"),
    "sign_uses_max_not_abs": (MCS, "i = int(np.argmax(np.abs(vec)))", "i = int(np.argmax(vec))"),
    "projection_on_the_mean": (MCS, "proj = (q[ids] - mu) @ vec", "proj = (q[ids] - mu) @ mu"),
    "pooled_query_sum_over_all": (DIAG, "return scale * (kbar @ _f64(q)[rows].mean(axis=0))",
                                  "return scale * (kbar @ _f64(q).mean(axis=0))"),
    "sparse_lse_drops_max": (MCS, "out[members] = m + np.log(np.exp(s - m[:, None]).sum(axis=1))",
                             "out[members] = np.log(np.exp(s - m[:, None]).sum(axis=1))"),
    "kept_mass_first_keys": (MCS, "out[members] = probabilities(q[members], k[sel], lse[members], scale).sum(axis=1)",
                             "out[members] = probabilities(q[members], k[:sel.size], lse[members], scale).sum(axis=1)"),
    "pooled_blocks_budget_off_by_one": (DIAG, "return _top_ids(mean_pooled_scores(q, kbar, rows, scale), max(1, K // KV_BLOCK))",
                                        "return _top_ids(mean_pooled_scores(q, kbar, rows, scale), max(1, K // KV_BLOCK) + 1)"),
    "block_oracle_uses_first_block": (DIAG, '"block_oracle": _block_keys(_top_ids(bmass, nblk), N),',
                                      '"block_oracle": _block_keys(np.arange(nblk), N),'),
    "perquery_ties_to_larger_id": (DIAG, "keep = gt | (eq & (np.cumsum(eq, axis=1) <= need))",
                                   "keep = gt | (eq & (np.cumsum(eq[:, ::-1], axis=1)[:, ::-1] <= need))"),
    "rel_l1_over_kept_total": (DIAG, "total = np.abs(o_held).sum()", "total = np.abs(o_held).sum() / Nq"),
}


def mutated_source(name: str) -> tuple[str, str]:
    path, old, new = MUTANTS[name]
    src = open(os.path.join(ROOT, path)).read()
    if src.count(old) != 1:
        raise AssertionError(f"mutant {name}: the text to replace occurs {src.count(old)} times in {path}")
    return path, src.replace(old, new)


def apply(name: str) -> None:
    """Load the oracle with the named mutant in place of the original module."""
    import oracle
    path, src = mutated_source(name)
    modname = "oracle.mcs_oracle" if path == MCS else "oracle.diagnostics"
    spec = importlib.util.spec_from_loader(modname, loader=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__package__ = "oracle"
    mod.__file__ = os.path.join(ROOT, path)
    sys.modules[modname] = mod
    exec(compile(src, mod.__file__, "exec"), mod.__dict__)
    if path == MCS:
        for attr in getattr(mod, "__all__", []) + ["default_scale"]:
            setattr(oracle, attr, getattr(mod, attr))
        setattr(oracle, "mcs_oracle", mod)
        sys.modules.pop("oracle.diagnostics", None)      # re-imported against the mutant
    else:
        setattr(oracle, "diagnostics", mod)
