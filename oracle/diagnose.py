"""Recall, output error and k-means alignment inflation on synthetic heads.

    python -m oracle.diagnose [--workloads tiny small asset3d] [--heads 1] [--rounds 20] [--groups 48]

Test-infrastructure script (it uses only ``oracle`` and the seeded input
generators): for one or more heads of each workload, every selector of
``oracle.diagnostics`` at densities 0.1, 0.2 and 0.3 (K = 128*floor(s*N/128)),
with three query groupings: C consecutive queries, PDDP groups, and k-means
clusters (ceil(N/C) of them, Lloyd's algorithm from distinct queries drawn
with a seeded generator); recall and output error are means over the queries
of a seeded sample of --groups query blocks per grouping (all of them when a
grouping has fewer).  A second table gives the alignment inflation of
k-means (query clusters padded to C; key clusters, ceil(N/64) of them, padded
to 64) and the recall k-means grouping keeps when its inflated compute is held
to the nominal budget (token oracle with floor(K/f_tok) keys, block oracle
with the largest multiple of 64 below K/f_blk).  Prints markdown ("-" where
the budget is below one 128-key step).
"""
from __future__ import annotations

import argparse
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from oracle import diagnostics as dg  # noqa: E402
from token_sparse_attention_amd import synth  # noqa: E402

LABELS = {"mean_pooled_block": "mean-pooled blocks", "block_oracle": "block oracle",
          "token_oracle": "token oracle", "per_query_oracle": "per-query oracle"}
DENS = (0.1, 0.2, 0.3)


def _cell(r, K, sel, key):
    return f"{r[K][sel][key]:.3f}" if K in r else "-"


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workloads", nargs="+", default=["tiny", "small", "asset3d"])
    ap.add_argument("--heads", type=int, default=1)
    ap.add_argument("--rounds", type=int, default=20, help="k-means rounds")
    ap.add_argument("--groups", type=int, default=48, help="query blocks scored per grouping")
    args = ap.parse_args(argv)
    main_rows, km_rows = [], []
    for name in args.workloads:
        w = synth.WORKLOADS[name]
        heads = [(0, h) for h in range(min(args.heads, w.H))]
        x = synth.generate(name, heads=heads)
        scale = 1.0 / math.sqrt(w.D)
        Ks = {s: 128 * int(s * w.N // 128) for s in DENS}
        nominal = [K for K in Ks.values() if K > 0]
        G = -(-w.N // w.C)
        for i, (b, h) in enumerate(heads):
            q, k, v = (synth.to_f64(x[t][0, i]) for t in "qkv")
            t0 = time.time()
            rng = np.random.default_rng(7000 + 100 * w.cfg_id + h)
            qlab, _, _ = dg.kmeans(q, q[rng.choice(w.N, G, replace=False)], args.rounds)
            klab, _, _ = dg.kmeans(k, k[rng.choice(w.N, -(-w.N // 64), replace=False)], args.rounds)
            qgroups = dg.cluster_groups(qlab, G)
            f_tok = dg.alignment_inflation([g.size for g in qgroups if g.size], w.C)
            f_key = dg.alignment_inflation(np.bincount(klab)[np.bincount(klab) > 0], 64)
            f_blk = f_tok * f_key
            matched_tok = {K: int(K / f_tok) for K in nominal}
            matched_blk = {K: 64 * int(K / f_blk / 64) for K in nominal}
            def sample(groups):
                groups = [g for g in groups if g.size]
                if len(groups) <= args.groups:
                    return groups
                return [groups[i] for i in np.sort(rng.choice(len(groups), args.groups, replace=False))]

            res = {
                "contiguous": dg.diagnose_groups(q, k, v, sample(dg.groups_from_perm(np.arange(w.N), w.C)),
                                                 nominal, scale),
                "PDDP": dg.diagnose_groups(q, k, v, sample(dg.groups_from_perm(oracle.pddp(q, w.C), w.C)),
                                           nominal, scale),
            }
            extra = sorted(set(matched_tok.values()) | {m for m in matched_blk.values() if m > 0})
            res["k-means"] = dg.diagnose_groups(q, k, v, sample(qgroups), sorted(set(nominal) | set(extra)), scale)
            for gname, r in res.items():
                for sel in dg.SELECTORS:
                    rec = " | ".join(_cell(r, Ks[s], sel, "recall") for s in DENS)
                    err = " | ".join(_cell(r, Ks[s], sel, "rel_l1") for s in DENS)
                    main_rows.append(f"| {name} (h={h}) | {gname} | {LABELS[sel]} | {rec} | {err} |")
            km = res["k-means"]
            tok = " / ".join(f"{km[matched_tok[Ks[s]]]['token_oracle']['recall']:.3f}" if Ks[s] > 0 else "-"
                             for s in DENS)
            blk = " / ".join(f"{km[matched_blk[Ks[s]]]['block_oracle']['recall']:.3f}"
                             if Ks[s] > 0 and matched_blk[Ks[s]] > 0 else "-" for s in DENS)
            sizes = np.array([g.size for g in qgroups])
            km_rows.append(f"| {name} (h={h}) | {sizes.min()}–{sizes.max()} ({int((sizes == 0).sum())} empty) | "
                           f"{f_tok:.3f} | {f_key:.3f} | {f_blk:.3f} | {tok} | {blk} |")
            print(f"[diagnose] {name} head {h}: {time.time() - t0:.0f} s", file=sys.stderr, flush=True)
    print("| workload (head) | grouping | selector | " + " | ".join(f"recall s={s}" for s in DENS) + " | "
          + " | ".join(f"rel L1 s={s}" for s in DENS) + " |")
    print("|---|---|---|" + "---|" * (2 * len(DENS)))
    print("\n".join(main_rows))
    print()
    print("| workload (head) | k-means query cluster sizes | inflation, tokens (queries to C) | keys to 64 "
          "| inflation, blocks | token-oracle recall at matched realised density "
          + " / ".join(f"s={s}" for s in DENS) + " | block-oracle recall at matched realised density "
          + " / ".join(f"s={s}" for s in DENS) + " |")
    print("|---|---|---|---|---|" + "---|" * 2)
    print("\n".join(km_rows))
    return 0


if __name__ == "__main__":
    sys.exit(main())
