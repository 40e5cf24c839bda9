"""Recall and output error of the pages' diagnostic selectors on synthetic heads.

    python -m oracle.diagnose [--workloads tiny small asset3d] [--heads 1]

Test-infrastructure script (it uses only ``oracle`` and the seeded input
generators): for one or more heads of each workload, every selector of
``oracle.diagnostics`` at densities 0.1, 0.2 and 0.3 (K = 128*floor(s*N/128)),
with query blocks of C consecutive queries and with PDDP groups.  Prints a
markdown table ("-" where the budget is below one 128-key step).
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


def _cell(res, gname, s, sel, key):
    r = res.get((gname, s))
    return f"{r[sel][key]:.3f}" if r is not None else "-"


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workloads", nargs="+", default=["tiny", "small", "asset3d"])
    ap.add_argument("--heads", type=int, default=1)
    args = ap.parse_args(argv)
    dens = (0.1, 0.2, 0.3)
    print("| workload (head) | grouping | selector | " + " | ".join(f"recall s={s}" for s in dens) + " | "
          + " | ".join(f"rel L1 s={s}" for s in dens) + " |")
    print("|---|---|---|" + "---|" * (2 * len(dens)))
    for name in args.workloads:
        w = synth.WORKLOADS[name]
        heads = [(0, h) for h in range(min(args.heads, w.H))]
        x = synth.generate(name, heads=heads)
        scale = 1.0 / math.sqrt(w.D)
        for i, (b, h) in enumerate(heads):
            q, k, v = (synth.to_f64(x[t][0, i]) for t in "qkv")
            t0 = time.time()
            groupings = {"contiguous": np.arange(w.N), "PDDP": oracle.pddp(q, w.C)}
            res = {}
            for gname, perm in groupings.items():
                for s in dens:
                    K = 128 * int(s * w.N // 128)
                    if K > 0:       # no budget below one 128-key step
                        res[(gname, s)] = dg.diagnose_head(q, k, v, perm, w.C, K, scale)
            for gname in groupings:
                for sel in dg.SELECTORS:
                    rec = " | ".join(_cell(res, gname, s, sel, "recall") for s in dens)
                    err = " | ".join(_cell(res, gname, s, sel, "rel_l1") for s in dens)
                    print(f"| {name} (h={h}) | {gname} | {LABELS[sel]} | {rec} | {err} |", flush=True)
            print(f"[diagnose] {name} head {h}: {time.time() - t0:.0f} s", file=sys.stderr, flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
