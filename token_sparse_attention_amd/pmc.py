"""HBM traffic of the hot-path kernels from rocprofv3 counter runs.

    python -m token_sparse_attention_amd.pmc FETCH_DIR WRITE_DIR OUT.json [--workload large]
    python -m token_sparse_attention_amd.pmc --util UTIL_DIR OUT.json
    python -m token_sparse_attention_amd.pmc --l2 L2_DIR OUT.json
    python -m token_sparse_attention_amd.pmc --trace TRACE_DIR OUT.json

FETCH_DIR and WRITE_DIR are the output directories of two runs of

    rocprofv3 --pmc FETCH_SIZE -d FETCH_DIR -o pmc --output-format csv -- python3 bench.py ...
    rocprofv3 --pmc WRITE_SIZE -d WRITE_DIR -o pmc --output-format csv -- python3 bench.py ...

FETCH_SIZE / WRITE_SIZE (KiB per dispatch) do not read the same as bytes moved
on this part, so both are scaled by what they read for a plain streaming
kernel of known size measured in the same runs: residual_kernel, which reads
two bf16 tensors of B*H*N*D elements and writes one.  The result, per kernel,
is written to OUT.json together with a hash of the kernel sources, so that
bench.py reports the traffic only while the kernels are unchanged.

--util summarises one run of

    rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES SQ_BUSY_CU_CYCLES \
        SQ_ACTIVE_INST_VALU SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS \
        GRBM_GUI_ACTIVE -d UTIL_DIR -o pmc --output-format csv -- python3 bench.py ...

per kernel: the average shader clock over the dispatch (GRBM_GUI_ACTIVE, summed
over the 8 XCDs, divided by the dispatch time), the share of SIMD cycles in
which the MFMA unit was busy, the share in which a plain VALU instruction
issued while it was (co-execution), the share of SIMD cycles with a VALU
instruction (MFMA included) executing (SQ_ACTIVE_INST_VALU counts quad-cycles
per wave), and the VALU (MFMA excluded) and LDS instructions per MFMA.

--l2 summarises one run of

    rocprofv3 --pmc TCC_HIT_sum TCC_MISS_sum -d L2_DIR -o pmc --output-format csv -- python3 bench.py ...

per kernel: L2 hits and misses per dispatch and the hit rate (a miss is a
128-byte line requested from the fabric: MALL or HBM).

--trace summarises the kernel_trace.csv of one

    rocprofv3 --kernel-trace --stats -d TRACE_DIR -o bench --output-format csv -- python3 bench.py ...

per kernel: calls, mean / min / max dispatch time and share of the GPU time.

In all four, attention dispatches issued after the first block_means_kernel
(bench.py's block-sparse comparison, the same kernel over whole key blocks)
are reported under the kernel's name with " [block-sparse]" appended.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))


def _code_only(text: str) -> str:
    """Source text without comments and with whitespace collapsed (the code)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


# the files the attention kernels are built from
ATTN_SOURCES = ("attn.hip", "mcs_common.h", "mcs_internal.h")


def source_hash(files=None) -> str:
    """Hash of the code of the HIP sources the counters describe, all of them
    or the named files (comments and whitespace do not count, so editing a
    comment keeps the counters valid)."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(PKG, "csrc", "*"))):
        if files is not None and os.path.basename(f) not in files:
            continue
        with open(f, encoding="utf-8") as fh:
            h.update(os.path.basename(f).encode())
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


BSA_MARK = "block_means_kernel"   # bench.py's block-sparse comparison starts with it
BSA_SUFFIX = " [block-sparse]"


def _rows(directory: str, kind: str = "counter_collection"):
    """Counter rows of a run with the short kernel name; attention dispatches
    issued after the block-sparse comparison began (the same kernel over the
    blocks' tokens) are named apart, so the token-sparse figures hold only the
    token-sparse launches."""
    rows = []
    for f in glob.glob(os.path.join(directory, "**", f"*{kind}.csv"), recursive=True):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    names = [r["Kernel_Name"].split("(")[0].replace("void ", "").replace("mcs::", "") for r in rows]
    marks = [int(r["Dispatch_Id"]) for r, n in zip(rows, names) if n.startswith(BSA_MARK)]
    start = min(marks) if marks else None
    for r, n in zip(rows, names):
        if start is not None and n.startswith("attn_kernel") and int(r["Dispatch_Id"]) > start:
            n += BSA_SUFFIX
        yield n, r


def _per_kernel(directory: str, counter: str) -> dict:
    vals = defaultdict(lambda: defaultdict(float))
    for name, r in _rows(directory):
        if r["Counter_Name"] == counter:
            vals[name][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: sum(d.values()) / len(d) for k, d in vals.items() if d}


def summarize(fetch_dir: str, write_dir: str, workload: str) -> dict:
    from token_sparse_attention_amd import synth
    w = synth.WORKLOADS[workload]
    tensor_bytes = w.B * w.H * w.N * w.D * 2
    fetch = _per_kernel(fetch_dir, "FETCH_SIZE")
    write = _per_kernel(write_dir, "WRITE_SIZE")
    cal = "residual_kernel"
    f_read = (2 * tensor_bytes) / (fetch[cal] * 1024.0)
    f_write = tensor_bytes / (write[cal] * 1024.0)
    kernels = {}
    for k in sorted(set(fetch) | set(write)):
        rd = fetch.get(k, 0.0) * 1024.0 * f_read
        wr = write.get(k, 0.0) * 1024.0 * f_write
        kernels[k] = {"fetch_kib_raw": fetch.get(k), "write_kib_raw": write.get(k),
                      "read_bytes": rd, "write_bytes": wr, "traffic_bytes": rd + wr}
    return {"workload": workload, "calibration_kernel": cal, "read_scale": f_read,
            "write_scale": f_write, "source_hash": source_hash(),
            "attn_source_hash": source_hash(ATTN_SOURCES), "kernels": kernels}


N_XCD = 8
N_SIMD = 256 * 4


def utilisation(util_dir: str) -> dict:
    rows = defaultdict(lambda: defaultdict(float))
    times = defaultdict(dict)
    for name, r in _rows(util_dir):
        d = r["Dispatch_Id"]
        rows[(name, d)][r["Counter_Name"]] += float(r["Counter_Value"])
        times[(name, d)] = (int(r["Start_Timestamp"]), int(r["End_Timestamp"]))
    acc = defaultdict(lambda: defaultdict(float))
    for (name, d), c in rows.items():
        t0, t1 = times[(name, d)]
        dt = (t1 - t0) * 1e-9
        cyc = c.get("GRBM_GUI_ACTIVE", 0.0) / N_XCD
        if dt <= 0 or cyc <= 0:
            continue
        a = acc[name]
        a["n"] += 1
        a["ms"] += dt * 1e3
        a["clock_ghz"] += cyc / dt / 1e9
        a["mfma_busy"] += c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (N_SIMD * cyc)
        a["coexec"] += c.get("SQ_VALU_MFMA_COEXEC_CYCLES", 0.0) / (N_SIMD * cyc)
        a["cu_busy"] += c.get("SQ_BUSY_CU_CYCLES", 0.0) * 4 / (256 * cyc)
        if "SQ_ACTIVE_INST_VALU" in c:
            a["valu_active"] += c["SQ_ACTIVE_INST_VALU"] * 4 / (N_SIMD * cyc)
        mf = c.get("SQ_INSTS_MFMA", 0.0)
        if mf > 0:
            a["valu_per_mfma"] += (c.get("SQ_INSTS_VALU", 0.0) - mf) / mf
            a["lds_per_mfma"] += c.get("SQ_INSTS_LDS", 0.0) / mf
    out = {}
    for name, a in acc.items():
        n = a.pop("n")
        out[name] = {k: v / n for k, v in a.items()}
        out[name]["dispatches"] = int(n)
    return {"source_hash": source_hash(),
            "attn_source_hash": source_hash(ATTN_SOURCES), "kernels": out}


def l2(l2_dir: str) -> dict:
    hits = _per_kernel(l2_dir, "TCC_HIT_sum")
    miss = _per_kernel(l2_dir, "TCC_MISS_sum")
    out = {}
    for k in sorted(set(hits) & set(miss)):
        tot = hits[k] + miss[k]
        out[k] = {"hits": hits[k], "misses": miss[k], "hit_rate": hits[k] / tot if tot else None,
                  "miss_bytes": 128.0 * miss[k]}
    return {"source_hash": source_hash(),
            "attn_source_hash": source_hash(ATTN_SOURCES), "kernels": out}


def trace(trace_dir: str) -> dict:
    """Per kernel: calls, mean / min / max dispatch time (ms) and share of the
    GPU time, from a --kernel-trace run (block-sparse launches apart)."""
    ms = defaultdict(list)
    for name, r in _rows(trace_dir, "kernel_trace"):
        ms[name].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-6)
    total = sum(sum(v) for v in ms.values())
    out = {k: {"calls": len(v), "mean_ms": sum(v) / len(v), "min_ms": min(v), "max_ms": max(v),
               "share": sum(v) / total} for k, v in ms.items()}
    return {"source_hash": source_hash(), "attn_source_hash": source_hash(ATTN_SOURCES),
            "kernels": dict(sorted(out.items(), key=lambda kv: -kv[1]["share"]))}


def main(argv):
    if argv and argv[0] == "--l2":
        out = l2(argv[1])
        with open(argv[2], "w") as f:
            json.dump(out, f, indent=1)
        for k, v in sorted(out["kernels"].items(), key=lambda kv: -kv[1]["misses"]):
            print(f"{k:48s} hit rate {100 * (v['hit_rate'] or 0):5.1f}%  misses {v['misses']:.3e}"
                  f"  ({v['miss_bytes'] / 1e9:.2f} GB of lines)")
        return 0
    if argv and argv[0] == "--trace":
        out = trace(argv[1])
        with open(argv[2], "w") as f:
            json.dump(out, f, indent=1)
        for k, v in out["kernels"].items():
            print(f"| `{k}` | {v['calls']} | {v['mean_ms']:.3f} | {v['min_ms']:.3f} | {v['max_ms']:.3f}"
                  f" | {100 * v['share']:.2f} |")
        return 0
    if argv and argv[0] == "--util":
        out = utilisation(argv[1])
        with open(argv[2], "w") as f:
            json.dump(out, f, indent=1)
        for k, v in sorted(out["kernels"].items(), key=lambda kv: -kv[1]["ms"]):
            print(f"{k:48s} {v['ms']:9.3f} ms  clock {v['clock_ghz']:.3f} GHz  MFMA busy {100 * v['mfma_busy']:5.1f}%"
                  f"  co-exec {100 * v['coexec']:5.1f}%  VALU active {100 * v.get('valu_active', 0):5.1f}%")
        return 0
    if len(argv) < 3:
        print(__doc__)
        return 2
    workload = "large"
    if "--workload" in argv:
        workload = argv[argv.index("--workload") + 1]
    out = summarize(argv[0], argv[1], workload)
    with open(argv[2], "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps({k: round(v["traffic_bytes"] / 1e9, 3) for k, v in out["kernels"].items()}, indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
