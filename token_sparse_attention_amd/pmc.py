"""HBM traffic of the hot-path kernels from rocprofv3 counter runs.

    python -m token_sparse_attention_amd.pmc FETCH_DIR WRITE_DIR OUT.json [--workload large]

FETCH_DIR and WRITE_DIR are the output directories of two runs of

    rocprofv3 --pmc FETCH_SIZE -d FETCH_DIR -o pmc --output-format csv -- python3 bench.py ...
    rocprofv3 --pmc WRITE_SIZE -d WRITE_DIR -o pmc --output-format csv -- python3 bench.py ...

FETCH_SIZE / WRITE_SIZE (KiB per dispatch) do not read the same as bytes moved
on this part, so both are scaled by what they read for a plain streaming
kernel of known size measured in the same runs: residual_kernel, which reads
two bf16 tensors of B*H*N*D elements and writes one.  The result, per kernel,
is written to OUT.json together with a hash of the kernel sources, so that
bench.py reports the traffic only while the kernels are unchanged.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))


def source_hash() -> str:
    """Hash of the HIP sources the counters describe."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(PKG, "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def _per_kernel(directory: str, counter: str) -> dict:
    vals = defaultdict(lambda: defaultdict(float))
    for f in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                name = r["Kernel_Name"].split("(")[0].replace("void ", "").replace("mcs::", "")
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
            "write_scale": f_write, "source_hash": source_hash(), "kernels": kernels}


def main(argv):
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
