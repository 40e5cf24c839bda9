"""The rocprofv3 counter summaries behind bench.py's roofline.traffic, on
synthetic counter files: calibration by the residual kernel, and attention
dispatches of the block-sparse comparison kept apart from the token-sparse
ones."""
import csv
import os

import pytest

from token_sparse_attention_amd import pmc, synth

COLS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
ATTN = "void mcs::attn_kernel<128, 4, true, true, false, false>(mcs::AttnParams)"


def _write(directory, name, rows, cols=COLS):
    os.makedirs(directory, exist_ok=True)
    with open(os.path.join(directory, name), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(cols, r)))


def _run(tmp_path, counter, resid_kib, attn_kibs, bsa_kibs):
    """Dispatch order of one bench step: residual, token-sparse attention,
    then the block-sparse comparison (block means, its attention launches)."""
    rows = [(1, "void mcs::residual_kernel(...)", counter, resid_kib, 0, 10)]
    d = 2
    for v in attn_kibs:
        rows.append((d, ATTN, counter, v, 0, 10))
        d += 1
    rows.append((d, "void mcs::block_means_kernel<128>(...)", counter, 1.0, 0, 10))
    d += 1
    for v in bsa_kibs:
        rows.append((d, ATTN, counter, v, 0, 10))
        d += 1
    out = tmp_path / counter
    _write(str(out), "pmc_counter_collection.csv", rows)
    return str(out)


def test_traffic_calibrated_and_block_sparse_apart(tmp_path):
    w = synth.WORKLOADS["large"]
    tensor = w.B * w.H * w.N * w.D * 2
    # the counters read half the true bytes for reads, exactly for writes
    fdir = _run(tmp_path, "FETCH_SIZE", tensor / 1024.0, [100.0, 300.0], [1000.0, 1000.0])
    wdir = _run(tmp_path, "WRITE_SIZE", tensor / 1024.0, [10.0, 10.0], [20.0, 20.0])
    out = pmc.summarize(fdir, wdir, "large")
    assert out["read_scale"] == pytest.approx(2.0)
    assert out["write_scale"] == pytest.approx(1.0)
    k = out["kernels"]
    tok = k["attn_kernel<128, 4, true, true, false, false>"]
    assert tok["read_bytes"] == pytest.approx(2.0 * 200.0 * 1024)      # mean of the two, scaled
    assert tok["write_bytes"] == pytest.approx(10.0 * 1024)
    bsa = k["attn_kernel<128, 4, true, true, false, false>" + pmc.BSA_SUFFIX]
    assert bsa["read_bytes"] == pytest.approx(2.0 * 1000.0 * 1024)
    assert k["residual_kernel"]["traffic_bytes"] == pytest.approx(3.0 * tensor)


def test_no_block_sparse_mark_keeps_all_dispatches(tmp_path):
    rows = [(1, ATTN, "TCC_HIT_sum", 30.0, 0, 10), (1, ATTN, "TCC_MISS_sum", 10.0, 0, 10),
            (2, ATTN, "TCC_HIT_sum", 10.0, 0, 10), (2, ATTN, "TCC_MISS_sum", 10.0, 0, 10)]
    _write(str(tmp_path / "l2"), "pmc_counter_collection.csv", rows)
    k = pmc.l2(str(tmp_path / "l2"))["kernels"]
    assert list(k) == ["attn_kernel<128, 4, true, true, false, false>"]
    v = k["attn_kernel<128, 4, true, true, false, false>"]
    assert v["hit_rate"] == pytest.approx(20.0 / 30.0)
    assert v["miss_bytes"] == pytest.approx(128.0 * 10.0)


def test_trace_summary(tmp_path):
    cols = ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    rows = [(1, ATTN, 0, 2_000_000), (2, ATTN, 0, 4_000_000),
            (3, "void mcs::block_means_kernel<128>(...)", 0, 1_000_000),
            (4, ATTN, 0, 3_000_000)]
    _write(str(tmp_path / "t"), "bench_kernel_trace.csv", rows, cols)
    k = pmc.trace(str(tmp_path / "t"))["kernels"]
    tok = k["attn_kernel<128, 4, true, true, false, false>"]
    assert tok["calls"] == 2 and tok["mean_ms"] == pytest.approx(3.0)
    assert tok["min_ms"] == pytest.approx(2.0) and tok["max_ms"] == pytest.approx(4.0)
    assert tok["share"] == pytest.approx(6.0 / 10.0)
    assert k["attn_kernel<128, 4, true, true, false, false>" + pmc.BSA_SUFFIX]["calls"] == 1
