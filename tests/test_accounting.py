"""Pins of the host-side work/traffic accounting against numbers the pages print."""
import json
import os

import pytest

from token_sparse_attention_amd import accounting as acc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("row", _load("cache_transfer.json")["rows"], ids=lambda r: r["model"])
def test_cache_bytes_and_flops_reproduce_printed_values(row):
    K = acc.k_from_density(row["density"], row["N"])
    nbytes = acc.cache_bytes(row["N"], row["H"], row["D"], K, row["C"])
    flops = acc.sparse_flops(1, row["H"], row["N"], K, row["D"])
    assert round(nbytes / 2 ** 20) == row["MB"]
    assert round(flops / 1e12, 1) == row["TFLOP"]
    assert round(flops / nbytes) == row["flop_per_byte"]


def test_cache_rows_implied_rates_are_consistent():
    for row in _load("cache_transfer.json")["rows"]:
        # printed per-layer transfer rate ~53.6 GB/s and compute ~140 TFLOP/s
        gbps = row["MB"] * 2 ** 20 / (row["transfer_ms"] * 1e-3) / 1e9
        assert 53.0 < gbps < 54.0
        assert 135 < row["TFLOP"] / (row["compute_ms"] * 1e-3) < 145


@pytest.mark.parametrize("case", _load("kernel_efficiency.json")["cases"], ids=lambda c: str(c["density"]))
def test_kernel_efficiency_convention(case):
    eff = acc.kernel_efficiency(case["speedup"], case["density"])
    # the printed value is the efficiency rounded to two digits (half-up)
    assert abs(eff - case["efficiency_printed"]) <= 0.5 * 10 ** -case["digits"] + 1e-12


def test_k_from_density_for_workloads():
    assert acc.k_from_density(0.25, 1024) == 256
    assert acc.k_from_density(0.20, 32760) == 6528
    assert acc.k_from_density(0.20, 75600) == 15104
    assert acc.k_from_density(0.25, 118800) == 29696
    assert acc.k_from_density(0.15, 118800) == 17792
    assert acc.k_from_density(0.15, 49152) == 7296
    assert acc.k_from_density(0.01, 100) == 1


def test_group_counts_and_flops():
    assert acc.num_groups(75600, 128) == 591
    assert acc.num_groups(118800, 128) == 929
    assert acc.num_groups(49152, 64) == 768
    assert acc.sparse_flops(1, 40, 75600, 15104, 128) == pytest.approx(23.385e12, rel=1e-4)
    assert acc.dense_flops(1, 40, 75600, 128) == pytest.approx(117.05e12, rel=1e-4)
    assert acc.select_flops(1, 40, 75600, 128) * 2 == acc.dense_flops(1, 40, 75600, 128)
