import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# A planted mistake in the oracle (tests/oracle_mutants.py), applied before any
# test module imports the oracle; used only by tests/test_oracle_mutations.py.
if os.environ.get("MCS_ORACLE_MUTANT"):
    from tests import oracle_mutants

    oracle_mutants.apply(os.environ["MCS_ORACLE_MUTANT"])


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size parity cases")


def pytest_collection_modifyitems(config, items):
    # GPU tests cannot run where torch sees no GPU; say so instead of failing.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible to torch")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
