import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running (full-size workloads)")


@pytest.fixture(scope="session")
def c_oracle():
    from oracle import c_oracle as co
    co.lib()
    return co


@pytest.fixture(scope="session")
def np_oracle():
    from oracle import kda_ref
    return kda_ref


def pytest_sessionfinish(session, exitstatus):
    """With KDA_PARITY_RECORD set to a path, write every parity figure the GPU
    tests reported (rel-L2, largest per-block rel-L2, max-abs, RMS of the
    oracle's result, per test and output) there as JSON."""
    path = os.environ.get("KDA_PARITY_RECORD")
    if not path:
        return
    lib = sys.modules.get("tests.kda_testlib")
    records = list(getattr(lib, "RECORDS", [])) if lib is not None else []
    import json
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        json.dump({"exitstatus": int(exitstatus), "records": records}, f, indent=1)
