import json
import os
import sys
import time

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# GPU parity cases append one JSON line each here (flips, flip margins, free-run
# mismatches, clamped entries, proxy-loss agreement); tests/parity_report.py turns
# the file into a per-workload table. Override with BAKRON_PARITY_LOG.
PARITY_LOG = os.environ.get("BAKRON_PARITY_LOG", os.path.join(ROOT, "gpurun_out", "parity_records.jsonl"))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    return oracle


def record_parity(case: str, **fields):
    """Append one parity record (a JSON line) for the case; never fails the test."""
    rec = {"case": case, "time": time.strftime("%Y-%m-%dT%H:%M:%S")}
    for k, v in fields.items():
        if hasattr(v, "item"):
            v = v.item()
        rec[k] = v
    try:
        os.makedirs(os.path.dirname(PARITY_LOG), exist_ok=True)
        with open(PARITY_LOG, "a") as f:
            f.write(json.dumps(rec) + "\n")
    except OSError:
        pass
