import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name):
    """Parse a tests/golden/*.txt fixture: '# ...' comments; 'key values...'
    lines; 'row i : cols...' lines."""
    data = {"rows": {}}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("row "):
                head, cols = line.split(":")
                data["rows"][int(head.split()[1])] = [int(c) for c in cols.split()]
                continue
            key, *vals = line.split()
            data[key] = vals
    return data


@pytest.fixture
def golden():
    return read_golden
