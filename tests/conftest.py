import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long CPU statistics; run with FS_SLOW=1")


def pytest_collection_modifyitems(config, items):
    if os.environ.get("FS_SLOW") == "1":
        return
    skip = pytest.mark.skip(reason="slow CPU statistics; set FS_SLOW=1 to run")
    for item in items:
        if "slow" in item.keywords:
            item.add_marker(skip)


def read_golden(name):
    """Parse a whitespace table under tests/golden, skipping '#' comment lines."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line.split())
    return rows


@pytest.fixture(scope="session")
def golden():
    return read_golden
