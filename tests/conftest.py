import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a gfx950 GPU and the built libsvq")


def load_golden(name):
    """Parse a tests/golden/*.txt fixture: '# comments', then 'key values...'."""
    path = os.path.join(ROOT, "tests", "golden", name)
    out = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out.setdefault(key, []).append(vals)
    return out


@pytest.fixture
def golden():
    return load_golden
