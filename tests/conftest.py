import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP C-ABI library)")


GOLDEN = os.path.join(ROOT, "tests", "golden")


@pytest.fixture
def golden():
    import json

    def load(name):
        with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
            return json.load(f)

    return load
