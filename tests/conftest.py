import os
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

GOLDEN = Path(__file__).resolve().parent / "golden"


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size parity case (minutes of host work)")


def pytest_collection_modifyitems(config, items):
    # GPU tests cannot run without a device; the CPU suite deselects them with -m "not gpu".
    pass


@pytest.fixture(scope="session")
def golden():
    import json

    def load(name):
        with open(GOLDEN / name) as f:
            return json.load(f)
    return load
