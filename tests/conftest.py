import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path through the C-ABI")


def golden_path(name: str) -> str:
    return os.path.join(ROOT, "tests", "golden", name)


def read_golden(name: str):
    """key = value lines; repeated keys collect into lists."""
    out = {}
    with open(golden_path(name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = (s.strip() for s in line.split("=", 1))
            out.setdefault(k, []).append(v)
    return out


@pytest.fixture(scope="session")
def oracle_lib():
    from oracle import build
    build.build()
    from oracle import ref
    return ref
