import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def read_golden(name):
    """Parse a golden fixture: '#' comments, then 'KEY: row ; row ; ...' lines."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if ":" in line:
                k, v = line.split(":", 1)
                out[k.strip()] = [row.split() for row in v.split(";")]
            else:
                out.setdefault("_rows", []).append(line.split())
    return out


@pytest.fixture
def golden():
    return read_golden


@pytest.fixture
def progress(request):
    """Print a progress line past pytest's output capture (long oracle runs stay visible)."""
    capman = request.config.pluginmanager.getplugin("capturemanager")

    def say(msg):
        with capman.global_and_fixture_disabled():
            print(f"[progress] {msg}", file=sys.stderr, flush=True)
    return say
