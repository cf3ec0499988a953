import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def pytest_runtest_setup(item):
    # Name the case before any GPU work so that a crash still says which test ran.
    if item.get_closest_marker("gpu") is not None:
        print(f"\n[gpu-case] {item.nodeid}", flush=True)
