"""Shared pytest configuration: the ``gpu`` marker and library fixtures."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; run with -m gpu")


@pytest.fixture(scope="session")
def orc():
    """The fp64 oracle, compiled from oracle/oracle.c if not built yet."""
    import oracle
    return oracle.default()


@pytest.fixture(scope="session")
def golden():
    import json
    with open(os.path.join(ROOT, "tests", "golden", "page_cases.json")) as f:
        return json.load(f)
