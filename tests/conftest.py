"""Shared pytest setup: the `gpu` marker and repository import path."""

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads (minutes on the CPU side)")


def pytest_sessionfinish(session, exitstatus):
    """Writes the comparison statistics (tests/support.py REPORT) as JSON when
    MONO_PARITY_REPORT names a file."""
    path = os.environ.get("MONO_PARITY_REPORT")
    sup = sys.modules.get("support")
    if path and sup is not None and sup.REPORT:
        sup.write_report(path)
