import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionfinish(session, exitstatus):
    # BDATTN_PARITY_REPORT=<file>: write the errors the GPU parity checks
    # measured (tests/parity_report.py) to that JSON file
    path = os.environ.get("BDATTN_PARITY_REPORT")
    if path:
        import parity_report
        if parity_report.RECORDS:
            parity_report.write(path)
