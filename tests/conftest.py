import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """Lists how many split rows the large sampled GPU tests compared with the oracle."""
    b = sys.modules.get("tests.bounds")
    if b is not None and b.REPORT:
        terminalreporter.section("rows checked against the oracle")
        for line in b.REPORT:
            terminalreporter.write_line(line)
