import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """Print the full-tensor errors against the oracle that the parity tests recorded."""
    mod = sys.modules.get("tests._parity")
    lines = getattr(mod, "REPORT", None)
    if lines:
        terminalreporter.section("errors against the fp64 oracle (full tensors)")
        for line in lines:
            terminalreporter.write_line(line)
