import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    import parity_log

    if parity_log.LINES:
        terminalreporter.write_sep("-", "headline parity errors (GPU vs the fp64 oracle)")
        for line in parity_log.LINES:
            terminalreporter.write_line(line)
