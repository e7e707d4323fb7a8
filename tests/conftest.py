import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Print the parity margins (err/tol per output) that the GPU tests recorded."""
    import margins
    lines = margins.summary_lines()
    if not lines:
        return
    terminalreporter.write_sep("-", "parity margins: max|gpu - oracle| / tol (pass <= 1)")
    for line in lines:
        terminalreporter.write_line(line)
    out = os.path.join(ROOT, "gpurun_out")
    if os.path.isdir(out):
        try:
            with open(os.path.join(out, "parity_margins.json"), "w") as f:
                json.dump(margins.RECORDS, f, indent=1)
        except OSError:
            pass
