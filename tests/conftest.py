import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU-only check")


def pytest_runtest_logreport(report):
    # Print a failure as soon as it happens, so that a run cut short by a
    # time limit still shows every failure before it.
    if report.failed:
        import sys
        sys.stdout.write(f"\n[FAILED {report.nodeid} ({report.when})]\n{report.longreprtext[-4000:]}\n")
        sys.stdout.flush()
