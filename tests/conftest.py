import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP library)")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Every use of the conditioning criterion of the floating-point parity checks, listed where a quiet run
    still shows it."""
    try:
        import parity_log
    except ImportError:
        return
    uses = parity_log.USES
    if not uses:
        terminalreporter.write_line("[conditioning] 0 tensors needed the one-ulp perturbation criterion")
        return
    terminalreporter.write_line(f"[conditioning] {len(uses)} tensors passed only through the one-ulp "
                                f"perturbation criterion (ratio = largest error / largest one-ulp response):")
    for u in uses:
        terminalreporter.write_line("  " + u)
