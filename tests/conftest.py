import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP library through its C ABI)")
    config.addinivalue_line("markers", "slow: long CPU test")


TIE_CLASSES = ("argmax_gap", "gumbel_key_gap", "budget", "mean_entropy", "accept_cut", "allowed_argmax",
               "tiny_loop_divergence", "serving_divergence", "lmhead_argmax_gap", "lmhead_key_gap")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Near-ties counted by the parity tests, by class (zeros included): outputs allowed to differ
    from the oracle because the deciding values lie within the stated tie bands."""
    from tests import parity
    counts = dict.fromkeys(TIE_CLASSES, 0)
    counts.update(parity.NEAR_TIES)
    terminalreporter.write_sep("-", "near-ties (counted, not failed)")
    terminalreporter.write_line("  ".join(f"{k}={v}" for k, v in counts.items()))
