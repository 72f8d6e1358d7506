import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload, minutes of CPU oracle time")


def pytest_terminal_summary(terminalreporter):
    """Totals of the draft-token rows whose oracle top-2 gap fell between 1e-2
    and twice the measured logit error (see pe_gpu.assert_tokens_logits)."""
    mod = sys.modules.get("pe_gpu")
    if mod is not None and mod.BAND["rows"]:
        terminalreporter.write_line(
            f"draft rows with 1e-2 < top-2 gap <= 2 x logit error: {mod.BAND['rows']}, "
            f"of which {mod.BAND['differ']} drafted another near-maximal token")
