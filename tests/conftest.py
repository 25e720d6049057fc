import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP library on cuda:0)")


@pytest.fixture(scope="session")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def pytest_terminal_summary(terminalreporter):
    """Every oracle comparison of the session: pairs compared and the worst error over
    the tolerance, for the outputs and the final state."""
    mod = sys.modules.get("tests.gpu_helpers")
    rows = getattr(mod, "RESULTS", None) if mod else None
    if not rows:
        return
    tr = terminalreporter
    tr.write_sep("-", f"oracle comparisons: worst err/tol over the compared (sequence, head) pairs ({len(rows)})")
    for what, pairs, eo, es in rows:
        st = "   -  " if es is None else f"{es:6.3f}"
        tr.write_line(f"  o {eo:6.3f}  state {st}  pairs {pairs:5d}  {what}")
