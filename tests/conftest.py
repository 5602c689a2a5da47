import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle.get()


def pytest_terminal_summary(terminalreporter):
    """After a GPU run: the worst (batch, head) slab error of every parity
    check, relative to its bar, largest first."""
    mod = sys.modules.get("gpu_common")
    res = getattr(mod, "RESULTS", None) if mod else None
    if not res:
        return
    tr = terminalreporter
    tr.section("parity: worst (batch, head) slab per check")
    rows = sorted(res, key=lambda r: -r[3] / r[5])
    for test, name, e, w, at, tol in rows[:40]:
        tr.write_line(f"{w:9.2e} (bar {tol:.0e}, tensor {e:9.2e})  "
                      f"{test}  {name}  slab {at}")
    if len(rows) > 40:
        tr.write_line(f"... {len(rows) - 40} more checks, all smaller")
