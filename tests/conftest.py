import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """One JSON line per checked parity comparison (rows, oracle-flagged near
    ties, rows where the GPU took a listed alternative, mismatches)."""
    import json
    import sys
    mod = sys.modules.get("tests.parity")
    recs = getattr(mod, "RECORDS", None) if mod is not None else None
    if not recs:
        return
    terminalreporter.write_sep("-", f"parity records ({len(recs)})")
    for r in recs:
        terminalreporter.write_line("[parity-record] " + json.dumps(r))
