import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """List the near-tie tokens each GPU parity case met (tokens whose oracle k-th/(k+1)-th
    score gap, or group gap, is below the tie threshold), so that they are reported even when
    the run is quiet."""
    mc = sys.modules.get("moe_case")
    ties = getattr(mc, "NEAR_TIES", None) if mc is not None else None
    if not ties:
        return
    tr = terminalreporter
    tr.write_sep("-", f"near-tie tokens (oracle score gap below {mc.TIE_GAP:g})")
    for label in sorted(ties):
        n, differ, T = ties[label]
        tr.write_line(f"{label}: {n} of {T} tokens near a tie, {differ} with a different expert set")
