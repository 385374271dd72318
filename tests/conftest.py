import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """Parity errors of the GPU tests, absolute and in ulps of the output type."""
    mod = sys.modules.get("gpu_util") or sys.modules.get("tests.gpu_util")
    rows = getattr(mod, "REPORT", None) if mod else None
    if not rows:
        return
    tr = terminalreporter
    tr.section("parity errors vs the float64 oracle")
    tr.write_line(f"{'check':60s} {'dtype':5s} {'elements':>10s} {'max abs':>10s} {'max ulp':>8s}")
    for what, dtype, n, err, ulps in rows:
        tr.write_line(f"{(what or '-')[:60]:60s} {dtype:5s} {n:10d} {err:10.3g} {ulps:8.2f}")
    worst = {}
    for what, dtype, n, err, ulps in rows:
        w = worst.setdefault(dtype, [0.0, 0.0])
        w[0], w[1] = max(w[0], err), max(w[1], ulps)
    for dtype, (err, ulps) in sorted(worst.items()):
        tr.write_line(f"worst {dtype}: max abs {err:.3g}, {ulps:.2f} ulp of the output type")
