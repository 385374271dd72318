import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """Parity errors of the GPU tests vs the float64 oracle, per test and output type:
    elements compared, max absolute error, max error in ulps of the output type."""
    mod = sys.modules.get("gpu_util")
    rows = getattr(mod, "REPORT", None) if mod else None
    if not rows:
        return
    agg = {}
    for test, dtype, n, err, ulps, kerr, exact in rows:
        a = agg.setdefault((test, dtype), [0, 0.0, 0.0, 0.0, 0.0])
        a[0] += n
        a[1], a[2], a[3] = max(a[1], err), max(a[2], ulps), max(a[3], kerr)
        a[4] += exact * n
    tr = terminalreporter
    tr.section("parity errors vs the float64 oracle")
    tr.write_line("elements: outputs compared; max abs: |gpu - oracle|; max ulp: in output ulps; "
                  "kernel err: distance from the oracle to the reals that round to the gpu "
                  "output; =RNE: share of outputs equal to the oracle rounded to nearest even")
    tr.write_line(f"{'test':60s} {'dtype':5s} {'elements':>10s} {'max abs':>9s} {'max ulp':>8s} "
                  f"{'kernel err':>10s} {'=RNE':>7s}")
    for (test, dtype), (n, err, ulps, kerr, exact) in agg.items():
        name = test.split("::", 1)[-1]
        tr.write_line(f"{name[:60]:60s} {dtype:5s} {n:10d} {err:9.3g} {ulps:8.1f} {kerr:10.3g} "
                      f"{exact / max(n, 1):7.4f}")
