import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """The strict relative figure of every parity comparison that ran: its
    distribution and the worst cases (the bar itself is the tolerance)."""
    mod = sys.modules.get("tests.parity")
    rows = getattr(mod, "STRICT", None) if mod else None
    if not rows:
        return
    import numpy as np
    vals = np.array([r[1] for r in rows])
    tr = terminalreporter
    tr.section("parity: strict relative figure, max |gpu - oracle| / max |oracle row|")
    tr.write_line(f"{len(rows)} comparisons over {sum(r[2] for r in rows)} rows: median {np.median(vals):.3g}, "
                  f"p90 {np.percentile(vals, 90):.3g}, max {vals.max():.3g} (tolerance 1e-2 of the row's max + 1e-3)")
    for what, v, n in sorted(rows, key=lambda r: -r[1])[:10]:
        tr.write_line(f"  {v:.3g}  {what} ({n} rows)")
