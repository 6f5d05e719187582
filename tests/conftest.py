import sys
from pathlib import Path

ROOT = Path(__file__).resolve().parents[1]
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))
TESTS = Path(__file__).resolve().parent
if str(TESTS) not in sys.path:
    sys.path.insert(0, str(TESTS))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def pytest_terminal_summary(terminalreporter):
    """After a GPU session: how many bf16 elements of each judged output passed
    only through the cancellation rule (a correct fp32 sum that rounds more
    than one bf16 ulp from the oracle's rounding, next to a near-zero
    result), and the largest distance seen."""
    gu = sys.modules.get("gpu_util")
    rows = getattr(gu, "CANCEL_REPORT", None) if gu else None
    if not rows:
        return
    tr = terminalreporter
    tr.section("bf16 cancellation rule")
    elements = sum(r[1] for r in rows)
    rescued = sum(r[2] for r in rows)
    tr.write_line(f"{len(rows)} outputs judged, {elements:,} bf16 elements, "
                  f"{rescued} passed through the cancellation rule")
    for what, n, k, ulp in rows:
        if k:
            tr.write_line(f"  {what}: {k} of {n:,} (max distance {ulp} ulp)")
