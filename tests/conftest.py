import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def golden_path(name):
    return os.path.join(ROOT, "tests", "golden", name)


def read_golden(name):
    """key = value lines of a fixture; '#' starts a comment."""
    out = {}
    with open(golden_path(name), encoding="utf-8") as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = line.split("=", 1)
            out[k.strip()] = v.strip()
    return out


@pytest.fixture
def golden():
    return read_golden


def pytest_terminal_summary(terminalreporter):
    try:
        import parity_log
    except ImportError:
        return
    recs = parity_log.RECORDS
    if not recs:
        return
    tr = terminalreporter
    tr.section("parity: gated error (over the magnitude before cancellation) and plain relative error over |y_ref| >= 1e-3 max")
    for r in recs:
        tr.write_line(f"{r['test']} [{r['case']}]: rows {r['rows']}, gated {r['gated_max']:.3e}, "
                      f"plain {r['plain_max']:.3e}")
    out = os.environ.get("BQD_PARITY_REPORT")
    if out:
        with open(out, "w", encoding="utf-8") as f:
            json.dump(recs, f, indent=1)
