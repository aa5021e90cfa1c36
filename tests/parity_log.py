"""Parity figures gathered while the tests run, printed at the end of the
session (and written as JSON to $BQD_PARITY_REPORT when that is set).

Each record holds the gated error of the pages' reading (|y - y_ref| over
the row's magnitude before cancellation, the 1e-5 gate) beside the plain
relative error |y - y_ref| / |y_ref| over the rows with |y_ref| at least
1e-3 of the largest |y_ref|."""
import os

import numpy as np

import oracle as O

RECORDS = []


def record(test, label, gated, plain, rows):
    RECORDS.append({"test": test, "case": label, "gated_max": float(gated), "plain_max": float(plain),
                    "rows": int(rows)})


def check_rowwise(label, y, y_ref, sw, sx, acc, bias, tol):
    """Assert the gated error and record it with the plain one, under the
    running test's name."""
    gated = O.rel_err_rowwise(y, y_ref, sw, sx, acc, bias).max(initial=0.0)
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    record(test, str(label), gated, O.rel_err_plain(y, y_ref), np.size(y_ref))
    assert gated <= tol, (label, gated)
    return gated
