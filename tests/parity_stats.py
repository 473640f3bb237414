"""Collects, per GPU parity test, the largest error measured against the oracle:
the ratio to the tolerance 1e-5 * max(|y|, mag) and the plain relative error
|y - y_exact| / |y_exact| (which cancellation can make large where |y| << mag;
it is reported, the tolerance is what is asserted).  Printed by conftest at the
end of the run."""
import numpy as np

STATS = {}
CURRENT = "?"


def record(y, y64, mag, test: str | None = None):
    err = np.abs(np.asarray(y, dtype=np.float64) - y64)
    bound = 1e-5 * np.maximum(np.abs(y64), mag)
    nz = y64 != 0
    plain = float((err[nz] / np.abs(y64[nz])).max()) if nz.any() else 0.0
    ratio = float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0
    note(test or CURRENT, ratio, plain)


def note(test: str, ratio: float, plain: float):
    r0, p0 = STATS.get(test, (0.0, 0.0))
    STATS[test] = (max(r0, ratio), max(p0, plain))
