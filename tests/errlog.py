"""Measured errors of the GPU parity tests, printed at the end of the run.

Each parity check records (case, measured error, bar it was held to); the
pytest terminal summary lists them, so a run's log keeps every value and not
only pass/fail."""
from __future__ import annotations

RECORDS = []


def record(case: str, err: float, bar: float) -> None:
    RECORDS.append((case, float(err), float(bar)))
