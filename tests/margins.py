"""Worst parity margins seen by the GPU tests, reported at the end of the run.

Every element-wise comparison against the oracle records its max|GPU - oracle| /
RMS(oracle) here under the running test's name; the conftest prints the worst
value per test in pytest's terminal summary (shown also with -q) and writes them
to gpu_margins.json in the run-output folder, so a margin creeping toward the
2e-3 bound is visible in every run, not only when a test fails.
"""
from __future__ import annotations

import os

_worst: dict = {}


def current_test() -> str:
    return os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]


def record(what: str, err: float):
    key = current_test()
    prev = _worst.get(key)
    if prev is None or err > prev[1]:
        _worst[key] = (what, float(err))


def table():
    return dict(sorted(_worst.items()))
