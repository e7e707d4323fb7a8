"""Err/tol margins of the GPU parity checks, collected so that a quiet (-q) test
run still prints them: tests/conftest.py writes one line per test at the end of
the session, and the same records as JSON into the run's output folder when one
exists.

A margin is max|gpu - oracle| / (1e-2 max|oracle| + 1e-3) for one output; it
must be at most 1.  Rounding the bf16 intermediates alone costs 0.12-0.24 of it
on the benchmark shapes, so values well above 0.3 point at a bug rather than at
rounding."""
import os
from collections import OrderedDict

RECORDS = OrderedDict()  # test id -> OrderedDict(output name -> ratio)


def _test_id() -> str:
    cur = os.environ.get("PYTEST_CURRENT_TEST", "?")
    return cur.split("::", 1)[-1].rsplit(" ", 1)[0]


def record(name: str, ratio: float) -> None:
    RECORDS.setdefault(_test_id(), OrderedDict())[name] = float(ratio)


def summary_lines(detail_prefixes=("test_config",)):
    """One line per test: its worst output, and every output for the benchmark
    configurations."""
    lines = []
    worst = (0.0, "", "")
    for test, outs in RECORDS.items():
        name, r = max(outs.items(), key=lambda kv: kv[1])
        if r > worst[0]:
            worst = (r, test, name)
        if test.startswith(detail_prefixes):
            lines.append(f"{test}: " + " ".join(f"{k}={v:.3f}" for k, v in outs.items()))
        else:
            lines.append(f"{test}: max {r:.3f} ({name}) over {len(outs)} outputs")
    if RECORDS:
        lines.append(f"worst margin {worst[0]:.3f}: {worst[1]} {worst[2]}")
    return lines
