"""Turns the parity log of a GPU test run into a markdown table.

    GDN_PARITY_LOG=/tmp/parity.jsonl python -m pytest tests -m gpu ...
    python tests/parity_report.py /tmp/parity.jsonl "<the test command>" > profiles/parity.md

Each line of the log is one comparison made by tests/helpers.assert_close:
the test id, the tensor, max|got - ref| / max|ref| and the tolerance.  The
table lists them per test with the margin (tolerance / error)."""
from __future__ import annotations

import json
import sys


def main(path: str, cmd: str = "") -> None:
    rows = [json.loads(line) for line in open(path) if line.strip()]
    print("# Parity margins of the GPU tests")
    print()
    print("max|GPU - reference| / max|reference| per output tensor, from the GPU run's own")
    print("log (`GDN_PARITY_LOG`); the reference is the fp64 oracle unless the tensor name says")
    print("otherwise (`vs unsplit`: the same batch run unsplit on the GPU). Tolerances: 2e-2")
    print("bfloat16, 1e-4 float32.")
    if cmd:
        print()
        print("Command: `%s`" % cmd)
    print()
    print("| test | tensor | rel err | tol | margin |")
    print("|---|---|---|---|---|")
    worst = 0.0
    for r in rows:
        margin = r["tol"] / r["rel_err"] if r["rel_err"] > 0 else float("inf")
        worst = max(worst, r["rel_err"] / r["tol"])
        print("| %s | %s | %.2e | %.0e | %s |" % (r["test"].replace("tests/", ""), r["tensor"],
                                                r["rel_err"], r["tol"],
                                                "inf" if margin == float("inf") else "%.0fx" % margin))
    print()
    print("%d comparisons; the largest error is %.1f%% of its tolerance." % (len(rows), 100 * worst))


if __name__ == "__main__":
    main(sys.argv[1], " ".join(sys.argv[2:]))
