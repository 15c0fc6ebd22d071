"""Summarise the GPU parity records as a markdown table.

The GPU tests append one JSON line per solve case to the parity log (see
tests/conftest.py). This script groups them by case and prints, per case: the
shape, the quantiser, how many entries were replayed, the boundary flips and
their largest margin (in grid steps), entries that are neither exact nor a
flip ("bad", which fail the test), the clamped count, the free-run code
differences against the oracle's own sweep where it ran, and the proxy-loss
agreement.

usage: python tests/parity_report.py [parity_records.jsonl] > report.md
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT = os.path.join(os.path.dirname(HERE), "gpurun_out", "parity_records.jsonl")


def fmt(v, spec="%.2e"):
    if v is None:
        return "—"
    if isinstance(v, bool):
        return "yes" if v else "no"
    if isinstance(v, int):
        return str(v)
    return spec % v


def main(path):
    recs = [json.loads(ln) for ln in open(path) if ln.strip()]
    cols = ["case", "m × n", "bits", "rounding", "H_O = I", "replayed", "flips", "max flip margin", "bad",
            "clamped", "free-run diffs", "loss rel. (replay)", "loss rel. (free run / chain)"]
    print("| " + " | ".join(cols) + " |")
    print("|" + "---|" * len(cols))
    for r in recs:
        row = [r["case"], "%d × %d" % (r["m"], r["n"]), fmt(r["bits"]), r["rounding"], fmt(r.get("one_sided")),
               "%d of %d" % (r["replayed"], r["entries"]), fmt(r["flips"]), fmt(r["max_flip_margin"]),
               fmt(r["bad"]), fmt(r["clamped"]), fmt(r.get("free_mismatch")), fmt(r.get("loss_rel")),
               fmt(r.get("free_loss_rel"))]
        print("| " + " | ".join(row) + " |")
    flips = sum(r["flips"] for r in recs)
    bad = sum(r["bad"] for r in recs)
    print()
    print("%d cases; %d boundary flips in all, %d bad entries." % (len(recs), flips, bad))


if __name__ == "__main__":
    main(sys.argv[1] if len(sys.argv) > 1 else DEFAULT)
