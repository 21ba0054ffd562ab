"""Renders the parity records the GPU tests write (one JSON object per parity
case, to the file named by MOE_PARITY_LOG) as a markdown report: per case the
rows, near-tie rows, id-set and order differences on ties, the worst row error
of y, and each projection class's worst-column and aggregate error against the
fp64 oracle.

    MOE_PARITY_LOG=gpurun_out/parity.jsonl python -m pytest tests -m gpu
    python tests/parity_report.py gpurun_out/parity.jsonl > tests/parity_report.md
"""
import json
import sys

CLASSES = ("logits", "gate", "up", "h", "down", "shared_h", "shared_down", "y")


def render(path):
    recs = [json.loads(l) for l in open(path) if l.strip()]
    out = ["# Parity report of the GPU tests", "",
           f"Written by `python tests/parity_report.py {path}` from the records of "
           f"`MOE_PARITY_LOG={path} python -m pytest tests -m gpu`.", "",
           "Per case: near-tie rows (8th/9th logit gap below 1e-5), rows whose id set differs "
           "on such a tie, rows whose pick order differs only within ties, the worst row error "
           "of y (max |y - y_ref| over the row's max |y_ref|; the bar is 2e-3), and per class "
           "`worst column / aggregate` relative error against the fp64 oracle.", "",
           "| case | rows | near-tie | set differs | order differs | worst row err | "
           + " | ".join(CLASSES) + " |",
           "|---" * (6 + len(CLASSES)) + "|"]
    for d in recs:
        cells = []
        for c in CLASSES:
            v = d.get(c)
            cells.append(f"{v['worst_col']:.1e} / {v['aggregate']:.1e}" if isinstance(v, dict) else "-")
        out.append(f"| {d['name']} | {d['rows']} | {d['near_tie_rows']} | {d['set_differs_on_ties']} | "
                   f"{d['order_differs_within_ties']} | {d['worst_row_err']:.2e} | " + " | ".join(cells) + " |")
    return "\n".join(out) + "\n"


if __name__ == "__main__":
    sys.stdout.write(render(sys.argv[1]))
