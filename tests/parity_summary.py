"""Summarise the GPU parity tests' JSON-lines report as a markdown table.

usage: python tests/parity_summary.py REPORT.jsonl [OUT.md] [--command "..."]

One row per compared case: tokens compared, the largest log-prob, entropy,
token-loss and support log-prob errors against the fp64 oracle, the widest
near-threshold band, the label decisions counted within 1e-6 and in
(1e-6, band] of their thresholds (and how many of those differ), the loss's
relative error and the dh / dW relative Frobenius errors (with whether the
rounding floor was applied).  Not a test; run by hand after a GPU test run.
"""

from __future__ import annotations

import json
import sys


def _fmt(v, spec=".2e"):
    if v is None:
        return "-"
    if isinstance(v, bool):
        return "floor" if v else ""
    if isinstance(v, (int,)):
        return str(v)
    return format(v, spec)


def summarise(rows, command=None):
    out = ["# GPU parity against the fp64 oracle: per-case figures", ""]
    if command:
        out += ["Command:", "", "```", command, "```", ""]
    out += ["Tolerances: log-probs, entropy and support log-probs 2e-3 absolute, the loss 1e-4",
            "relative, dh and dW 1e-2 relative Frobenius. Per-token near-threshold band: " +
            (rows[0].get("band_rule", "-") if rows else "-") + " (u = 2^-24); label decisions",
            "are counted by their oracle margin from the threshold, and every decision beyond its",
            "band must agree. \"(floor)\": the exact gradient is no larger than the rounding level",
            "of the bf16 operand (it vanishes for a one-entry vocabulary), so the absolute floor",
            "applies instead of the relative bound and the relative figure carries no meaning.", "",
            "| case | tokens | max abs lp err | max abs entropy err | max token-loss err | "
            "max support lp err | widest band | labels within 1e-6 (differ) | "
            "labels in (1e-6, band] (differ) | differ beyond band | loss rel err | "
            "dh rel Frobenius | dW rel Frobenius |",
            "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for r in rows:
        if "tokens_compared" not in r:
            continue
        dh = _fmt(r.get("dh_rel")) + (" (floor)" if r.get("dh_floor_used") else "")
        dw = _fmt(r.get("dW_rel")) + (" (floor)" if r.get("dW_floor_used") else "")
        out.append(
            f"| {r['case']} | {r['tokens_compared']} | {_fmt(r.get('max_lp_err'))} | "
            f"{_fmt(r.get('max_entropy_err'))} | {_fmt(r.get('max_token_loss_err'))} | "
            f"{_fmt(r.get('max_support_lp_err'))} | {_fmt(r.get('band_max'))} | "
            f"{r.get('labels_within_1e-6', 0)} ({r.get('labels_within_1e-6_differing', 0)}) | "
            f"{r.get('labels_in_(1e-6,band]', 0)} ({r.get('labels_in_(1e-6,band]_differing', 0)}) | "
            f"{r.get('labels_beyond_band_differing', 0)} | {_fmt(r.get('loss_rel_err'))} | "
            f"{dh} | {dw} |")
    return "\n".join(out) + "\n"


def main(argv):
    args = list(argv)
    command = None
    if "--command" in args:
        i = args.index("--command")
        command = args[i + 1]
        del args[i:i + 2]
    rows = [json.loads(line) for line in open(args[0]) if line.strip()]
    text = summarise(rows, command)
    if len(args) > 1:
        with open(args[1], "w") as f:
            f.write(text)
    else:
        sys.stdout.write(text)


if __name__ == "__main__":
    main(sys.argv[1:])
