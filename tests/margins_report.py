"""Parity margins summary: reads the JSON that a GPU test run writes when
PKV_MARGINS names a file (tests/conftest.py) and prints a markdown table of how
far each attention comparison sits under the bounds (max-abs 2e-3, relative L2
1e-3 against the fp64 oracle).

    python tests/margins_report.py <margins.json> "<command that made it>"
"""

import json
import sys
from collections import defaultdict

TOL_MAX_ABS = 2e-3
TOL_REL_L2 = 1e-3


def main(path, command):
    data = json.load(open(path))
    rows = data["margins"]
    out = ["# Parity margins: every attention comparison of the GPU test suite", "",
           "Command (one MI355X):", "", f"    {command}", "",
           f"{len(rows)} comparisons against the fp64 oracle; pytest exit status "
           f"{data['exitstatus']}.  Headroom = bound / error (larger is safer).", "",
           "## Full-size workloads (every request and head compared)", "",
           "| Case | Rows | max-abs | headroom | rel-L2 | headroom |", "|---|---|---|---|---|---|"]
    for r in rows:
        if not r["label"]:
            continue
        out.append(f"| {r['label']} | {r['rows']} | {r['max_abs']:.2e} | "
                   f"{TOL_MAX_ABS / max(r['max_abs'], 1e-30):.0f}x | {r['rel_l2']:.2e} | "
                   f"{TOL_REL_L2 / max(r['rel_l2'], 1e-30):.0f}x |")
    worst = defaultdict(lambda: {"n": 0, "max_abs": 0.0, "rel_l2": 0.0})
    for r in rows:
        w = worst[r["test"].split("[")[0]]
        w["n"] += 1
        w["max_abs"] = max(w["max_abs"], r["max_abs"])
        w["rel_l2"] = max(w["rel_l2"], r["rel_l2"])
    out += ["", "## Worst case per test function (all parametrisations)", "",
            "| Test | Comparisons | worst max-abs | headroom | worst rel-L2 | headroom |",
            "|---|---|---|---|---|---|"]
    for name, w in sorted(worst.items(), key=lambda kv: -kv[1]["max_abs"] / TOL_MAX_ABS
                          - kv[1]["rel_l2"] / TOL_REL_L2):
        out.append(f"| `{name}` | {w['n']} | {w['max_abs']:.2e} | "
                   f"{TOL_MAX_ABS / max(w['max_abs'], 1e-30):.0f}x | {w['rel_l2']:.2e} | "
                   f"{TOL_REL_L2 / max(w['rel_l2'], 1e-30):.0f}x |")
    print("\n".join(out))


if __name__ == "__main__":
    main(sys.argv[1], sys.argv[2] if len(sys.argv) > 2 else "")
