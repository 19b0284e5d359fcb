"""Compact form of a GPU parity record (written by the GPU tests' session,
see conftest.py): per test and output the largest max-abs error, the max
|ref| it was measured against, their ratio, the closest approach to the
bound (largest error minus bound over the elements, <= 0 when inside) and
the number of comparisons; plus a markdown table of the same.

    python tests/parity_summary.py gpurun_out/parity_record.json profiles/parity_record
writes profiles/parity_record.json and profiles/parity_record.md.
"""
import json
import sys


def summarise(doc):
    per = {}
    for r in doc["comparisons"]:
        key = (r["test"], r["output"])
        e = per.setdefault(key, {"test": r["test"], "output": r["output"], "max_abs": 0.0, "max_ref": 0.0,
                                 "excess": -float("inf"), "comparisons": 0, "elements": 0, "tol": r["tol"]})
        if r["max_abs"] >= e["max_abs"]:
            e["max_abs"], e["max_ref"] = r["max_abs"], r["max_ref"]
        e["excess"] = max(e["excess"], r["excess"])
        e["comparisons"] += 1
        e["elements"] += int(r["n"])
    rows = sorted(per.values(), key=lambda e: (e["test"], "out lse dq dk dv".split().index(e["output"])))
    for e in rows:
        e["rel_to_max_ref"] = e["max_abs"] / e["max_ref"] if e["max_ref"] else 0.0
    return rows


def main(src, dst):
    doc = json.load(open(src))
    rows = summarise(doc)
    out = {"exitstatus": doc["exitstatus"], "n_comparisons": doc["n_comparisons"],
           "largest_error_per_output": {k: {f: v[f] for f in ("test", "ctx", "max_abs", "max_ref", "tol")}
                                        for k, v in doc["largest_error_per_output"].items()},
           "closest_to_bound_per_output": {k: {f: v[f] for f in ("test", "ctx", "max_abs", "max_ref", "excess")}
                                           for k, v in doc["closest_to_bound_per_output"].items()},
           "per_test": rows}
    with open(dst + ".json", "w") as f:
        json.dump(out, f, indent=0)
    lines = ["# Parity record of the GPU tests", "",
             "Every comparison of the HIP path with the fp64 oracle made by `pytest -m gpu` (session exit status "
             f"{doc['exitstatus']}, {doc['n_comparisons']} comparisons). Bounds: out max-abs 2e-2, lse max-abs "
             "1e-3, dq/dk/dv max-abs 2e-2 plus 2^-8 |ref| where |ref| >= 4 (bf16's half ulp). `closest` is the "
             "largest (error - bound) over the elements: negative means inside the bound.", "",
             "Command: `python -m pytest $(ls tests/test_*.py) -m gpu -x -q` on the MI355X box, then "
             "`python tests/parity_summary.py gpurun_out/parity_record.json profiles/parity_record`.", "",
             "| output | largest max-abs | its max \\|ref\\| | test |", "|---|---|---|---|"]
    for k, v in doc["largest_error_per_output"].items():
        lines.append(f"| {k} | {v['max_abs']:.3e} | {v['max_ref']:.3g} | {v['test'].split('::', 1)[1]} |")
    lines += ["", "| test | output | max-abs | max \\|ref\\| | ratio | closest | elements |", "|---|---|---|---|---|---|---|"]
    for e in rows:
        lines.append(f"| {e['test'].split('::', 1)[1]} | {e['output']} | {e['max_abs']:.2e} | {e['max_ref']:.3g} | "
                     f"{e['rel_to_max_ref']:.1e} | {e['excess']:.2e} | {e['elements']} |")
    with open(dst + ".md", "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main(sys.argv[1], sys.argv[2])
