"""Largest deviations of the GPU outputs from the oracle, gathered per test
file and PV mode while the GPU tests run and printed at the end of the run by
``conftest.pytest_terminal_summary``, so that the margin to each bar shows in
a quiet run's tail as well as in the per-case lines."""
import os
import re

MAX_ABS_BAR = 2e-2
COS_O1_BAR = 0.9995
COS_O2_BAR = 0.998

RECORDS = {}


def _where():
    node = os.environ.get("PYTEST_CURRENT_TEST", "?::?").split(" ")[0]
    path, _, name = node.partition("::")
    params = name[name.find("["):] if "[" in name else ""
    fname = os.path.basename(path)
    if "mxfp4" in fname or "mxfp4" in params:
        mode = "mxfp4"
    elif re.search(r"fp8", params):
        mode = "fp8"
    else:
        mode = "fp16"
    return fname, mode


def record(label, max_abs, cos_o1=None, cos_o2=None):
    """Note one comparison of GPU output with the oracle's method (O1) and,
    where made, with exact fp64 attention (O2)."""
    key = _where()
    r = RECORDS.setdefault(key, {"max_abs": -1.0, "label": "", "cos_o1": 2.0, "cos_o2": 2.0, "n": 0})
    r["n"] += 1
    if max_abs > r["max_abs"]:
        r["max_abs"], r["label"] = float(max_abs), label
    if cos_o1 is not None:
        r["cos_o1"] = min(r["cos_o1"], float(cos_o1))
    if cos_o2 is not None:
        r["cos_o2"] = min(r["cos_o2"], float(cos_o2))


def summary_lines():
    if not RECORDS:
        return []
    out = [f"worst output deviation from the oracle per test file and PV mode (bars: max-abs <= {MAX_ABS_BAR:g} "
           f"and cos >= {COS_O1_BAR} vs the method O1; cos >= {COS_O2_BAR} vs exact attention O2):"]
    for (fname, mode), r in sorted(RECORDS.items()):
        c1 = f"{r['cos_o1']:.6f}" if r["cos_o1"] <= 1.0 else "-"
        c2 = f"{r['cos_o2']:.6f}" if r["cos_o2"] <= 1.0 else "-"
        out.append(f"  {fname} [{mode}] {r['n']} checks: max_abs {r['max_abs']:.3e} "
                   f"(margin {MAX_ABS_BAR - r['max_abs']:.3e}; {r['label']}), min cos_O1 {c1}, min cos_O2 {c2}")
    return out
