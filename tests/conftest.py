import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def _gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


def pytest_sessionfinish(session, exitstatus):
    """Write the parity record of the GPU comparisons made in this session
    (nothing when none ran) to $FFA_PARITY_RECORD, by default
    gpurun_out/parity_record.json under the repository root."""
    gu = sys.modules.get("gpu_util")
    rec = getattr(gu, "PARITY", None) if gu is not None else None
    if not rec:
        return
    import json
    import platform

    path = os.environ.get("FFA_PARITY_RECORD", os.path.join(ROOT, "gpurun_out", "parity_record.json"))
    os.makedirs(os.path.dirname(path) or ".", exist_ok=True)
    worst, closest = {}, {}
    for r in rec:
        k = r["output"]
        if k not in worst or r["max_abs"] > worst[k]["max_abs"]:
            worst[k] = r
        if k not in closest or r["excess"] > closest[k]["excess"]:
            closest[k] = r
    doc = {"host": platform.node(), "exitstatus": int(exitstatus), "n_comparisons": len(rec),
           "largest_error_per_output": worst, "closest_to_bound_per_output": closest, "comparisons": rec}
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
