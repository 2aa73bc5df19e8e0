import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionfinish(session, exitstatus):
    """Writes the per-test parity record of the GPU tests (worst relative L2,
    compared and excluded positions) to the JSON file named by
    $FDLLM_PARITY_SUMMARY (nothing is written when it is unset)."""
    import json

    from tests import helpers
    path = os.environ.get("FDLLM_PARITY_SUMMARY")
    if not helpers.PARITY or not path:
        return
    out = {}
    for test, ent in sorted(helpers.PARITY.items()):
        rec = {"rel_l2_max": ent["rel_l2_max"], "rel_l2_count": ent["rel_l2_count"]}
        checks = [c.summary() for c in ent["checks"]]
        if checks:
            rec["step_checks"] = {k: sum(c[k] for c in checks) for k in checks[0]}
        rec.update(ent.get("extra", {}))
        out[test] = rec
    tot = {}
    for rec in out.values():
        for k, v in rec.get("step_checks", {}).items():
            tot[k] = tot.get(k, 0) + v
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        json.dump({"exitstatus": int(exitstatus), "totals": tot, "tests": out}, f, indent=1)
