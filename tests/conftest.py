import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests are skipped, not failed, on a machine without a GPU so that
    # `-m "not gpu"` and plain runs behave the same here.
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU on this machine")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_sessionfinish(session, exitstatus):
    # the tie-band counts of the selection comparisons (GPU parity tests):
    # per test, the groups compared, |A| in total and at most, and the in-band
    # swaps (out-of-band differences fail the test itself); written as
    # tie_band.json into the directory SS_TIE_BAND_DIR names, if it is set
    try:
        import parity
    except Exception:  # pragma: no cover
        return
    if not parity.TIE_LOG:
        return
    import json
    agg = {}
    for r in parity.TIE_LOG:
        a = agg.setdefault(r["test"], {"groups": 0, "band_total": 0, "band_max": 0,
                                        "swaps_total": 0, "swaps_max": 0, "m": r["m"], "K": r["K"]})
        a["groups"] += 1
        a["band_total"] += r["band"]
        a["band_max"] = max(a["band_max"], r["band"])
        a["swaps_total"] += r["swaps"]
        a["swaps_max"] = max(a["swaps_max"], r["swaps"])
    out = os.environ.get("SS_TIE_BAND_DIR")
    if not out:
        return
    try:
        os.makedirs(out, exist_ok=True)
        with open(os.path.join(out, "tie_band.json"), "w") as f:
            json.dump(agg, f, indent=1)
    except OSError:  # pragma: no cover
        pass
