import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionfinish(session, exitstatus):
    """With GQA_PARITY_STATS=<path>, write every parity comparison of the
    session (max abs and relative RMS error per case) to that JSON file."""
    path = os.environ.get("GQA_PARITY_STATS")
    if not path:
        return
    try:
        from tests.parity import STATS
    except Exception:   # noqa: BLE001 - nothing was compared
        return
    import json
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        json.dump([{"case": w, "dtype": d, "tol": t, "max_abs": m, "rel_rms": r}
                   for w, d, t, m, r in STATS], f, indent=0)
