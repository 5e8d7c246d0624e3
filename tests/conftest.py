import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionfinish(session, exitstatus):
    """Writes the session's parity statistics (tests/parity.py RECORD) to the
    JSON file named by MOE_PARITY_RECORD, when set."""
    path = os.environ.get("MOE_PARITY_RECORD")
    if not path:
        return
    try:
        import parity
    except ImportError:
        return
    if parity.RECORD:
        os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
        with open(path, "w") as f:
            json.dump(parity.RECORD, f, indent=1, sort_keys=True)
