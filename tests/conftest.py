import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle.build(force=False)
    return oracle


def pytest_sessionfinish(session, exitstatus):
    """Write the parity errors measured in this session to
    $ATTN_PARITY_RECORD (a JSON measurement record), if that is set."""
    path = os.environ.get("ATTN_PARITY_RECORD")
    if not path:
        return
    try:
        import json
        import support
    except ImportError:
        return
    if support.ERRORS:
        with open(path, "w") as f:
            json.dump(dict(sorted(support.ERRORS.items())), f, indent=1)
