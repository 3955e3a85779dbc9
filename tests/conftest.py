import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


@pytest.fixture(scope="session")
def oracle():
    import oracle as _oracle
    return _oracle


def pytest_collection_finish(session):
    """Start the oracle runs of the selected full-size forward checks in
    background threads, so they overlap the GPU tests collected before them."""
    if session.config.option.collectonly:
        return
    wanted = set()
    for item in session.items:
        if getattr(item, "originalname", "") == "test_forward_full_size":
            callspec = getattr(item, "callspec", None)
            if callspec is not None and "name" in callspec.params:
                wanted.add(callspec.params["name"])
    if wanted:
        import oracle_bg
        oracle_bg.prefetch(sorted(wanted))
