import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle.get()


def pytest_sessionstart(session):
    # Build the library only if nothing is built yet (build() always rebuilds).
    from replicated_fp8_sparse_amd import build, kvpub
    if not os.path.exists(kvpub.LIB_PATH):
        build.build_library()
