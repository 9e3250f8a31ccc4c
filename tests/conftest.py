import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session", autouse=True)
def built_libraries():
    """Build liblsh.so if it is missing or was built from other sources than
    those in the tree (its recorded source digest differs), and the oracle if
    it is missing or older than its source."""
    from lsh_sparse_attention_hash_amd import build as lib_build
    from oracle import oracle
    if not lib_build.is_current():
        print("liblsh.so is missing or stale: rebuilding", flush=True)
        lib_build.build()
    oracle.build(force=False)
    yield
