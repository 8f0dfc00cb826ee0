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


@pytest.fixture
def scratch_limit():
    """Set the library's stored-tile scratch limit (bytes) for one test; the
    previous limit is restored afterwards."""
    from causal_gqa_attention_bwd_amd import binding
    saved = []

    def set_limit(nbytes):
        prev = binding.set_scratch_limit(int(nbytes))
        if not saved:
            saved.append(prev)

    yield set_limit
    if saved:
        binding.set_scratch_limit(saved[0])
