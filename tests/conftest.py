import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU work (full-size oracle)")


_CACHE = {}


@pytest.fixture(scope="session")
def block_inputs():
    """Seeded block inputs per config name (drawn once per session)."""
    from flow_matching_diffusion_adaln_amd import configs, inputs

    def get(name, seed=0, block_id=0):
        key = (name, seed, block_id)
        if key not in _CACHE:
            _CACHE[key] = inputs.make_block_inputs(configs.CONFIGS[name], seed, block_id)
        return _CACHE[key]
    return get
