import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


_MASKS = {}


@pytest.fixture(scope="session")
def config_mask():
    """Cached [S, S] bool mask of a workload id (generation of the 16k mask
    takes a few seconds, so it is built once per session)."""
    from workloads import get_config, make_mask

    def get(cid):
        if cid not in _MASKS:
            _MASKS[cid] = make_mask(get_config(cid))
        return _MASKS[cid]
    return get


_ENCS = {}


@pytest.fixture(scope="session")
def config_encoding(config_mask):
    """Cached oracle (scalar C) encoding of a workload's mask."""
    from oracle.encode import encode_c

    def get(cid):
        if cid not in _ENCS:
            _ENCS[cid] = encode_c(config_mask(cid))
        return _ENCS[cid]
    return get
