import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: longer CPU test")


@pytest.fixture(scope="session")
def oracle_mod():
    from tests._orc import Oracle
    return Oracle()


@pytest.fixture(autouse=True)
def _device_contract_checks(request):
    """GPU tests check every call's device-content contract (lengths, page
    ids, query offsets, slots) on the host before it is launched."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    import paged_gqa_attention_02_amd as pa
    prev = pa.set_input_checks(True)
    try:
        yield
    finally:
        pa.set_input_checks(prev)
