import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(autouse=True)
def _no_nonfinite_outputs(request):
    """After every GPU test: no retention call wrote a non-finite value that
    the test did not itself query (the library's non-finite record is clear)."""
    yield
    if request.node.get_closest_marker("gpu") is None:
        return
    import torch
    if not torch.cuda.is_available():
        return
    from linear_attention_sequence_retention_amd import binding
    msg = binding.range_status()
    assert msg is None, f"non-finite outputs were written: {msg}"
