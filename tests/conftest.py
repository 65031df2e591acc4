import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    import _progress
    _progress.bind(config)


def pytest_runtest_logstart(nodeid, location):
    # name the case on the real stderr before it runs, so a run that dies
    # inside a GPU call still says which case it was
    sys.__stderr__.write(f"[case] {nodeid}\n")
    sys.__stderr__.flush()


@pytest.fixture(scope="session")
def device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import post_weight_quantization_gq_amd as gq
    gq.library()          # raises if the HIP library was not built
    return torch.device("cuda:0")
