import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    # name the case before any GPU work, so a run that dies names its test
    gpu = request.node.get_closest_marker("gpu") is not None
    if gpu:
        print(f"\n[gpu case] {request.node.nodeid}", flush=True)
    yield
    # no bounded wait (chunked look-back, matrix ring) may have given up
    # during a GPU test: its results would be NaN and counted here
    if gpu and "device" in request.fixturenames:
        import linear_attention_rnn_forward_amd as wkv
        before = request.config.stash.get(_WAIT_KEY, 0)
        now = wkv.bounded_wait_failures()
        request.config.stash[_WAIT_KEY] = now
        assert now == before, f"{now - before} bounded wait(s) gave up during {request.node.nodeid}"


_WAIT_KEY = pytest.StashKey[int]()


@pytest.fixture(scope="session")
def device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import linear_attention_rnn_forward_amd as wkv
    wkv.lib()  # fails loudly when the library was not built
    return torch.device("cuda:0")
