import os
import shutil
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def gpu():
    # the oracle's worker processes fork from a server started before this process
    # touches the GPU (no worker is a copy of a process holding the device)
    from oracle import pool
    pool.start_server()
    if not gpu_available():
        pytest.skip("no GPU visible")
    import torch
    return torch.device("cuda:0")


@pytest.fixture(scope="session")
def oracle_pool(gpu):
    """Worker processes (one per core, at most 16) that run the fp64 oracle."""
    from oracle import pool
    p = pool.make_pool()
    yield p
    p.terminate()
    p.join()


@pytest.fixture
def result_dir(tmp_path):
    """A directory for one test's result files (several GB for a full batch),
    removed when the test ends, passed or not, so that a session's full-batch
    tests do not fill the disk between them."""
    yield str(tmp_path)
    shutil.rmtree(tmp_path, ignore_errors=True)
