import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (MI355X / gfx950) and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The built library on a GPU.  Fails loudly (not skips) when the library is missing on a machine with a GPU."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from paged_kv_cache_199_amd import _lib

    return _lib.load()


@pytest.fixture(autouse=True)
def _poison_library_workspaces(monkeypatch):
    """Workspaces the binding allocates for a call are filled with 0xFF bytes (NaN in every fp32 word)
    instead of left uninitialized: the ABI says their contents on entry do not matter, so a kernel that
    reads a slot before writing it shows up as NaN in the output under test."""
    import torch

    from paged_kv_cache_199_amd import _lib

    def poisoned(nbytes, device):
        return torch.full((max(int(nbytes), 1),), 0xFF, dtype=torch.uint8, device=device)

    monkeypatch.setattr(_lib, "new_workspace", poisoned)
