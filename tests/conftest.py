import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle():
    import oracle as o
    o.lib()
    return o


@pytest.fixture
def poisoned_outputs(monkeypatch):
    """Tensors that the binding allocates (outputs, DAPD workspaces) start as
    0xA5 bytes instead of whatever the caching allocator hands back, so an
    element that a kernel fails to write cannot pass by still holding an
    earlier call's value.  The zero-filled statistics workspace is made with
    torch.zeros and is left alone."""
    import torch
    from diffusion_lm_unmask_amd import api

    class _Torch:
        def __getattr__(self, name):
            return getattr(torch, name)

        @staticmethod
        def empty(*args, **kwargs):
            t = torch.empty(*args, **kwargs)
            if t.numel():
                t.view(-1).view(torch.uint8).fill_(0xA5)
            return t

    monkeypatch.setattr(api, "torch", _Torch())
