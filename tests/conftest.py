import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")


def golden(name):
    import json
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library, built if missing; skips nothing — a GPU test without a
    GPU or without the library fails loudly."""
    import torch
    from scale_deformable_attention_msdeformattn_amd import _binding
    if not os.path.exists(_binding.LIB_PATH):
        from scale_deformable_attention_msdeformattn_amd import build
        build.build()
    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    return _binding.load()
