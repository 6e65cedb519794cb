import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload, sampled outputs")


def pytest_collection_modifyitems(config, items):
    # A GPU test that runs without a GPU would only test the skip path: say so loudly.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible (torch.cuda.is_available() is False)")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


@pytest.fixture
def force():
    """Pin the library's kernel choice for one test through tmm_set_override:
    force(tile) / force(tile, skinny="<bm>x<bn>") / force(conv="quad") /
    force(tile, ring=8) / force() for the automatic choice; the automatic
    choice is restored when the test ends."""
    import tiled_matrix_multiplication_amd as t

    def pin(tile=None, skinny=None, conv=None, ring=None):
        items = ([f"tile={tile}"] if tile else []) + ([f"skinny={skinny}"] if skinny else []) + \
                ([f"conv={conv}"] if conv else []) + ([f"ring={ring}"] if ring else [])
        t.tmm_set_override(";".join(items) or None)

    yield pin
    t.tmm_set_override(None)
