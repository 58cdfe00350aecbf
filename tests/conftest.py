"""Shared test setup: marker registration, repo root on sys.path, and a check
that the in-tree native libraries exist (built by __graft_entry__.build())."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the HIP library")


def _ensure_cpu_libs():
    import __graft_entry__ as g
    if not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")):
        g.build_oracle()
    if not os.path.exists(os.path.join(ROOT, "synth", "libsynth.so")):
        g.build_synth()


_ensure_cpu_libs()


@pytest.fixture(scope="session")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")
