import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
for _p in (ROOT, os.path.dirname(os.path.abspath(__file__))):
    if _p not in sys.path:
        sys.path.insert(0, _p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size parity case")


def _ensure_library():
    """Tests load the built library; they build it only when none exists."""
    lib = os.path.join(ROOT, "cross_model_attention_mf_amd", "libmapflow.so")
    if not os.path.exists(lib):
        from cross_model_attention_mf_amd import build_lib
        build_lib.build()


_ensure_library()
