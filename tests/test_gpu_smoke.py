"""The package's smoke entry point (one small bf16 GBLA forward+backward on
cuda:0 through the C ABI, checked against the float64 oracle) runs clean."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
def test_smoke_entry_point():
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import __graft_entry__

    __graft_entry__.smoke()
