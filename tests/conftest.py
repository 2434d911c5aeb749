import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU work (full-size oracle runs)")


_FULL_LCE = {}


@pytest.fixture(scope="session")
def full_lce():
    """The full-size linear cross-entropy inputs, N = 8192, D = 4096, V = 151,936 (H, W as
    bf16 bits, targets), and W decoded to float64 for the oracle: drawn once per session
    and shared by the forward and backward tests."""
    if not _FULL_LCE:
        from oracle import lce as olce
        from softmax_cross_entropy_amd import inputs
        H, W, y = inputs.linear_ce(8192, 4096, 151936)
        _FULL_LCE.update(H=H, W=W, y=y, W64=olce.decode_bf16(W))
    return _FULL_LCE


def full_lce_oracle(d):
    """The oracle's (loss, m, log s) on every row of the full-size inputs, computed once."""
    if "ref" not in d:
        from oracle import lce as olce
        d["ref"] = olce.forward(d["H"], d["W"], d["y"], W64=d["W64"])
    return d["ref"]
