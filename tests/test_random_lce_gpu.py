"""GPU: lce_forward and lce_backward on seeded random shapes against the float64 oracle.

Each case draws N (1 to 600), D (a multiple of 8, 8 to 512), V (log-uniform, 1 to 20,000,
or for odd seeds 8193 to 24,576, more than one backward chunk) and a logit scale s (W ~ N(0, s^2 / D), s log-uniform in [0.3, 6]), so that the tiles'
row, column and K tails land anywhere and the softmax runs from flat to nearly one-hot.
Targets are uniform, and about a quarter of the rows point at their own argmax.  Checks:
the forward's loss and lse under the rule of tests/test_lce_gpu.py; the backward in both
layouts (chunks of 8192 columns and one chunk over the whole vocabulary) equal bit for
bit, and within the bound of tests/test_lce_backward_gpu.py against the oracle, plus the
cancellation allowance at each row's target: a nearly one-hot row's dZ_iy = g_i (p_y - 1)
comes from a float32 p_y within 2^-23 of the exact value, so it carries up to |g_i| 2^-23
of absolute error, which reaches dH row i through W_y and dW row y through H_i; 2^-22 is
allowed.
"""

import numpy as np
import pytest
import torch

from oracle import lce as olce
from softmax_cross_entropy_amd import abi, inputs
from tests.test_lce_backward_gpu import REL, upstream, within
from tests.test_lce_gpu import check, dev_bf16

pytestmark = pytest.mark.gpu


def draw(seed):
    g = np.random.default_rng([779, seed])
    N = int(g.integers(1, 601))
    D = 8 * int(g.integers(1, 65))
    # odd seeds take more than one 8192-column chunk, where the two backward layouts differ
    V = int(np.exp(g.uniform(0.0, np.log(20000)))) if seed % 2 == 0 else int(g.integers(8193, 24577))
    s = float(np.exp(g.uniform(np.log(0.3), np.log(6.0))))
    H, W, y = inputs.linear_ce(N, D, V, seed_stream=1000 + seed, w_scale=s * D ** -0.5)
    Z = olce.logits(olce.decode_bf16(H), olce.decode_bf16(W))
    pick = g.random(N) < 0.25
    y = np.where(pick, np.argmax(Z, axis=1), y).astype(np.int32)
    return N, D, V, s, H, W, y


@pytest.mark.parametrize("seed", range(16))
def test_random_shape(seed):
    N, D, V, s, H, W, y = draw(seed)
    _, lse, err = check(H, W, y)
    g = upstream(N, seed)
    Hd, Wd = dev_bf16(H), dev_bf16(W)
    yd = torch.from_numpy(y).cuda()
    lse_d = torch.from_numpy(lse.astype(np.float32)).cuda()
    gd = torch.from_numpy(g.astype(np.float32)).cuda()
    cH, cW = abi.lce_backward(Hd, Wd, yd, lse_d, gd)
    oH, oW = abi.lce_backward(Hd, Wd, yd, lse_d, gd, one_pass=True)
    torch.cuda.synchronize()
    assert torch.equal(cH.view(torch.int32), oH.view(torch.int32))
    assert torch.equal(cW.view(torch.int32), oW.view(torch.int32))
    rH, rW, bH, bW = olce.grad(H, W, y, g, bounds=True)
    # the targets' cancellation allowance, folded into the bounds (within() scales them by REL)
    H64, W64 = olce.decode_bf16(H), olce.decode_bf16(W)
    slack = np.abs(g)[:, None] * 2.0 ** -22
    xH = slack * np.abs(W64[y])
    xW = np.zeros_like(W64)
    np.add.at(xW, y, slack * np.abs(H64))
    eH = within(oH.cpu().numpy().astype(np.float64), rH, bH + xH / REL, "dH")
    eW = within(oW.cpu().numpy().astype(np.float64), rW, bW + xW / REL, "dW")
    print(f"seed {seed}: N={N} D={D} V={V} scale {s:.2f}: max |dloss| {err:.1e}, "
          f"dH {eH:.1e}, dW {eW:.1e} of the bound")
