"""GPU: ce_forward and ce_vjp on seeded random views against the float64 oracle.

Each case draws a dtype, a vocabulary size (log-uniform up to 70,000, so it lands in
every layout: one lane per row, lanes per row, a workgroup per row, the chunked VJP),
and a strided [B, L, V] view cut out of a wider padded buffer: a slice of its rows
([:, :-1] or [:, 1:]) and a column offset, so rows start at any element alignment.
Logits are N(0, s^2) with a random scale s; targets are uniform; g is U[0.25, 2).
Tolerances are the stated ones (tests/gpu_util.py), with the target elements' cancellation
allowance: at scale 20 a short row's target probability can round to 1 in float32.
"""

import numpy as np
import pytest
import torch

from oracle import ce as oce
from softmax_cross_entropy_amd import abi, inputs
from tests.gpu_util import check_grad, check_lse, check_loss, from_dev, to_dev

pytestmark = pytest.mark.gpu

DTYPES = ["f32", "f16", "bf16"]


def draw(seed):
    g = np.random.default_rng([777, seed])
    dtype = DTYPES[int(g.integers(3))]
    V = int(np.exp(g.uniform(0.0, np.log(70000))))
    B = int(g.integers(1, 5))
    L = int(g.integers(2, 60))
    pad = int(g.integers(0, 10))        # extra columns per stored row
    off = int(g.integers(0, pad + 1))   # the view's first column
    cut = int(g.integers(3))            # 0: all rows, 1: [:, :-1], 2: [:, 1:]
    scale = float(np.exp(g.uniform(np.log(0.1), np.log(20.0))))
    store = inputs.encode(inputs.normal_f32(g, (B, L, V + pad), scale), dtype)
    rows = {0: slice(0, L), 1: slice(0, L - 1), 2: slice(1, L)}[cut]
    view = store[:, rows, off:off + V]
    n = view.shape[0] * view.shape[1]
    y = inputs.uniform_targets(g, (n,), V)
    gr = g.uniform(0.25, 2.0, n).astype(np.float32)
    return dtype, V, store, rows, off, view, y, gr


@pytest.mark.parametrize("seed", range(40))
def test_random_view(seed):
    dtype, V, store, rows, off, view, y, gr = draw(seed)
    dev = to_dev(store, dtype)
    x = dev[:, rows, off:off + V]
    t = torch.from_numpy(y).cuda()
    loss, lse = abi.ce_forward(x, t)
    d = abi.ce_vjp(x, t, lse, torch.from_numpy(gr).cuda())
    torch.cuda.synchronize()
    z = oce.decode(np.ascontiguousarray(view).reshape(-1, V), dtype)
    rl, rm, rls = oce.forward(z, y)
    rd = oce.grad(z, y, gr.astype(np.float64), rm, rls)
    check_loss(loss.cpu().numpy(), rl, dtype)
    check_lse(lse.cpu().numpy(), rm, rls, dtype)
    check_grad(from_dev(d).reshape(-1, V), rd, dtype, targets=y, g=gr)
    print(f"seed {seed}: {dtype} V={V} view {tuple(x.shape)} strides {tuple(x.stride())}")
