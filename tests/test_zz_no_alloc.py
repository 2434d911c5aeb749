"""ce_forward_ex_noalloc: the allocation-free variant of ce_forward_ex, through the C ABI.

Its sum or mean keeps the reduction partials in the library's fixed per-GPU array
instead of a caller workspace.  Each call is checked bit for bit against ce_forward_ex
on the same inputs (same kernels, same fixed split of the rows), and the reduced totals
against the float64 oracle to the options tolerance.  Calls follow each other with
shrinking inputs, so a later call runs on an array that still holds more partials from
the call before: 1024 parts, then 13, then 1, then none (no reduction).
"""

import numpy as np
import pytest
import torch

from oracle import ce_options as oco
from softmax_cross_entropy_amd import abi, inputs
from tests.gpu_util import decode, from_dev, to_dev
from tests.test_ce_options_gpu import check_rows, check_total

pytestmark = pytest.mark.gpu


def _batch(rows, V, dtype, stream):
    b = inputs.normal_rows(rows, V, dtype, workload=70, stream=stream)
    y = b.targets.copy()
    y[::7] = -100
    return b.logits, y


def _both(x, y, eps, red, dtype):
    xd = to_dev(x, dtype)
    yd = torch.from_numpy(y).cuda()
    n = len(y)
    a = abi.ce_forward_ex(xd, yd, eps, -100, red)
    loss = torch.full((n,), float("nan"), device="cuda")
    lse = torch.full((n, 2), float("nan"), device="cuda")
    total = torch.full((1,), float("nan"), device="cuda") if red != "none" else None
    count = torch.full((1,), -1, dtype=torch.int64, device="cuda") if red != "none" else None
    b = abi.ce_forward_ex_noalloc(xd, yd, eps, -100, red, loss, lse, total, count)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        if u is None:
            assert v is None
            continue
        assert np.array_equal(from_dev(u).view(np.uint8), from_dev(v).view(np.uint8))
    return [None if t is None else from_dev(t) for t in b]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_noalloc_matches_ce_forward_ex_on_shrinking_calls(dtype):
    # 1024 parts (the cap): 4096 * 1024 + 777 rows of 16 classes
    x, y = _batch(4096 * 1024 + 777, 16, dtype, 1)
    loss, _, total, count = _both(x, y, 0.1, "mean", dtype)
    counted = y != -100
    assert int(count[0]) == int(counted.sum())
    # 13 parts, on an array that still holds 1024 partials
    x, y = _batch(50000, 300, dtype, 2)
    loss, _, total, count = _both(x, y, 0.5, "sum", dtype)
    z = decode(x, dtype)
    rl, _, _, rt, rc = oco.forward_index(z, y, 0.5, -100, "sum")
    check_rows(loss, rl, dtype, "loss")
    assert int(count[0]) == rc
    check_total(float(total[0]), rl, y != -100, "sum", dtype, rc)
    # one part: the partial kernel writes the result itself
    x, y = _batch(3000, 1000, dtype, 3)
    loss, _, total, count = _both(x, y, 0.1, "mean", dtype)
    z = decode(x, dtype)
    rl, _, _, rt, rc = oco.forward_index(z, y, 0.1, -100, "mean")
    check_rows(loss, rl, dtype, "loss")
    check_total(float(total[0]), rl, y != -100, "mean", dtype, rc)
    # no reduction: the array is not used
    _both(x[:100], y[:100], 0.1, "none", dtype)


def test_noalloc_argument_errors():
    n, V = 64, 100
    x = torch.zeros(n, V, device="cuda")
    y = torch.zeros(n, dtype=torch.int32, device="cuda")
    loss = torch.empty(n, device="cuda")
    lse = torch.empty(n, 2, device="cuda")
    lay = abi.CELayout(n, V, n * V)
    L = abi.lib()
    opts = abi.options(0.1, -100, "mean")
    # a mean without total or count
    st = L.ce_forward_ex_noalloc(abi._ptr(x), lay, 0, abi._ptr(y), n, V, opts, abi._ptr(loss), abi._ptr(lse),
                                 None, None, None)
    assert st == -1
    # an output overlapping the logits
    total = torch.empty(1, device="cuda")
    count = torch.empty(1, dtype=torch.int64, device="cuda")
    st = L.ce_forward_ex_noalloc(abi._ptr(x), lay, 0, abi._ptr(y), n, V, opts, abi._ptr(x), abi._ptr(lse),
                                 abi._ptr(total), abi._ptr(count), None)
    assert st == -7
    # empty batch: total of a mean is NaN, count 0
    st = L.ce_forward_ex_noalloc(abi._ptr(x), lay, 0, abi._ptr(y), 0, V, opts, abi._ptr(loss), abi._ptr(lse),
                                 abi._ptr(total), abi._ptr(count), None)
    torch.cuda.synchronize()
    assert st == 0 and int(count.item()) == 0 and np.isnan(float(total.item()))
