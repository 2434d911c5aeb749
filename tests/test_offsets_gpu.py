"""GPU parity at large per-row offsets for the KL, Jensen-Shannon and cross-entropy
option kernels.

"Shift by the max in cross_entropy", Proposed changes: the max shift comes before
anything else, so every path gains from it, label smoothing and probability targets
included.  Each student row and each teacher row here carries its own offset, drawn
independently from {0, 1e2, 1e4, 1e6, 1e8} (float32) or {0, 1e4} (float16: it cannot
store 1e6), so a pair's two offsets differ by up to 1e8.  Results are held to the same
tolerances as the unshifted tests (tests/test_kl_gpu.py, tests/test_js_gpu.py,
tests/test_ce_options_gpu.py), against the float64 oracle on the stored values.
"""

import numpy as np
import pytest
import torch

from oracle import ce_options as oco
from softmax_cross_entropy_amd import abi, inputs
from tests import test_js_gpu as tjs
from tests import test_kl_gpu as tkl
from tests.test_ce_options_gpu import check_opt_grad, check_rows, check_total, full_index_check, upstream
from tests.gpu_util import decode, from_dev, to_dev

pytestmark = pytest.mark.gpu

OFFSETS = {"f32": (0.0, 1e2, 1e4, 1e6, 1e8), "f16": (0.0, 1e4)}
SHAPES = ((64, 151936), (96, 1000), (40, 37))


def offset_pair(rows, V, dtype, workload):
    q, p, _ = inputs.kl_pair(rows, V, dtype, scale=4.0 if dtype == "f32" else 2.0, workload=workload)
    q, cq = inputs.with_row_offsets(q, dtype, OFFSETS[dtype], workload, 1)
    p, cp = inputs.with_row_offsets(p, dtype, OFFSETS[dtype], workload, 2)
    assert np.any(cq != cp)
    g = np.linspace(0.5, 2.0, rows).astype(np.float32)
    return q, p, g


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("rows,V", SHAPES)
def test_kl_offsets(dtype, rows, V):
    q, p, g = offset_pair(rows, V, dtype, workload=60 + V % 97)
    _, _, e = tkl.full_check(q, p, g, dtype)
    print(f"kl {dtype} V={V}: max |dkl| {e:.2e}")


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("rows,V", SHAPES)
def test_js_offsets(dtype, rows, V):
    q, p, g = offset_pair(rows, V, dtype, workload=61 + V % 97)
    _, _, e = tjs.full_check(q, p, g, dtype)
    print(f"js {dtype} V={V}: max |djs| {e:.2e}")


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("rows,V", SHAPES)
def test_index_options_offsets(dtype, rows, V):
    b = inputs.normal_rows(rows, V, dtype, workload=62, stream=V)
    x, _ = inputs.with_row_offsets(b.logits, dtype, OFFSETS[dtype], 62, V)
    y = b.targets.copy()
    y[::9] = -100
    for eps in (0.1, 0.5):
        for red in ("none", "mean"):
            full_index_check(x, y, eps, -100, red, dtype, seed=V)


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("rows,V", SHAPES)
def test_probability_targets_offsets(dtype, rows, V):
    b = inputs.normal_rows(rows, V, dtype, workload=63, stream=V)
    x, _ = inputs.with_row_offsets(b.logits, dtype, OFFSETS[dtype], 63, V)
    ts = inputs.prob_targets(rows, V, dtype, workload=63, stream=V + 1, normalised_rows=rows // 2)
    z, zt = decode(x, dtype), decode(ts, dtype)
    for eps in (0.0, 0.1, 0.5):
        for red in ("none", "sum"):
            g = upstream(red, rows, V)
            xd, td = to_dev(x, dtype), to_dev(ts, dtype)
            loss, lse, wsum, total, count = abi.ce_forward_probs(xd, td, eps, red)
            d = abi.ce_vjp_probs(xd, td, lse, wsum, torch.from_numpy(g).cuda(), eps, red, count=count)
            torch.cuda.synchronize()
            rl, rm, _, _, _, _ = oco.forward_probs(z, zt, eps, red)
            check_rows(from_dev(loss), rl, dtype, f"probs loss V={V} eps={eps} red={red}")
            fin = np.isfinite(rm)
            assert np.array_equal(from_dev(lse)[fin, 0], rm[fin])
            counted = np.ones(rows, bool)
            if red != "none":
                check_total(float(total.item()), rl, counted, red, dtype, rows)
            gg = g if red == "none" else g[0]
            gi = oco.row_upstream(gg, counted, red, rows)
            check_opt_grad(from_dev(d), oco.grad_probs(z, zt, gg, eps, red), z, oco.prob_weights(zt, eps), gi,
                           dtype, f"probs dlogits V={V} eps={eps} red={red}")
