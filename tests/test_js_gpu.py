"""GPU parity of js_forward / js_vjp against the float64 oracle (oracle/js.py).

Tolerances.  js is a sum of terms each computed in float32 with errors of a few 1e-7 of
its P_j + Q_j, so for float32 inputs |js - ref| <= 1e-5 (1 + |ref|); for 16-bit inputs
1e-3 |ref| + 1e-5.  H (the student's half) follows the same rule.  A gradient entry
g Q_k (h_k - H) keeps only an absolute accuracy of about 1e-5 g (Q_k + P_k) where h_k ~ H,
so the gradient rule of tests/gpu_util.py is widened by that term, as for the KL.
"""

import math

import numpy as np
import pytest
import torch

from oracle import js as ojs
from softmax_cross_entropy_amd import abi, inputs
from tests.gpu_util import TORCH_DT, decode, from_dev, to_dev, ulp16

pytestmark = pytest.mark.gpu

LN2 = math.log(2.0)


def check_val(got, ref, dtype, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(ref)), f"{what}: NaN pattern differs"
    ok = ~np.isnan(ref)
    tol = 1e-5 * (1 + np.abs(ref[ok])) if dtype == "f32" else 1e-3 * np.abs(ref[ok]) + 1e-5
    err = np.abs(got[ok] - ref[ok])
    assert np.all(err <= tol), f"{what}: {np.sum(err > tol)} rows off, worst {err.max():.3e}"
    return float(err.max()) if err.size else 0.0


def check_dq(got_store, zq, zp, g, dtype):
    ref = ojs.grad(zq, zp, g)
    got = decode(got_store, dtype)
    assert np.array_equal(np.isnan(got), np.isnan(ref)), "dq: NaN pattern differs"
    ok = ~np.isnan(ref)
    with np.errstate(invalid="ignore", over="ignore"):
        Q = np.exp(ojs.kl.log_softmax(zq))
        P = np.exp(ojs.kl.log_softmax(zp))
    cancel = 1e-5 * np.abs(np.asarray(g, np.float64))[:, None] * np.nan_to_num(Q + P)
    base = np.full_like(ref, 1e-5) if dtype == "f32" else np.maximum(1e-3 * np.abs(ref), ulp16(ref, dtype))
    tol = base + cancel
    err = np.abs(got - ref)
    bad = ok & (err > tol)
    assert not bad.any(), (f"dq: {bad.sum()} elements off; first at {np.argwhere(bad)[0]}: "
                           f"got {got[bad][0]!r} ref {ref[bad][0]!r} tol {tol[bad][0]!r}")


def run(q, p, g, dtype, lanes=0, qd=None, pd=None):
    qd = to_dev(q, dtype) if qd is None else qd
    pd = to_dev(p, dtype) if pd is None else pd
    js, lq, lp, hq = abi.js_forward(qd, pd, lanes_per_row=lanes)
    dq = abi.js_vjp(qd, pd, lq, lp, hq, torch.from_numpy(np.asarray(g, np.float32)).cuda(), lanes_per_row=lanes)
    torch.cuda.synchronize()
    return from_dev(js), from_dev(lq), from_dev(lp), from_dev(hq), from_dev(dq)


def full_check(q, p, g, dtype, lanes=0):
    js, lq, lp, hq, dq = run(q, p, g, dtype, lanes)
    zq, zp = decode(q, dtype), decode(p, dtype)
    rj, mq, lsq, mp, lsp, rH = ojs.forward(zq, zp)
    e = check_val(js, rj, dtype, "js")
    check_val(hq, rH, dtype, "hq")
    fin = np.isfinite(mq)
    assert np.array_equal(lq[fin, 0], mq[fin])
    check_dq(dq, zq, zp, g, dtype)
    return js, dq, e


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_barrier_regression_shape_and_repeat(dtype):
    """128 x 151,936 ("One barrier short", The fix: the regression test's shape), then
    ten more calls bit-identical to the first."""
    q, p, g = inputs.kl_pair(128, 151936, dtype, scale=4.0 if dtype != "f16" else 2.0, workload=30)
    js, dq, e = full_check(q, p, g, dtype)
    print(f"{dtype}: max |djs| {e:.2e}")
    for _ in range(10):
        j2, _, _, _, d2 = run(q, p, g, dtype)
        assert np.array_equal(j2.view(np.uint32), js.view(np.uint32))
        assert np.array_equal(d2, dq)


def test_logit_scale_20_is_finite():
    """"One barrier short", The fix: at a logit scale of 20 the Jensen-Shannon loss overflowed
    to non-finite values; with the stable softplus it is finite and matches the oracle."""
    q, p, g = inputs.kl_pair(64, 151936, "f32", scale=20.0, workload=31)
    js, dq, _ = full_check(q, p, g, "f32")
    assert np.isfinite(js).all() and np.all(js >= 0) and np.all(js <= LN2 + 1e-5)
    assert np.isfinite(dq).all()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_boundary_sizes_all_lane_counts(dtype):
    for V in (1, 2, 7, 8, 9, 63, 64, 65, 1000, 1024, 4097, 9001):
        q, p, g = inputs.kl_pair(67, V, dtype, workload=32, stream=V)
        g = np.linspace(0.5, 2.0, 67).astype(np.float32)
        for lanes in (0, 1, 4, 16, 64, 128, 1024):
            full_check(q, p, g, dtype, lanes)


def test_identical_rows_give_zero_and_disjoint_supports_ln2():
    q, _, g = inputs.kl_pair(64, 5000, "f32", workload=33)
    js, _, _, hq, dq = run(q, q, g, "f32")
    assert np.all(js == 0.0) and np.all(hq == 0.0) and np.all(dq == 0.0)
    V = 4096
    q, p, g = inputs.kl_pair(8, V, "f32", workload=34)
    q[:, V // 2:] = -np.inf
    p[:, : V // 2] = -np.inf
    js, *_ = run(q, p, g, "f32")
    np.testing.assert_allclose(js, LN2, rtol=0, atol=2e-6)


def test_infinite_entries():
    q, p, g = inputs.kl_pair(8, 300, "f32", workload=35)
    p[0, :150] = -np.inf           # teacher mass on half the row
    q[1, 7] = -np.inf              # student zero where the teacher has mass: still finite
    p[2, :] = -np.inf              # no teacher softmax: NaN
    q[3, :] = -np.inf              # no student softmax: NaN
    q[4, 5] = np.inf               # +inf logit: NaN
    js, _, _, _, dq = run(q, p, g, "f32")
    zq, zp = decode(q, "f32"), decode(p, "f32")
    rj, *_ = ojs.forward(zq, zp)
    check_val(js, rj, "f32", "js")
    assert np.isfinite(js[[0, 1, 5, 6, 7]]).all() and np.isnan(js[[2, 3, 4]]).all()
    ok = [0, 1, 5, 6, 7]
    check_dq(dq[ok], zq[ok], zp[ok], g[ok], "f32")


def test_strided_views_and_in_place():
    """q and p as [B, L - 1, V] views of larger tensors (V past the chunking threshold);
    the VJP in place on q."""
    B, L, V = 3, 7, 9001
    q, p, g = inputs.kl_pair(B * L, V, "f32", workload=36)
    qd = to_dev(q, "f32").view(B, L, V)
    pd = to_dev(p, "f32").view(B, L, V)
    qv, pv = qd[:, :-1], pd[:, 1:]
    n = B * (L - 1)
    gd = torch.from_numpy(np.linspace(0.5, 1.5, n).astype(np.float32)).cuda()
    js, lq, lp, hq = abi.js_forward(qv, pv)
    ref_q = decode(q, "f32").reshape(B, L, V)[:, :-1].reshape(n, V)
    ref_p = decode(p, "f32").reshape(B, L, V)[:, 1:].reshape(n, V)
    rj, *_ = ojs.forward(ref_q, ref_p)
    check_val(from_dev(js), rj, "f32", "js")
    expect = abi.js_vjp(qv, pv, lq, lp, hq, gd, lanes_per_row=1024)
    before = qd.clone()
    abi.js_vjp(qv, pv, lq, lp, hq, gd, dq=qv)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(qv), from_dev(expect))
    assert torch.equal(qd[:, -1], before[:, -1])
    check_dq(from_dev(qv).reshape(n, V), ref_q, ref_p, gd.cpu().numpy(), "f32")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_misaligned_and_other_phase(dtype):
    """p starting off a 16-byte boundary (element path), and a gradient written to a view
    in another 16-byte phase, on rows long enough for the chunked VJP."""
    V = 20003
    q, p, g = inputs.kl_pair(19, V, dtype, workload=37)
    qd = to_dev(q, dtype)
    big = torch.empty(19 * V + 3, dtype=TORCH_DT[dtype], device="cuda")
    pd = big[3:].view(19, V)
    pd.copy_(to_dev(p, dtype))
    js, lq, lp, hq = abi.js_forward(qd, pd)
    gd = torch.from_numpy(g).cuda()
    dq = abi.js_vjp(qd, pd, lq, lp, hq, gd)
    out = torch.empty(19, V + 1, dtype=TORCH_DT[dtype], device="cuda")[:, 1:]
    dq2 = abi.js_vjp(qd, to_dev(p, dtype), lq, lp, hq, gd, dq=out)
    torch.cuda.synchronize()
    zq, zp = decode(q, dtype), decode(p, dtype)
    rj, *_ = ojs.forward(zq, zp)
    check_val(from_dev(js), rj, dtype, "js")
    check_dq(from_dev(dq), zq, zp, g, dtype)
    check_dq(from_dev(dq2), zq, zp, g, dtype)
