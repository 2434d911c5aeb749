"""GPU parity of kl_forward / kl_vjp against the float64 oracle.

Tolerances.  The (m, log s) pairs follow tests/gpu_util.py (as for the cross-entropy).
The KL value is a difference of row terms of its own size (t / s_p against the two
log-sum-exps), so for float32 inputs it is held to |kl - ref| <= 1e-5 (1 + |ref|), ten
times tighter than the 1e-4 relative check of "One barrier short", Run it yourself;
for 16-bit inputs to 1e-3 |ref| + 1e-5.  A gradient entry g (Q_j - P_j) is a
difference of two probabilities, each computed in float32 with a relative error of a
few 1e-6 (the rounding of the exponent's argument, up to |x| 2^-24 for |x| ~ 100), so
where Q_j ~ P_j the difference keeps only an absolute accuracy of about
1e-5 g (Q_j + P_j).  The gradient rule of tests/gpu_util.py (1e-5 absolute for
float32; max(1e-3 |ref|, one ulp) for 16-bit outputs) is widened by that term.
"""

import numpy as np
import pytest
import torch

from oracle import kl as okl
from softmax_cross_entropy_amd import abi, inputs
from tests.gpu_util import TORCH_DT, decode, from_dev, to_dev, ulp16

pytestmark = pytest.mark.gpu


def check_kl(got, ref, dtype):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(ref)), "kl: NaN pattern differs"
    inf = np.isinf(ref)
    assert np.array_equal(got[inf], ref[inf]), "kl: infinities differ"
    ok = np.isfinite(ref)
    tol = 1e-5 * (1 + np.abs(ref[ok])) if dtype == "f32" else 1e-3 * np.abs(ref[ok]) + 1e-5
    err = np.abs(got[ok] - ref[ok])
    assert np.all(err <= tol), f"kl: {np.sum(err > tol)} rows off, worst {err.max():.3e} at ref {ref[ok][np.argmax(err - tol)]:.4f}"
    return float(err.max()) if err.size else 0.0


def check_dq(got_store, zq, zp, g, dtype):
    ref = okl.grad(zq, zp, g)
    got = decode(got_store, dtype)
    assert np.array_equal(np.isnan(got), np.isnan(ref)), "dq: NaN pattern differs"
    ok = ~np.isnan(ref)
    with np.errstate(invalid="ignore", over="ignore"):
        mass = np.exp(okl.log_softmax(zq)) + np.exp(okl.log_softmax(zp))
    cancel = 1e-5 * np.abs(np.asarray(g, np.float64))[:, None] * mass
    base = np.full_like(ref, 1e-5) if dtype == "f32" else np.maximum(1e-3 * np.abs(ref), ulp16(ref, dtype))
    tol = base + cancel
    err = np.abs(got - ref)
    bad = ok & (err > tol)
    assert not bad.any(), (f"dq: {bad.sum()} elements off; first at {np.argwhere(bad)[0]}: "
                           f"got {got[bad][0]!r} ref {ref[bad][0]!r} tol {tol[bad][0]!r}")


def run(q, p, g, dtype, lanes=0, dq_out=None):
    qd, pd = to_dev(q, dtype), to_dev(p, dtype)
    kl, lq, lp = abi.kl_forward(qd, pd, lanes_per_row=lanes)
    dq = abi.kl_vjp(qd, pd, lq, lp, torch.from_numpy(np.asarray(g, np.float32)).cuda(), dq=dq_out,
                    lanes_per_row=lanes)
    torch.cuda.synchronize()
    return (kl.cpu().numpy().astype(np.float64), lq.cpu().numpy().astype(np.float64),
            lp.cpu().numpy().astype(np.float64), from_dev(dq))


def full_check(q, p, g, dtype, lanes=0):
    kl, lq, lp, dq = run(q, p, g, dtype, lanes)
    zq, zp = decode(q, dtype), decode(p, dtype)
    rk, mq, lsq, mp, lsp = okl.forward(zq, zp)
    e = check_kl(kl, rk, dtype)
    fin = np.isfinite(mq)
    assert np.array_equal(lq[fin, 0], mq[fin]) and np.array_equal(lp[np.isfinite(mp), 0], mp[np.isfinite(mp)])
    check_dq(dq, zq, zp, g, dtype)
    return kl, dq, e


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_barrier_regression_shape_and_repeat(dtype):
    """128 x 151,936 ("One barrier short", The fix: the regression test's shape), then ten
    more calls bit-identical to the first."""
    q, p, g = inputs.kl_pair(128, 151936, dtype, scale=4.0 if dtype != "f16" else 2.0)
    kl, dq, e = full_check(q, p, g, dtype)
    print(f"{dtype}: max |dkl| {e:.2e}")
    for _ in range(10):
        k2, _, _, d2 = run(q, p, g, dtype)
        assert np.array_equal(k2.view(np.uint64), kl.view(np.uint64))
        assert np.array_equal(d2, dq)


def test_run_it_yourself_shape():
    """512 x 151,936 fp32 at scale 4, as the page's reproduction draws it."""
    q, p, g = inputs.kl_pair(512, 151936, "f32", scale=4.0, workload=21)
    _, _, e = full_check(q, p, g, "f32")
    print(f"max |dkl| {e:.2e}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_boundary_sizes_all_lane_counts(dtype):
    for V in (1, 2, 7, 8, 9, 63, 64, 65, 1000, 1024, 4097):
        q, p, g = inputs.kl_pair(67, V, dtype, workload=22, stream=V)
        g = np.linspace(0.5, 2.0, 67).astype(np.float32)
        for lanes in (0, 1, 4, 16, 64, 128, 1024):
            full_check(q, p, g, dtype, lanes)


def test_identical_rows_give_zero():
    q, _, g = inputs.kl_pair(64, 5000, "f32", workload=23)
    kl, _, _, dq = run(q, q, g, "f32")
    assert np.all(kl == 0.0)
    assert np.all(dq == 0.0)


def test_infinite_entries():
    q, p, g = inputs.kl_pair(8, 300, "f32", workload=24)
    p[0, :150] = -np.inf           # teacher mass on half the row
    p[1, 7] = -np.inf              # one empty teacher column
    q[2, 11] = -np.inf             # student -inf under teacher mass: +inf
    p[3, :] = -np.inf              # no teacher mass: NaN
    q[4, 5] = np.inf               # +inf logit: NaN
    kl, _, _, dq = run(q, p, g, "f32")
    zq, zp = decode(q, "f32"), decode(p, "f32")
    rk, *_ = okl.forward(zq, zp)
    check_kl(kl, rk, "f32")
    assert kl[2] == np.inf and np.isnan(kl[3]) and np.isnan(kl[4])
    ok = [0, 1, 5, 6, 7]
    check_dq(dq[ok], zq[ok], zp[ok], g[ok], "f32")


def test_strided_views_and_in_place():
    """q and p as [B, L - 1, V] views of larger tensors; the VJP in place on q."""
    B, L, V = 4, 9, 4096
    q, p, g = inputs.kl_pair(B * L, V, "f32", workload=25)
    qd = to_dev(q, "f32").view(B, L, V)
    pd = to_dev(p, "f32").view(B, L, V)
    qv, pv = qd[:, :-1], pd[:, 1:]
    n = B * (L - 1)
    gd = torch.from_numpy(np.linspace(0.5, 1.5, n).astype(np.float32)).cuda()
    kl, lq, lp = abi.kl_forward(qv, pv)
    ref_q = decode(q, "f32").reshape(B, L, V)[:, :-1].reshape(n, V)
    ref_p = decode(p, "f32").reshape(B, L, V)[:, 1:].reshape(n, V)
    rk, *_ = okl.forward(ref_q, ref_p)
    check_kl(kl.cpu().numpy(), rk, "f32")
    before = qd.clone()
    abi.kl_vjp(qv, pv, lq, lp, gd, dq=qv)
    torch.cuda.synchronize()
    check_dq(qv.reshape(n, V).cpu().numpy(), ref_q, ref_p, gd.cpu().numpy(), "f32")
    assert torch.equal(qd[:, -1], before[:, -1])  # the row outside the view is untouched


def test_misaligned_rows_take_the_scalar_path():
    q, p, g = inputs.kl_pair(33, 1001, "bf16", workload=26)
    qd = to_dev(q, "bf16")
    big = torch.empty(33 * 1001 + 3, dtype=torch.bfloat16, device="cuda")
    pd = big[3:].view(33, 1001)
    pd.copy_(to_dev(p, "bf16"))
    kl, lq, lp = abi.kl_forward(qd, pd)
    dq = abi.kl_vjp(qd, pd, lq, lp, torch.ones(33, device="cuda"))
    torch.cuda.synchronize()
    zq, zp = decode(q, "bf16"), decode(p, "bf16")
    rk, *_ = okl.forward(zq, zp)
    check_kl(kl.cpu().numpy(), rk, "bf16")
    check_dq(from_dev(dq), zq, zp, np.ones(33), "bf16")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunked_vjp_phases(dtype):
    """Rows of at least 2048 16-byte vectors take the chunked VJP layout by default:
    against the oracle and, bit for bit, against one workgroup per row, with q starting
    0, 1 or 3 elements off a 16-byte boundary, p and dq in the same or another phase."""
    Vs = [8189, 10243] if dtype == "f32" else [16377, 20483]
    for V in Vs:
        for shift in (0, 1, 3):
            q, p, g = inputs.kl_pair(19, V + 4, dtype, workload=27, stream=V + shift)
            g = np.linspace(-1.0, 2.0, 19).astype(np.float32)
            qd = to_dev(q, dtype)[:, shift:shift + V]
            zq = decode(q, dtype)[:, shift:shift + V]
            for pshift in (shift, 2):
                pd = to_dev(p, dtype)[:, pshift:pshift + V]
                zp = decode(p, dtype)[:, pshift:pshift + V]
                kl, lq, lp = abi.kl_forward(qd, pd)
                gd = torch.from_numpy(g).cuda()
                dq = abi.kl_vjp(qd, pd, lq, lp, gd)
                rows = abi.kl_vjp(qd, pd, lq, lp, gd, lanes_per_row=1024)
                out = torch.empty(19, V + 1, dtype=TORCH_DT[dtype], device="cuda")[:, 1:]
                dq2 = abi.kl_vjp(qd, pd, lq, lp, gd, dq=out)
                torch.cuda.synchronize()
                rk, *_ = okl.forward(zq, zp)
                check_kl(kl.cpu().numpy(), rk, dtype)
                check_dq(from_dev(dq), zq, zp, g, dtype)
                check_dq(from_dev(dq2), zq, zp, g, dtype)
                assert np.array_equal(from_dev(dq), from_dev(rows))
                assert np.array_equal(from_dev(dq2), from_dev(rows))


def test_chunked_vjp_in_place_strided():
    B, L, V = 3, 7, 9001
    q, p, g = inputs.kl_pair(B * L, V, "f32", workload=28)
    qd = to_dev(q, "f32").view(B, L, V)
    pd = to_dev(p, "f32").view(B, L, V)
    qv, pv = qd[:, :-1], pd[:, 1:]
    n = B * (L - 1)
    gd = torch.from_numpy(np.linspace(0.5, 1.5, n).astype(np.float32)).cuda()
    kl, lq, lp = abi.kl_forward(qv, pv)
    expect = abi.kl_vjp(qv, pv, lq, lp, gd, lanes_per_row=1024)
    before = qd.clone()
    abi.kl_vjp(qv, pv, lq, lp, gd, dq=qv)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(qv), from_dev(expect))
    assert torch.equal(qd[:, -1], before[:, -1])
    ref_q = decode(q, "f32").reshape(B, L, V)[:, :-1].reshape(n, V)
    ref_p = decode(p, "f32").reshape(B, L, V)[:, 1:].reshape(n, V)
    check_dq(from_dev(qv).reshape(n, V), ref_q, ref_p, gd.cpu().numpy(), "f32")
