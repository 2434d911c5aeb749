"""GPU parity of the cross-entropy options against the float64 oracle (oracle/ce_options.py).

Calls go through the C ABI: ce_forward_ex / ce_vjp_ex (class-index targets with label
smoothing, ignore_index and the sum / mean reductions) and ce_forward_probs /
ce_vjp_probs (probability targets).

Tolerances.  Per-row losses: |loss - ref| <= 1e-5 (1 + |ref|) for float32 logits (the
smoothing term adds the mean logit, a float32 sum of V terms, so the absolute 1e-5 of
the plain loss is widened by the loss's own size) and 1e-3 |ref| + 1e-5 for 16-bit
logits.  A reduced total sums the per-row losses in float64, so it may move by the sum
of the per-row allowances (divided by the count for a mean) plus one float32 rounding.
Gradients: the rule of tests/gpu_util.py plus 1e-5 |g| (W p + |w|).  An entry
g (W p_j - w_j) is a difference of two terms computed in float32 with relative errors of
a few 1e-7; where W p_j ~ w_j only that absolute accuracy remains.
"""

import math

import numpy as np
import pytest
import torch

from oracle import ce as oce
from oracle import ce_options as oco
from softmax_cross_entropy_amd import abi, inputs
from tests.gpu_util import TORCH_DT, decode, from_dev, to_dev, ulp16

pytestmark = pytest.mark.gpu

EPS = (0.0, 0.1, 0.5)
REDUCTIONS = ("none", "sum", "mean")


def loss_tol(ref, dtype):
    a = np.abs(ref)
    return 1e-5 * (1 + a) if dtype == "f32" else 1e-3 * a + 1e-5


def check_rows(got, ref, dtype, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(ref)), f"{what}: NaN pattern differs"
    inf = np.isinf(ref)
    assert np.array_equal(got[inf], ref[inf]), f"{what}: infinities differ"
    ok = np.isfinite(ref)
    err = np.abs(got[ok] - ref[ok])
    tol = loss_tol(ref[ok], dtype)
    bad = err > tol
    assert not bad.any(), f"{what}: {bad.sum()} rows off; worst {(err - tol).max():.3e}"


def check_total(got, ref_rows, counted, reduction, dtype, count_ref):
    if reduction == "none":
        return
    allow = float(np.sum(np.where(counted & np.isfinite(ref_rows), loss_tol(ref_rows, dtype), 0.0)))
    ref_sum = float(np.sum(np.where(counted, ref_rows, 0.0)))
    if reduction == "mean":
        if count_ref == 0:
            assert math.isnan(got)
            return
        ref, allow = ref_sum / count_ref, allow / count_ref
    else:
        ref = ref_sum
    if not math.isfinite(ref):
        assert (math.isnan(ref) and math.isnan(got)) or got == ref
        return
    assert abs(got - ref) <= allow + 2.0 ** -23 * abs(ref), (got, ref, allow)


def check_opt_grad(got_store, ref, z, w, gi, dtype, what):
    got = decode(got_store, dtype)
    assert np.array_equal(np.isnan(got), np.isnan(ref)), f"{what}: NaN pattern differs"
    ok = ~np.isnan(ref)
    with np.errstate(invalid="ignore", over="ignore"):
        m = oce.row_max(z)
        p = np.exp((z - m[:, None]) - oce.row_log_sum(z, m)[:, None])
        cancel = 1e-5 * np.abs(gi)[:, None] * (np.abs(w.sum(axis=1))[:, None] * p + np.abs(w))
    base = np.full_like(ref, 1e-5) if dtype == "f32" else np.maximum(1e-3 * np.abs(ref), ulp16(ref, dtype))
    tol = np.where(ok, base + np.nan_to_num(cancel), 0)
    err = np.abs(got - ref)
    bad = ok & (err > tol)
    assert not bad.any(), (f"{what}: {bad.sum()} elements off; first at {np.argwhere(bad)[0]}: "
                           f"got {got[bad][0]!r} ref {ref[bad][0]!r} tol {tol[bad][0]!r}")


def upstream(reduction, n, seed):
    if reduction == "none":
        return np.random.default_rng(seed).uniform(0.25, 2.0, n).astype(np.float32)
    return np.array([1.75], np.float32)


def run_index(x, y, g, eps, ign, red, dtype):
    xd = to_dev(x, dtype) if isinstance(x, np.ndarray) else x
    yd = torch.from_numpy(np.ascontiguousarray(y, np.int32)).cuda()
    loss, lse, total, count = abi.ce_forward_ex(xd, yd, eps, ign, red)
    d = abi.ce_vjp_ex(xd, yd, lse, torch.from_numpy(g).cuda(), eps, ign, red, count=count)
    torch.cuda.synchronize()
    return (from_dev(loss), from_dev(lse), None if total is None else float(total.item()),
            None if count is None else int(count.item()), from_dev(d))


def full_index_check(x, y, eps, ign, red, dtype, z=None, seed=0):
    n = len(y)
    g = upstream(red, n, seed)
    loss, lse, total, count, d = run_index(x, y, g, eps, ign, red, dtype)
    z = decode(x, dtype) if z is None else z
    rl, rm, rls, rt, rc = oco.forward_index(z, y, eps, ign, red)
    check_rows(loss, rl, dtype, f"loss eps={eps} ign={ign} red={red}")
    fin = np.isfinite(rm)
    assert np.array_equal(lse[fin, 0], rm[fin])
    w, counted = oco.index_weights(y, z.shape[1], eps, ign)
    if red != "none":
        assert count == rc
        check_total(total, rl, counted, red, dtype, rc)
    gi = oco.row_upstream(g if red == "none" else g[0], counted, red, rc)
    check_opt_grad(d, oco.grad_index(z, y, g if red == "none" else g[0], eps, ign, red), z, w, gi, dtype,
                   f"dlogits eps={eps} ign={ign} red={red}")
    return loss, total, d


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_index_targets_all_options(dtype):
    """Every smoothing, ignore_index (none, -100, an in-range class) and reduction, on
    rows short and long, with -inf entries and a target at -inf."""
    for V in (1, 7, 64, 1000, 4097, 16389):
        b = inputs.normal_rows(37, V, dtype, workload=40, stream=V)
        x = b.logits.copy()
        y = b.targets.copy()
        if V > 3:
            x[1, : V // 2] = -np.inf if dtype != "bf16" else np.uint16(0xFF80)
            y[1] = V - 1
            x[2, y[2]] = -np.inf if dtype != "bf16" else np.uint16(0xFF80)
        y_ign = y.copy()
        y_ign[[0, 5, 9]] = -100
        y_in = y.copy()
        cls = min(3, V - 1)
        y_in[[4, 6]] = cls
        for eps in EPS:
            for red in REDUCTIONS:
                for yy, ign in ((y, None), (y_ign, -100), (y_in, cls)):
                    full_index_check(x, yy, eps, ign, red, dtype, seed=V)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_probability_targets(dtype):
    """Normalised and unnormalised targets, zero targets at -inf logits, every smoothing
    and reduction, rows short and long."""
    for V in (1, 9, 300, 4100, 20001):
        rows = 29
        b = inputs.normal_rows(rows, V, dtype, workload=41, stream=V)
        x = b.logits.copy()
        ts = inputs.prob_targets(rows, V, dtype, workload=41, stream=V + 1, normalised_rows=rows // 2)
        if V > 3:
            x[3, :2] = -np.inf if dtype != "bf16" else np.uint16(0xFF80)
            ts[3, :2] = 0
        zt = decode(ts, dtype)
        z = decode(x, dtype)
        for eps in EPS:
            for red in REDUCTIONS:
                g = upstream(red, rows, V)
                xd, td = to_dev(x, dtype), to_dev(ts, dtype)
                loss, lse, wsum, total, count = abi.ce_forward_probs(xd, td, eps, red)
                d = abi.ce_vjp_probs(xd, td, lse, wsum, torch.from_numpy(g).cuda(), eps, red, count=count)
                torch.cuda.synchronize()
                rl, rm, rls, rW, rt, rc = oco.forward_probs(z, zt, eps, red)
                check_rows(from_dev(loss), rl, dtype, f"loss V={V} eps={eps} red={red}")
                np.testing.assert_allclose(from_dev(wsum), rW, rtol=2e-6, atol=1e-7)
                counted = np.ones(rows, bool)
                if red != "none":
                    assert int(count.item()) == rows
                    check_total(float(total.item()), rl, counted, red, dtype, rows)
                gg = g if red == "none" else g[0]
                gi = oco.row_upstream(gg, counted, red, rows)
                check_opt_grad(from_dev(d), oco.grad_probs(z, zt, gg, eps, red), z, oco.prob_weights(zt, eps), gi,
                               dtype, f"dlogits V={V} eps={eps} red={red}")


def test_eps_zero_matches_the_plain_calls_bit_for_bit():
    b = inputs.normal_rows(300, 5000, "bf16", workload=42)
    xd = to_dev(b.logits, "bf16")
    yd = torch.from_numpy(b.targets).cuda()
    g = torch.from_numpy(np.linspace(0.5, 1.5, 300).astype(np.float32)).cuda()
    l0, s0 = abi.ce_forward(xd, yd)
    d0 = abi.ce_vjp(xd, yd, s0, g)
    l1, s1, _, _ = abi.ce_forward_ex(xd, yd, 0.0, None, "none")
    d1 = abi.ce_vjp_ex(xd, yd, s1, g, 0.0, None, "none")
    # ignore_index that matches nothing takes the options VJP kernel: same bits
    d2 = abi.ce_vjp_ex(xd, yd, s1, g, 0.0, -100, "none")
    torch.cuda.synchronize()
    assert torch.equal(l0, l1) and torch.equal(s0, s1) and torch.equal(d0, d1) and torch.equal(d0, d2)


def test_strided_views_misaligned_and_in_place():
    """[B, L - 1, V] views for logits and probability targets, a view off a 16-byte
    boundary, and the VJP written in place over the logits."""
    B, L, V = 3, 7, 9001
    x, y = inputs.strided_view_source(B, L, V)
    yv = inputs.shifted_targets(y)
    n = B * (L - 1)
    X = torch.from_numpy(x).cuda()
    view = X[:, :-1]
    z = decode(np.ascontiguousarray(x[:, :-1]).reshape(n, V), "f32")
    yd = torch.from_numpy(yv).cuda()
    loss, lse, total, count = abi.ce_forward_ex(view, yd, 0.1, -100, "mean")
    rl, *_ = oco.forward_index(z, yv, 0.1, -100, "mean")
    check_rows(from_dev(loss), rl, "f32", "strided loss")
    g = torch.tensor([2.0], device="cuda")
    expect = abi.ce_vjp_ex(view, yd, lse, g, 0.1, -100, "mean", count=count)
    abi.ce_vjp_ex(view, yd, lse, g, 0.1, -100, "mean", count=count, dlogits=view)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(view), from_dev(expect))
    assert np.array_equal(from_dev(X[:, -1]), x[:, -1])
    w, counted = oco.index_weights(yv, V, 0.1, -100)
    gi = oco.row_upstream(2.0, counted, "mean", n)
    check_opt_grad(from_dev(expect).reshape(n, V), oco.grad_index(z, yv, 2.0, 0.1, -100, "mean"), z, w, gi, "f32",
                   "strided dlogits")
    # probability targets through a view that starts 1 element off a 16-byte boundary
    t = inputs.prob_targets(n, V + 1, "f32", workload=45)
    T = torch.from_numpy(t).cuda()
    tv = T[:, 1:]
    zs = torch.from_numpy(np.ascontiguousarray(z.astype(np.float32))).cuda()
    loss, lse, wsum, _, _ = abi.ce_forward_probs(zs, tv, 0.1, "none")
    rl, *_ = oco.forward_probs(z, t[:, 1:].astype(np.float64), 0.1)
    check_rows(from_dev(loss), rl, "f32", "misaligned probs loss")
    gg = torch.ones(n, device="cuda")
    d = abi.ce_vjp_probs(zs, tv, lse, wsum, gg, 0.1, "none")
    torch.cuda.synchronize()
    wt = oco.prob_weights(t[:, 1:].astype(np.float64), 0.1)
    check_opt_grad(from_dev(d), oco.grad_probs(z, t[:, 1:].astype(np.float64), np.ones(n), 0.1), z, wt, np.ones(n),
                   "f32", "misaligned probs dlogits")


def test_out_of_range_target_is_a_nan_row():
    b = inputs.normal_rows(40, 300, "f32", workload=46)
    y = b.targets.copy()
    y[[3, 8]] = [300, -5]
    y[11] = -100
    xd = to_dev(b.logits, "f32")
    yd = torch.from_numpy(y).cuda()
    loss, lse, total, count = abi.ce_forward_ex(xd, yd, 0.1, -100, "sum")
    d = abi.ce_vjp_ex(xd, yd, lse, torch.ones(1, device="cuda"), 0.1, -100, "sum", count=count)
    torch.cuda.synchronize()
    l, dd = from_dev(loss), from_dev(d)
    assert np.isnan(l[[3, 8]]).all() and l[11] == 0.0 and np.isfinite(np.delete(l, [3, 8])).all()
    assert np.isnan(dd[[3, 8]]).all() and np.all(dd[11] == 0.0)
    assert math.isnan(float(total.item())) and int(count.item()) == 39
    rl, *_ = oco.forward_index(decode(b.logits, "f32"), y, 0.1, -100)
    check_rows(l, rl, "f32", "loss")


def test_every_row_ignored_and_empty_batch():
    b = inputs.normal_rows(50, 700, "f32", workload=43)
    xd = to_dev(b.logits, "f32")
    y = torch.full((50,), -100, dtype=torch.int32, device="cuda")
    loss, lse, total, count = abi.ce_forward_ex(xd, y, 0.1, -100, "mean")
    d = abi.ce_vjp_ex(xd, y, lse, torch.ones(1, device="cuda"), 0.1, -100, "mean", count=count)
    torch.cuda.synchronize()
    assert int(count.item()) == 0 and math.isnan(float(total.item()))
    assert torch.all(loss == 0).item() and torch.all(d == 0).item()
    e = torch.empty(0, 700, device="cuda")
    t = torch.empty(0, dtype=torch.int32, device="cuda")
    for red, want in (("sum", 0.0), ("mean", float("nan"))):
        total = torch.full((1,), 7.0, device="cuda")
        count = torch.full((1,), 7, dtype=torch.int64, device="cuda")
        abi.ce_forward_ex(e, t, 0.1, -100, red, total=total, count=count)
        torch.cuda.synchronize()
        got = float(total.item())
        assert int(count.item()) == 0 and (got == want or (math.isnan(want) and math.isnan(got)))


def test_repeat_is_bitwise_stable():
    b = inputs.normal_rows(700, 33000, "bf16", workload=44)
    xd = to_dev(b.logits, "bf16")
    y = b.targets.copy()
    y[::7] = -100
    yd = torch.from_numpy(y).cuda()
    g = torch.tensor([1.0], device="cuda")
    outs = []
    for _ in range(4):
        loss, lse, total, count = abi.ce_forward_ex(xd, yd, 0.1, -100, "mean")
        d = abi.ce_vjp_ex(xd, yd, lse, g, 0.1, -100, "mean", count=count)
        torch.cuda.synchronize()
        outs.append((from_dev(loss), from_dev(total), from_dev(d)))
    for o in outs[1:]:
        for a, b_ in zip(o, outs[0]):
            assert np.array_equal(a.view(np.uint8), b_.view(np.uint8))


def test_large_vocab_bf16_mean_sampled():
    """2048 x 151,936 bf16 with eps = 0.1, ignore_index on every 16th row and a mean: the
    total against the oracle over all rows (in chunks), the gradient on sampled rows."""
    rows, V = 2048, 151936
    b = inputs.large_vocab(rows, V)
    y = b.targets.copy()
    y[::16] = -100
    xd = to_dev(b.logits, "bf16")
    yd = torch.from_numpy(y).cuda()
    loss, lse, total, count = abi.ce_forward_ex(xd, yd, 0.1, -100, "mean")
    g = torch.tensor([3.0], device="cuda")
    d = abi.ce_vjp_ex(xd, yd, lse, g, 0.1, -100, "mean", count=count)
    torch.cuda.synchronize()
    ref = np.empty(rows)
    for r0 in range(0, rows, 256):
        z = decode(b.logits[r0:r0 + 256], "bf16")
        ref[r0:r0 + 256], *_ = oco.forward_index(z, y[r0:r0 + 256], 0.1, -100)
    check_rows(from_dev(loss), ref, "bf16", "loss")
    counted = y != -100
    assert int(count.item()) == int(counted.sum())
    check_total(float(total.item()), ref, counted, "mean", "bf16", int(counted.sum()))
    sample = np.unique(np.concatenate([[0, 1, 16, rows - 1], np.random.default_rng(0).choice(rows, 24, False)]))
    z = decode(b.logits[sample], "bf16")
    w, c = oco.index_weights(y[sample], V, 0.1, -100)
    gi = np.where(c, 3.0 / counted.sum(), 0.0)
    refd = oco.weighted_grad(z, w, gi, c)
    check_opt_grad(from_dev(d)[sample], refd, z, w, gi, "bf16", "dlogits")
