"""Pins for the cross-entropy options oracle (oracle/ce_options.py), CPU only.

Source of the options: MLX PR #4188 "Shift by the max in cross_entropy", Proposed
changes (label smoothing 0, 0.1 and 0.5, probability targets, the three reductions, and
the gradients, all checked against PyTorch; every magnitude from 1e0 to 1e36).  The
pins below fix the oracle to closed forms, PyTorch's float64 cross_entropy and its
autograd, a 50-digit brute force without the max shift, and invariants; planted
mistakes at the end must each fail at least one of them.
"""

import contextlib
import math

import mpmath
import numpy as np
import scipy.special
import torch
import torch.nn.functional as F

from oracle import ce as oce
from oracle import ce_options as oco
from tests import golden_io

LOG2 = math.log(2.0)
EPS = (0.0, 0.1, 0.5)


def f32_rows(rows):
    return oce.decode(np.asarray(rows, np.float64).astype(np.float32), "f32")


def rand_rows(rows, V, seed, scale=3.0):
    return np.random.default_rng(seed).normal(0.0, scale, (rows, V))


def rand_probs(rows, V, seed, normalised=True):
    t = np.random.default_rng(seed).uniform(0.0, 1.0, (rows, V))
    return t / t.sum(axis=1, keepdims=True) if normalised else t


# --- PyTorch float64 cross_entropy and autograd ---------------------------------

def torch_index(z, y, g, eps, ignore_index, reduction):
    zt = torch.tensor(z, dtype=torch.float64, requires_grad=True)
    kw = {} if ignore_index is None else {"ignore_index": int(ignore_index)}
    loss = F.cross_entropy(zt, torch.tensor(y, dtype=torch.int64), reduction=reduction, label_smoothing=eps, **kw)
    (loss * torch.tensor(g, dtype=torch.float64)).sum().backward()
    return loss.detach().numpy(), zt.grad.numpy()


def torch_probs(z, t, g, eps, reduction):
    zt = torch.tensor(z, dtype=torch.float64, requires_grad=True)
    loss = F.cross_entropy(zt, torch.tensor(t, dtype=torch.float64), reduction=reduction, label_smoothing=eps)
    (loss * torch.tensor(g, dtype=torch.float64)).sum().backward()
    return loss.detach().numpy(), zt.grad.numpy()


def pin_torch():
    rows, V = 13, 37
    z = rand_rows(rows, V, 1)
    y = np.random.default_rng(2).integers(0, V, rows)
    y_ign = y.copy()
    y_ign[[2, 5, 11]] = -100
    y_in = y.copy()
    y_in[[1, 4]] = 7  # an in-range ignore_index
    gr = np.random.default_rng(3).uniform(0.5, 2.0, rows)
    for eps in EPS:
        for red in oco.REDUCTIONS:
            g = gr if red == "none" else np.float64(1.75)
            for yy, ign in ((y, None), (y_ign, -100), (y_in, 7)):
                tl, tg = torch_index(z, yy, g, eps, ign, red)
                loss, _, _, total, _ = oco.forward_index(z, yy, eps, ign, red)
                got = loss if red == "none" else total
                np.testing.assert_allclose(got, tl, rtol=1e-12, atol=1e-13)
                np.testing.assert_allclose(oco.grad_index(z, yy, g, eps, ign, red), tg, rtol=1e-12, atol=1e-14)
            for norm in (True, False):
                t = rand_probs(rows, V, 4, norm)
                tl, tg = torch_probs(z, t, g, eps, red)
                loss, _, _, _, total, _ = oco.forward_probs(z, t, eps, red)
                got = loss if red == "none" else total
                np.testing.assert_allclose(got, tl, rtol=1e-12, atol=1e-13)
                np.testing.assert_allclose(oco.grad_probs(z, t, g, eps, red), tg, rtol=1e-12, atol=1e-14)


def test_matches_torch():
    pin_torch()


# --- the page's magnitudes -------------------------------------------------------

def pin_equal_logits(g=1.5):
    """[v, v] at every magnitude the page checks: log 2 for any smoothing and for any
    probability target summing to 1; gradient g (W/2 - w)."""
    gold = golden_io.read("shift_by_max.txt")
    values = tuple(gold["equal_values"]) + (gold["equal_checked_max"],)
    z = f32_rows([[v, v] for v in values])
    n = len(values)
    for eps in EPS:
        loss, m, ls, _, _ = oco.forward_index(z, np.zeros(n, np.int32), eps)
        np.testing.assert_allclose(loss, LOG2, rtol=0, atol=1e-15)
        d = oco.grad_index(z, np.zeros(n, np.int32), np.full(n, g), eps)
        w0 = (1 - eps) + eps / 2
        np.testing.assert_allclose(d, np.tile([g * (0.5 - w0), g * (0.5 - (1 - w0))], (n, 1)), atol=1e-15)
        for t0 in (1.0, 0.5, 0.25):
            t = np.tile([t0, 1 - t0], (n, 1))
            loss, *_ = oco.forward_probs(z, t, eps)
            np.testing.assert_allclose(loss, LOG2, rtol=0, atol=1e-15)


def test_equal_logits_every_magnitude():
    pin_equal_logits()


def pin_gap_rows():
    """[2 + c, -1 + c], target 0: the stored gap is 3 at c = 0, 1e4, 1e6, so the loss is
    log(1 + e^-3) + 1.5 eps (the mean logit sits 1.5 below the target); at c = 1e8 float32
    storage makes the two logits equal and the loss is log 2."""
    gold = golden_io.read("shift_by_max.txt")
    offs = gold["gap_offsets"]
    z = f32_rows([[2.0 + c, -1.0 + c] for c in offs])
    y = np.zeros(len(offs), np.int32)
    base = math.log1p(math.exp(-3.0))
    for eps in EPS:
        loss, *_ = oco.forward_index(z, y, eps)
        want = [base + 1.5 * eps if c < 1e8 else LOG2 for c in offs]
        np.testing.assert_allclose(loss, want, rtol=0, atol=2e-15)


def test_gap_rows():
    pin_gap_rows()


# --- closed forms ------------------------------------------------------------------

def pin_uniform_rows(g=0.75):
    """A row of V equal logits: loss = log V whatever the smoothing or the (normalised)
    probability target, gradient g (1/V - w)."""
    for V in (1, 8, 1024, 151936):
        z = np.full((2, V), 3.25)
        y = np.array([0, V - 1])
        t = np.zeros((2, V))
        t[0, 0] = 1.0
        t[1] = 1.0 / V
        for eps in EPS:
            loss, *_ = oco.forward_index(z, y, eps)
            np.testing.assert_allclose(loss, math.log(V), rtol=1e-14, atol=1e-15)
            lp, *_ = oco.forward_probs(z, t, eps)
            np.testing.assert_allclose(lp, math.log(V), rtol=1e-14, atol=1e-15)
            w, _ = oco.index_weights(y, V, eps)
            np.testing.assert_allclose(oco.grad_index(z, y, np.full(2, g), eps), g * (1.0 / V - w), atol=1e-15)


def test_uniform_rows():
    pin_uniform_rows()


def pin_eps_one():
    """eps = 1 makes every weight 1/V: loss = logsumexp(z) - mean(z) for any target."""
    z = rand_rows(9, 23, 5, scale=7.0)
    want = scipy.special.logsumexp(z, axis=1) - z.mean(axis=1)
    loss, *_ = oco.forward_index(z, np.arange(9), 1.0)
    np.testing.assert_allclose(loss, want, rtol=1e-13)
    lp, *_ = oco.forward_probs(z, rand_probs(9, 23, 6, normalised=False), 1.0)
    np.testing.assert_allclose(lp, want, rtol=1e-13)


def test_eps_one():
    pin_eps_one()


def test_eps_zero_is_the_plain_cross_entropy():
    z = rand_rows(40, 300, 7)
    z[3, 10:] = -np.inf
    z[4, 0] = 1e8
    y = np.random.default_rng(8).integers(0, 300, 40)
    y[3] = 2
    loss, m, ls, _, _ = oco.forward_index(z, y, 0.0)
    rl, rm, rls = oce.forward(z, y)
    np.testing.assert_allclose(loss, rl, rtol=1e-13, atol=1e-13)
    assert np.array_equal(m, rm) and np.array_equal(ls, rls)
    g = np.linspace(0.5, 2.0, 40)
    np.testing.assert_allclose(oco.grad_index(z, y, g, 0.0), oce.grad(z, y, g), rtol=1e-13, atol=1e-16)


# --- brute force ---------------------------------------------------------------------

def brute(z, w):
    """50 digits, no max shift: -sum_j w_j log(e^z_j / sum e^z) and W p - w."""
    loss, grads = [], []
    with mpmath.workdps(50):
        for zr, wr in zip(z.tolist(), w.tolist()):
            e = [mpmath.exp(mpmath.mpf(v)) for v in zr]
            s = mpmath.fsum(e)
            p = [x / s for x in e]
            W = mpmath.fsum(mpmath.mpf(x) for x in wr)
            terms = [mpmath.mpf(wj) * mpmath.log(pj) if wj != 0 else mpmath.mpf(0) for wj, pj in zip(wr, p)]
            loss.append(float(-mpmath.fsum(terms)))
            grads.append([float(W * pj - mpmath.mpf(wj)) for wj, pj in zip(wr, p)])
    return np.array(loss), np.array(grads)


def pin_bruteforce():
    for V in (1, 2, 3, 5, 17):
        z = rand_rows(6, V, V, scale=9.0)
        z[1] += 300.0  # a shared offset far past exp's float64 range of the unshifted form
        y = np.random.default_rng(V).integers(0, V, 6)
        t = rand_probs(6, V, V + 1, normalised=(V % 2 == 1))
        for eps in EPS:
            w, _ = oco.index_weights(y, V, eps)
            bl, bg = brute(z, w)
            loss, *_ = oco.forward_index(z, y, eps)
            np.testing.assert_allclose(loss, bl, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(oco.grad_index(z, y, np.ones(6), eps), bg, atol=1e-13)
            w = oco.prob_weights(t, eps)
            bl, bg = brute(z, w)
            lp, *_ = oco.forward_probs(z, t, eps)
            np.testing.assert_allclose(lp, bl, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(oco.grad_probs(z, t, np.ones(6), eps), bg, atol=1e-13)


def test_bruteforce():
    pin_bruteforce()


# --- invariants --------------------------------------------------------------------

def pin_invariants():
    rows, V = 11, 64
    # dyadic logits stay exact under the shared offsets below
    z = np.random.default_rng(9).integers(-40, 40, (rows, V)) / 8.0
    y = np.random.default_rng(10).integers(0, V, rows)
    t = rand_probs(rows, V, 11)
    for eps in EPS:
        a, *_ = oco.forward_index(z, y, eps)
        for c in (1e4, 1e6, -3e5):
            b, *_ = oco.forward_index(z + c, y, eps)
            np.testing.assert_allclose(b, a, rtol=1e-12, atol=1e-12)
        # one-hot probability targets are the index targets
        oh = np.zeros((rows, V))
        oh[np.arange(rows), y] = 1.0
        lp, *_ = oco.forward_probs(z, oh, eps)
        np.testing.assert_allclose(lp, a, rtol=1e-14, atol=1e-14)
        np.testing.assert_allclose(oco.grad_probs(z, oh, np.ones(rows), eps),
                                   oco.grad_index(z, y, np.ones(rows), eps), atol=1e-15)
        # targets summing to 1: every gradient row sums to 0
        assert np.all(np.abs(oco.grad_probs(z, t, np.full(rows, 2.0), eps).sum(axis=1)) <= 1e-14)
        assert np.all(np.abs(oco.grad_index(z, y, np.full(rows, 2.0), eps).sum(axis=1)) <= 1e-14)
        # the reductions are the sum and the mean of the per-row losses
        _, _, _, s, n = oco.forward_index(z, y, eps, reduction="sum")
        _, _, _, mu, _ = oco.forward_index(z, y, eps, reduction="mean")
        assert n == rows
        np.testing.assert_allclose(s, a.sum(), rtol=1e-15)
        np.testing.assert_allclose(mu, a.sum() / rows, rtol=1e-15)


def test_invariants():
    pin_invariants()


def pin_ignore_index(eps=0.1):
    rows, V = 10, 20
    z = rand_rows(rows, V, 12)
    y = np.random.default_rng(13).integers(0, V, rows)
    y[[0, 7]] = -100
    loss, _, _, total, count = oco.forward_index(z, y, eps, -100, "mean")
    keep = np.setdiff1d(np.arange(rows), [0, 7])
    assert count == rows - 2 and loss[0] == 0.0 and loss[7] == 0.0
    ref, *_ = oco.forward_index(z[keep], y[keep], eps)
    np.testing.assert_allclose(loss[keep], ref, rtol=1e-15)
    np.testing.assert_allclose(total, ref.mean(), rtol=1e-14)
    d = oco.grad_index(z, y, 3.0, eps, -100, "mean")
    assert np.all(d[[0, 7]] == 0.0)
    np.testing.assert_allclose(d[keep], oco.grad_index(z[keep], y[keep], np.full(len(keep), 3.0 / len(keep)), eps),
                               rtol=1e-14, atol=1e-16)
    # every row ignored: the mean is 0 / 0
    _, _, _, total, count = oco.forward_index(z, np.full(rows, -100), eps, -100, "mean")
    assert count == 0 and math.isnan(total)
    assert np.all(oco.grad_index(z, np.full(rows, -100), 1.0, eps, -100, "mean") == 0.0)
    # a target out of range that is not ignore_index is a NaN row
    y2 = y.copy()
    y2[3] = V
    loss, *_ = oco.forward_index(z, y2, eps, -100)
    assert math.isnan(loss[3]) and np.isfinite(np.delete(loss, 3)).all()


def test_ignore_index():
    pin_ignore_index()


def pin_infinite_entries():
    z = np.array([[0.5, -np.inf, 1.5, -2.0]] * 4)
    y = np.array([0, 1, 2, 3])
    # eps = 0: a -inf logit has probability 0; a target at -inf gives +inf
    loss, *_ = oco.forward_index(z, y, 0.0)
    assert np.isfinite(loss[[0, 2, 3]]).all() and loss[1] == np.inf
    # eps > 0 puts weight on the -inf logit: +inf for every row
    loss, *_ = oco.forward_index(z, y, 0.1)
    assert np.all(loss == np.inf)
    # probability targets: zero weight on the -inf logit contributes nothing (0 log 0)
    t = np.array([[0.5, 0.0, 0.25, 0.25], [0.0, 0.5, 0.5, 0.0]] * 2)
    lp, *_ = oco.forward_probs(z, t, 0.0)
    assert np.isfinite(lp[[0, 2]]).all() and lp[1] == np.inf
    ref, *_ = oco.forward_probs(z[:1, [0, 2, 3]], t[:1, [0, 2, 3]], 0.0)
    np.testing.assert_allclose(lp[0], ref[0], rtol=1e-15)
    d = oco.grad_probs(z, t, np.ones(4), 0.0)
    assert np.all(d[[0, 2], 1] == 0.0) and np.all(d[[1, 3], 1] == -0.5)


def test_infinite_entries():
    pin_infinite_entries()


# --- planted mistakes: each must fail at least one pin ---------------------------

@contextlib.contextmanager
def planted(name, fn):
    old = getattr(oco, name)
    setattr(oco, name, fn)
    try:
        yield
    finally:
        setattr(oco, name, old)


def fails(pin):
    try:
        pin()
    except (AssertionError, FloatingPointError, ValueError):
        return True
    return False


PINS = (pin_torch, pin_equal_logits, pin_gap_rows, pin_uniform_rows, pin_eps_one, pin_bruteforce,
        pin_invariants, pin_ignore_index, pin_infinite_entries)


def caught():
    return [p.__name__ for p in PINS if fails(p)]


def test_planted_smoothing_over_the_other_classes_is_caught():
    real = oco.index_weights

    def other(y, V, eps, ignore_index=None):
        w, c = real(y, V, 0.0, ignore_index)
        if V > 1:
            w = np.where(w == 1.0, 1.0 - eps, eps / (V - 1))
        return w, c

    with planted("index_weights", other):
        assert caught()


def test_planted_unscaled_target_weight_is_caught():
    real = oco.index_weights

    def unscaled(y, V, eps, ignore_index=None):
        w, c = real(y, V, eps, ignore_index)
        w0, _ = real(y, V, 0.0, ignore_index)
        return w + eps * w0, c

    with planted("index_weights", unscaled):
        assert caught()


def test_planted_mean_over_all_rows_is_caught():
    real = oco.reduce

    def all_rows(loss, counted, reduction):
        return real(loss, np.ones_like(counted), reduction)

    with planted("reduce", all_rows):
        assert caught()


def test_planted_missing_zero_weight_guard_is_caught():
    def unguarded(z, w):
        z, m, ls = oco._stats(z)
        with np.errstate(invalid="ignore"):
            lp = oco._log_softmax(z, m, ls)
            return -(w * lp).sum(axis=1), m, ls, w.sum(axis=1)

    with planted("weighted_rows", unguarded):
        assert caught()


def test_planted_unnormalised_gradient_is_caught():
    def no_w(z, w, gi, counted):
        z, m, ls = oco._stats(z)
        with np.errstate(invalid="ignore", over="ignore"):
            d = gi[:, None] * (np.exp(oco._log_softmax(z, m, ls)) - w)
        d[~counted] = 0.0
        return d

    with planted("weighted_grad", no_w):
        assert caught()


def test_planted_ignored_rows_as_class_zero_is_caught():
    real = oco.index_weights

    def clamp(y, V, eps, ignore_index=None):
        y = np.asarray(y, np.int64)
        if ignore_index is not None:
            y = np.where(y == ignore_index, 0, y)
        return real(y, V, eps, None)

    with planted("index_weights", clamp):
        assert caught()
