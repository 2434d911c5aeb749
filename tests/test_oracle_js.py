"""Pins for the Jensen-Shannon oracle (oracle/js.py), CPU only.

"One barrier short" names the fused Jensen-Shannon kernels and their overflow at a logit
scale of 20 without giving a formula; the oracle takes the standard definition.  These
pins fix it to SciPy's jensenshannon, closed forms (0 for identical rows, ln 2 for
disjoint supports), a 50-digit brute force that includes scale-20 rows, central finite
differences for the gradient, and invariants; planted mistakes must each fail one.
"""

import contextlib
import math

import mpmath
import numpy as np
import scipy.spatial.distance
import scipy.special

from oracle import js as ojs

LN2 = math.log(2.0)


def rows(n=6, V=40, seed=0, scale=3.0):
    g = np.random.default_rng(seed)
    return g.normal(0, scale, (n, V)), g.normal(0, scale, (n, V))


def pin_scipy():
    for V, scale in ((2, 1.0), (37, 3.0), (500, 4.0)):
        q, p = rows(7, V, V, scale)
        js, *_ = ojs.forward(q, p)
        P, Q = scipy.special.softmax(p, axis=1), scipy.special.softmax(q, axis=1)
        ref = scipy.spatial.distance.jensenshannon(P, Q, axis=1) ** 2
        np.testing.assert_allclose(js, ref, rtol=1e-9, atol=1e-15)


def test_matches_scipy():
    pin_scipy()


def pin_closed_forms():
    q, _ = rows(5, 30, 1)
    js, *rest = ojs.forward(q, q)
    assert np.all(np.abs(js) <= 1e-15)
    assert np.all(np.abs(ojs.grad(q, q, np.ones(5))) <= 1e-15)
    # disjoint supports: M is half of each, so both KL terms are log 2
    V = 12
    q = np.full((3, V), -np.inf)
    p = np.full((3, V), -np.inf)
    q[:, : V // 2] = np.random.default_rng(2).normal(0, 2, (3, V // 2))
    p[:, V // 2:] = np.random.default_rng(3).normal(0, 2, (3, V // 2))
    js, *_ = ojs.forward(q, p)
    np.testing.assert_allclose(js, LN2, rtol=0, atol=1e-15)
    # a point mass against a uniform row of V: closed form from the definition
    V = 16
    q = np.full((1, V), 0.7)
    p = np.full((1, V), -np.inf)
    p[0, 3] = 1.0
    js, *_ = ojs.forward(q, p)
    m_hit = 0.5 * (1.0 + 1.0 / V)
    want = 0.5 * math.log(1.0 / m_hit) + 0.5 * ((1.0 / V) * math.log((1.0 / V) / m_hit) +
                                               (V - 1) / V * math.log((1.0 / V) / (0.5 / V)))
    np.testing.assert_allclose(js, want, rtol=1e-14)


def test_closed_forms():
    pin_closed_forms()


def brute(q, p):
    """50 digits, no max shift, M formed directly."""
    out, grads = [], []
    with mpmath.workdps(50):
        for qr, pr in zip(q.tolist(), p.tolist()):
            eq = [mpmath.exp(mpmath.mpf(v)) for v in qr]
            ep = [mpmath.exp(mpmath.mpf(v)) for v in pr]
            sq, sp = mpmath.fsum(eq), mpmath.fsum(ep)
            Q = [e / sq for e in eq]
            P = [e / sp for e in ep]
            M = [(a + b) / 2 for a, b in zip(P, Q)]
            kpm = mpmath.fsum(a * mpmath.log(a / m) for a, m in zip(P, M) if a != 0)
            kqm = mpmath.fsum(b * mpmath.log(b / m) for b, m in zip(Q, M) if b != 0)
            out.append(float((kpm + kqm) / 2))
            h = [mpmath.log(b / m) / 2 for b, m in zip(Q, M)]
            H = mpmath.fsum(b * hh for b, hh in zip(Q, h))
            grads.append([float(b * (hh - H)) for b, hh in zip(Q, h)])
    return np.array(out), np.array(grads)


def pin_bruteforce():
    for V, scale in ((1, 1.0), (2, 3.0), (5, 20.0), (17, 20.0), (33, 6.0)):
        q, p = rows(4, V, V + 7, scale)
        q[1] += 250.0  # far past exp's float64 range unshifted
        js, *_ = ojs.forward(q, p)
        bj, bg = brute(q, p)
        np.testing.assert_allclose(js, bj, rtol=1e-11, atol=1e-15)
        np.testing.assert_allclose(ojs.grad(q, p, np.ones(4)), bg, rtol=0, atol=1e-14)


def test_bruteforce():
    pin_bruteforce()


def pin_finite_differences(h=1e-6):
    q, p = rows(3, 9, 11, 2.5)
    g = np.array([1.0, 0.5, 2.0])
    d = ojs.grad(q, p, g)
    for i in range(3):
        for k in range(9):
            qp, qm = q.copy(), q.copy()
            qp[i, k] += h
            qm[i, k] -= h
            fd = g[i] * (ojs.forward(qp, p)[0][i] - ojs.forward(qm, p)[0][i]) / (2 * h)
            assert abs(fd - d[i, k]) <= 1e-8, (i, k, fd, d[i, k])


def test_gradient_finite_differences():
    pin_finite_differences()


def pin_invariants():
    q, p = rows(8, 64, 13, 4.0)
    js, mq, lsq, mp, lsp, H = ojs.forward(q, p)
    assert np.all(js >= -1e-15) and np.all(js <= LN2 + 1e-15)
    js2, *_ = ojs.forward(p, q)
    np.testing.assert_allclose(js2, js, rtol=1e-13, atol=1e-16)
    js3, *_ = ojs.forward(q + 1e5, p - 3e4)
    np.testing.assert_allclose(js3, js, rtol=1e-9, atol=1e-12)
    d = ojs.grad(q, p, np.full(8, 1.5))
    assert np.all(np.abs(d.sum(axis=1)) <= 1e-15)
    # H is the student's half: 1/2 KL(Q || M) >= 0, and js - H the teacher's
    assert np.all(H >= -1e-16) and np.all(js - H >= -1e-16)


def test_invariants():
    pin_invariants()


def test_scale_20_is_finite():
    """The page's overflow case: logits at scale 20 over the full vocabulary."""
    q, p = rows(4, 151936, 21, 20.0)
    js, *rest = ojs.forward(q, p)
    assert np.isfinite(js).all() and np.all(js >= 0) and np.all(js <= LN2 + 1e-15)
    assert np.isfinite(ojs.grad(q, p, np.ones(4))).all()


def test_rows_without_softmax_are_nan():
    q, p = rows(3, 10, 17)
    p[1] = -np.inf
    q[2] = -np.inf
    js, *_ = ojs.forward(q, p)
    assert np.isnan(js[1]) and np.isnan(js[2]) and np.isfinite(js[0])


# --- planted mistakes -----------------------------------------------------------------

@contextlib.contextmanager
def planted(module, name, fn):
    old = getattr(module, name)
    setattr(module, name, fn)
    try:
        yield
    finally:
        setattr(module, name, old)


PINS = (pin_scipy, pin_closed_forms, pin_bruteforce, pin_finite_differences, pin_invariants)


def caught():
    out = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, FloatingPointError, ValueError):
            out.append(pin.__name__)
    return out


def test_planted_mixture_without_half_is_caught():
    def no_half(lp, lq):
        with np.errstate(invalid="ignore", over="ignore"):
            lm = np.logaddexp(lp, lq)
            P, Q = np.exp(lp), np.exp(lq)
            return (np.where(P > 0, 0.5 * P * (lp - lm), 0.0), np.where(Q > 0, 0.5 * Q * (lq - lm), 0.0), lm)

    with planted(ojs, "_half_terms", no_half):
        assert caught()


def test_planted_one_sided_divergence_is_caught():
    real = ojs._half_terms

    def one_side(lp, lq):
        tp, tq, lm = real(lp, lq)
        return 2 * tp, 0 * tq, lm

    with planted(ojs, "_half_terms", one_side):
        assert caught()


def test_planted_uncentred_gradient_is_caught():
    def uncentred(q, p, g):
        lq = ojs.kl.log_softmax(np.asarray(q, np.float64))
        lp = ojs.kl.log_softmax(np.asarray(p, np.float64))
        lm = np.logaddexp(lp, lq) - ojs.LOG2
        Q = np.exp(lq)
        return np.asarray(g, np.float64)[:, None] * Q * 0.5 * (lq - lm)

    with planted(ojs, "grad", uncentred):
        assert caught()


def test_planted_gradient_for_the_teacher_is_caught():
    real = ojs.grad
    with planted(ojs, "grad", lambda q, p, g: real(p, q, g)):
        assert caught()
