"""CPU model, in float32 NumPy, of the per-lane state kl_forward keeps, checked against
the float64 oracle at large per-row offsets of the student and teacher rows.

The kernel keeps t = sum_j exp(p_j - m_p) ((p_j - m_p) - (q_j - m_q)) against the two
running maxima, so t / s_p is of the size of the rows' spread at any offset, and
kl = t / s_p - log s_p + log s_q.  A sum of the raw differences p_j - q_j instead carries
the gap between the two rows' offsets and cancels it against m_q - m_p at the end; in
float32 that loses the result once the gap reaches 1e4 ("Shift by the max in
cross_entropy", Proposed changes: the shift comes before anything else, so every path
gains from it).  The model follows the kernel's update order (groups of 8 elements, one
rescale per group, a merge of two half-row states) with NumPy's float32 exp standing in
for the hardware exp2; it is a model of the arithmetic, not of the rounding of each
instruction.
"""

import numpy as np
import pytest

from oracle import kl as okl
from softmax_cross_entropy_amd import inputs

F = np.float32


def _ref(m):
    return np.where(m == -np.inf, F(0), m).astype(F)


def _new_state(n):
    z = np.zeros(n, F)
    return dict(mq=np.full(n, -np.inf, F), sq=z.copy(), mp=np.full(n, -np.inf, F), sp=z.copy(), t=z.copy())


def _shift(t, sp, rq, rp, nq, np_, c):
    return ((t + sp * ((rp - np_) - (rq - nq))) * c).astype(F)


def _add_relative(st, q, p):
    """One group of columns folded the way the kernel folds it."""
    mq = np.maximum(st["mq"], q.max(axis=1))
    mp = np.maximum(st["mp"], p.max(axis=1))
    rq, rp = _ref(mq), _ref(mp)
    dq = (q - rq[:, None]).astype(F)
    dp = (p - rp[:, None]).astype(F)
    w = np.exp(dp).astype(F)
    with np.errstate(invalid="ignore"):
        t = np.where(w > 0, w * (dp - dq), F(0)).astype(F).sum(axis=1, dtype=F)
    cp = np.exp(st["mp"] - rp).astype(F)
    st["t"] = _shift(st["t"], st["sp"], _ref(st["mq"]), _ref(st["mp"]), rq, rp, cp) + t
    st["sq"] = st["sq"] * np.exp(st["mq"] - rq).astype(F) + np.exp(dq).astype(F).sum(axis=1, dtype=F)
    st["sp"] = st["sp"] * cp + w.sum(axis=1, dtype=F)
    st["mq"], st["mp"] = mq, mp


def _merge_relative(a, b):
    mq = np.maximum(a["mq"], b["mq"])
    mp = np.maximum(a["mp"], b["mp"])
    rq, rp = _ref(mq), _ref(mp)
    cqa, cqb = np.exp(a["mq"] - rq).astype(F), np.exp(b["mq"] - rq).astype(F)
    ca, cb = np.exp(a["mp"] - rp).astype(F), np.exp(b["mp"] - rp).astype(F)
    t = (_shift(a["t"], a["sp"], _ref(a["mq"]), _ref(a["mp"]), rq, rp, ca)
         + _shift(b["t"], b["sp"], _ref(b["mq"]), _ref(b["mp"]), rq, rp, cb))
    return dict(mq=mq, mp=mp, sq=(a["sq"] * cqa + b["sq"] * cqb).astype(F),
                sp=(a["sp"] * ca + b["sp"] * cb).astype(F), t=t.astype(F))


def _add_raw(st, q, p):
    """The raw-difference state: t = sum_j exp(p_j - m_p) (p_j - q_j)."""
    mq = np.maximum(st["mq"], q.max(axis=1))
    mp = np.maximum(st["mp"], p.max(axis=1))
    rq, rp = _ref(mq), _ref(mp)
    w = np.exp((p - rp[:, None]).astype(F)).astype(F)
    t = (w * (p - q).astype(F)).astype(F).sum(axis=1, dtype=F)
    cp = np.exp(st["mp"] - rp).astype(F)
    st["t"] = st["t"] * cp + t
    st["sq"] = st["sq"] * np.exp(st["mq"] - rq).astype(F) + np.exp((q - rq[:, None]).astype(F)).sum(axis=1, dtype=F)
    st["sp"] = st["sp"] * cp + w.sum(axis=1, dtype=F)
    st["mq"], st["mp"] = mq, mp


def model_kl(q, p, relative=True, group=8):
    n, V = q.shape
    halves = []
    for lo, hi in ((0, V // 2), (V // 2, V)):
        st = _new_state(n)
        for j in range(lo, hi, group):
            (_add_relative if relative else _add_raw)(st, q[:, j:min(j + group, hi)], p[:, j:min(j + group, hi)])
        halves.append(st)
    lsq = lambda s: np.log(s).astype(F)
    if relative:
        st = _merge_relative(*halves)
        return (st["t"] / st["sp"] + (lsq(st["sq"]) - lsq(st["sp"]))).astype(np.float64)
    a, b = halves  # raw form: merge of the two halves the same way, then the offset terms
    mq = np.maximum(a["mq"], b["mq"]); mp = np.maximum(a["mp"], b["mp"])
    ca, cb = np.exp(a["mp"] - mp).astype(F), np.exp(b["mp"] - mp).astype(F)
    sp = (a["sp"] * ca + b["sp"] * cb).astype(F)
    sq = (a["sq"] * np.exp(a["mq"] - mq) + b["sq"] * np.exp(b["mq"] - mq)).astype(F)
    t = (a["t"] * ca + b["t"] * cb).astype(F)
    return (t / sp + ((mq - mp) + (lsq(sq) - lsq(sp)))).astype(np.float64)


def _rows(c_q, c_p, V=4096, n=16):
    q, p, _ = inputs.kl_pair(n, V, "f32", scale=4.0, workload=90)
    q = (q.astype(np.float64) + c_q).astype(F)
    p = (p.astype(np.float64) + c_p).astype(F)
    return q, p


@pytest.mark.parametrize("c_q,c_p", [(0.0, 0.0), (1e4, 0.0), (0.0, 1e4), (1e6, -1e6), (1e8, 1e2), (-1e8, 1e8)])
def test_relative_state_error_does_not_grow_with_offset(c_q, c_p):
    q, p = _rows(c_q, c_p)
    ref, *_ = okl.forward(q.astype(np.float64), p.astype(np.float64))
    err = np.abs(model_kl(q, p) - ref)
    assert np.all(err <= 1e-5 * (1 + np.abs(ref))), err.max()


def test_raw_difference_state_fails_at_an_offset_gap():
    """The former raw-difference state, on the same rows: fine without offsets, off by far
    more than the tolerance once the two rows' offsets differ by 1e6."""
    q, p = _rows(0.0, 0.0)
    ref, *_ = okl.forward(q.astype(np.float64), p.astype(np.float64))
    assert np.all(np.abs(model_kl(q, p, relative=False) - ref) <= 1e-5 * (1 + np.abs(ref)))
    q, p = _rows(1e6, 0.0)
    ref, *_ = okl.forward(q.astype(np.float64), p.astype(np.float64))
    assert np.max(np.abs(model_kl(q, p, relative=False) - ref) / (1 + np.abs(ref))) > 1e-4


def test_identical_rows_give_zero_in_the_model():
    q, _ = _rows(1e6, 0.0)
    assert np.all(model_kl(q, q.copy()) == 0.0)
