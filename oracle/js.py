"""Float64 oracle for the row-wise Jensen-Shannon divergence between two logit rows.

TEST INFRASTRUCTURE: imported only by tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg.

Source: "One barrier short", first section and section "The fix": mlx-lm computes the
Jensen-Shannon divergence of a student and a teacher distribution in fused kernels
beside the KL ones, and at a logit scale of 20 its loss overflowed to non-finite values
until a numerically stable softplus was used.  The page gives no formula; this oracle
takes the standard definition, with P = softmax(p) (teacher) and Q = softmax(q)
(student):

    M  = (P + Q) / 2
    js = 1/2 KL(P || M) + 1/2 KL(Q || M)
       = 1/2 sum_j P_j (log P_j - log M_j) + 1/2 sum_j Q_j (log Q_j - log M_j)

and its gradient with respect to the student logits, scaled per row by g:

    d js / d q_k = Q_k (h_k - H),  h_k = (log Q_k - log M_k) / 2,  H = sum_j Q_j h_j.

log M is formed as logaddexp(log P, log Q) - log 2 (NumPy's logaddexp: the stable
softplus form max(a, b) + log1p(exp(-|a - b|))), on the log-softmaxes of
``oracle.kl``.  A zero probability contributes nothing (0 log 0 = 0); a row that has
no softmax (all -inf) gives NaN.  The function also returns H, the student's half,
which a VJP needs besides the two row normalisers.
"""

from __future__ import annotations

import numpy as np

from . import kl

LOG2 = np.log(2.0)


def _half_terms(lp: np.ndarray, lq: np.ndarray):
    """(1/2 P (log P - log M), 1/2 Q (log Q - log M)) elementwise, with 0 log 0 = 0."""
    with np.errstate(invalid="ignore", over="ignore"):
        lm = np.logaddexp(lp, lq) - LOG2
        P, Q = np.exp(lp), np.exp(lq)
        tp = np.where(P > 0, 0.5 * P * (lp - lm), 0.0)
        tq = np.where(Q > 0, 0.5 * Q * (lq - lm), 0.0)
    return tp, tq, lm


def forward(q: np.ndarray, p: np.ndarray):
    """Per-row (js, m_q, log s_q, m_p, log s_p, H) for float64 student q and teacher p."""
    q = np.asarray(q, np.float64)
    p = np.asarray(p, np.float64)
    mq, lsq = kl.row_stats(q)
    mp, lsp = kl.row_stats(p)
    lq = kl.log_softmax(q, mq, lsq)
    lp = kl.log_softmax(p, mp, lsp)
    tp, tq, _ = _half_terms(lp, lq)
    H = tq.sum(axis=1)
    js = tp.sum(axis=1) + H
    bad = (mq == -np.inf) | (mp == -np.inf)
    js[bad] = np.nan
    H[bad] = np.nan
    return js, mq, lsq, mp, lsp, H


def grad(q: np.ndarray, p: np.ndarray, g: np.ndarray) -> np.ndarray:
    """g_i Q_ik (h_ik - H_i)."""
    q = np.asarray(q, np.float64)
    p = np.asarray(p, np.float64)
    lq = kl.log_softmax(q)
    lp = kl.log_softmax(p)
    with np.errstate(invalid="ignore", over="ignore"):
        lm = np.logaddexp(lp, lq) - LOG2
        Q = np.exp(lq)
        h = np.where(Q > 0, 0.5 * (lq - lm), 0.0)
        H = (Q * h).sum(axis=1)
        return np.asarray(g, np.float64)[:, None] * Q * (h - H[:, None])
