"""Float64 oracle for the row-wise KL divergence between two logit rows.

TEST INFRASTRUCTURE: imported only by tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg.

Definition: "One barrier short", section "Run it yourself" (the reference the page
checks the fused kernel against).  For student logits q and teacher logits p of one
row, with the log-softmaxes lq = q - logsumexp(q) and lp = p - logsumexp(p),

    kl = sum_j exp(lp_j) (lp_j - lq_j)          (KL of the teacher from the student)

and the gradient of sum_i g_i kl_i with respect to the student row is
g_i (exp(lq_i) - exp(lp_i)) = g_i (softmax(q_i) - softmax(p_i)).

The oracle is that definition written out in float64, with the row statistics of
the softmax cross-entropy oracle (max shift, pairwise sums).  A teacher entry of
-inf has zero probability and contributes nothing (0 log 0 = 0); a student entry of
-inf under a teacher entry with positive probability makes the row +inf; a teacher
row that is -inf throughout has no softmax (0 / 0), so its kl is NaN, as an all -inf
logits row gives a NaN cross-entropy.
"""

from __future__ import annotations

import numpy as np

from . import ce


def row_stats(z: np.ndarray):
    """(m, log s) of each row: the max and the log of sum exp(z - m)."""
    z = np.asarray(z, np.float64)
    m = ce.row_max(z)
    return m, ce.row_log_sum(z, m)


def log_softmax(z: np.ndarray, m=None, ls=None) -> np.ndarray:
    if m is None or ls is None:
        m, ls = row_stats(z)
    with np.errstate(invalid="ignore"):
        return (np.asarray(z, np.float64) - m[:, None]) - ls[:, None]


def forward(q: np.ndarray, p: np.ndarray):
    """Per-row (kl, m_q, log s_q, m_p, log s_p) for float64 student q and teacher p."""
    mq, lsq = row_stats(q)
    mp, lsp = row_stats(p)
    lq = log_softmax(q, mq, lsq)
    lp = log_softmax(p, mp, lsp)
    P = np.exp(lp)
    with np.errstate(invalid="ignore"):
        terms = np.where(P > 0, P * (lp - lq), 0.0)
    kl = terms.sum(axis=1)
    # a teacher row without mass (all -inf) has no softmax: 0 / 0
    kl[mp == -np.inf] = np.nan
    return kl, mq, lsq, mp, lsp


def grad(q: np.ndarray, p: np.ndarray, g: np.ndarray, stats=None) -> np.ndarray:
    """g_i (softmax(q_i) - softmax(p_i)); stats = (m_q, log s_q, m_p, log s_p) if saved."""
    if stats is None:
        mq, lsq = row_stats(q)
        mp, lsp = row_stats(p)
    else:
        mq, lsq, mp, lsp = (np.asarray(s, np.float64) for s in stats)
    with np.errstate(invalid="ignore", over="ignore"):
        Q = np.exp(log_softmax(q, mq, lsq))
        P = np.exp(log_softmax(p, mp, lsp))
        return np.asarray(g, np.float64)[:, None] * (Q - P)
