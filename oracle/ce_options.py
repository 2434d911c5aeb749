"""Float64 oracle for the cross-entropy options: label smoothing, probability targets,
ignore_index and the 'sum' / 'mean' reductions.

TEST INFRASTRUCTURE: imported only by tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg.

Source: MLX PR #4188 "Shift by the max in cross_entropy", Proposed changes.  The loss
there takes class-index or probability targets, an optional label smoothing whose term
subtracts the mean logit, and three reductions, each checked against PyTorch; the max
shift applies to every one of these paths.

Definition, for one row z of V logits with log p_j = z_j - logsumexp(z):

    loss = - sum_j w_j log p_j

with the target weights

    class index y:          w = (1 - eps) onehot(y) + eps / V
    probabilities t:        w = (1 - eps) t + eps / V

With eps = 0 and an index target this is logsumexp(z) - z_y, the plain cross-entropy.
For an index target it equals (1 - eps)(lse - z_y) + eps (lse - mean_j z_j): the
smoothing term subtracts the mean logit, as the page says.  The gradient of
sum_i g_i loss_i with respect to z_i is g_i (W_i p_i - w_i), W_i = sum_j w_ij.

Readings where the page is silent:

* A weight of 0 contributes nothing, even where log p_j = -inf (0 log 0 = 0).
* ignore_index (index targets only): a row whose target equals it has loss 0 and
  gradient 0 and does not count towards the mean.  This is PyTorch's convention, the
  reference the page checks against.  Any other target outside [0, V) gives a NaN row.
* 'sum' adds the losses of the counted rows; 'mean' divides that sum by their number
  (NaN when no row counts, 0 / 0).  The VJP of a reduced loss with upstream scalar g
  is the per-row VJP with g_i = g ('sum') or g / count ('mean'), and 0 on ignored rows.

The log-softmax uses the row statistics of ``oracle.ce`` (max shift, log of the
shifted sum), so every path carries the shift.
"""

from __future__ import annotations

import numpy as np

from . import ce

REDUCTIONS = ("none", "sum", "mean")


def _stats(z):
    z = np.asarray(z, np.float64)
    m = ce.row_max(z)
    return z, m, ce.row_log_sum(z, m)


def _log_softmax(z, m, ls):
    with np.errstate(invalid="ignore"):
        return (z - m[:, None]) - ls[:, None]


def index_weights(y: np.ndarray, V: int, eps: float, ignore_index=None):
    """(w [rows, V], counted [rows]) for class-index targets.

    Ignored rows get weight 0 and counted = False; a target outside [0, V) that is not
    ignore_index gets NaN weights (a NaN row)."""
    y = np.asarray(y, np.int64)
    rows = y.shape[0]
    ignored = np.zeros(rows, bool) if ignore_index is None else (y == ignore_index)
    valid = (y >= 0) & (y < V)
    w = np.full((rows, V), eps / V)
    r = np.flatnonzero(valid & ~ignored)
    w[r, y[r]] += 1.0 - eps
    w[~valid & ~ignored] = np.nan
    w[ignored] = 0.0
    return w, ~ignored


def prob_weights(t: np.ndarray, eps: float):
    t = np.asarray(t, np.float64)
    return (1.0 - eps) * t + eps / t.shape[1]


def weighted_rows(z: np.ndarray, w: np.ndarray):
    """Per-row (loss, m, log s, W) of loss = -sum_j w_j log p_j, with 0 log 0 = 0."""
    z, m, ls = _stats(z)
    lp = _log_softmax(z, m, ls)
    with np.errstate(invalid="ignore"):
        terms = np.where(w != 0, w * lp, 0.0)
    return -terms.sum(axis=1), m, ls, w.sum(axis=1)


def reduce(loss: np.ndarray, counted: np.ndarray, reduction: str):
    """(total, count) of the counted rows; total is None for 'none'."""
    if reduction not in REDUCTIONS:
        raise ValueError(reduction)
    count = int(np.count_nonzero(counted))
    if reduction == "none":
        return None, count
    s = float(np.sum(np.where(counted, loss, 0.0)))
    if reduction == "sum":
        return s, count
    with np.errstate(invalid="ignore", divide="ignore"):
        return float(np.float64(s) / np.float64(count)), count


def row_upstream(g, counted: np.ndarray, reduction: str, count: int) -> np.ndarray:
    """Per-row upstream gradient: g itself for 'none', else the scalar g spread over the
    counted rows (divided by their number for 'mean'); 0 on rows that do not count."""
    if reduction == "none":
        gi = np.asarray(g, np.float64).copy()
    elif reduction == "sum":
        gi = np.full(counted.shape[0], float(g))
    else:
        with np.errstate(invalid="ignore", divide="ignore"):
            gi = np.full(counted.shape[0], np.float64(g) / np.float64(count))
    gi[~counted] = 0.0
    return gi


def weighted_grad(z: np.ndarray, w: np.ndarray, gi: np.ndarray, counted: np.ndarray) -> np.ndarray:
    """g_i (W_i p_ij - w_ij); rows that do not count are 0."""
    z, m, ls = _stats(z)
    with np.errstate(invalid="ignore", over="ignore"):
        p = np.exp(_log_softmax(z, m, ls))
        d = gi[:, None] * (w.sum(axis=1)[:, None] * p - w)
    d[~counted] = 0.0
    return d


# --- class-index targets ---------------------------------------------------------

def forward_index(z, y, eps=0.0, ignore_index=None, reduction="none"):
    """(loss [rows], m, log s, total, count)."""
    z = np.asarray(z, np.float64)
    w, counted = index_weights(y, z.shape[1], eps, ignore_index)
    loss, m, ls, _ = weighted_rows(z, w)
    loss[~counted] = 0.0
    total, count = reduce(loss, counted, reduction)
    return loss, m, ls, total, count


def grad_index(z, y, g, eps=0.0, ignore_index=None, reduction="none"):
    z = np.asarray(z, np.float64)
    w, counted = index_weights(y, z.shape[1], eps, ignore_index)
    gi = row_upstream(g, counted, reduction, int(np.count_nonzero(counted)))
    return weighted_grad(z, w, gi, counted)


# --- probability targets ---------------------------------------------------------

def forward_probs(z, t, eps=0.0, reduction="none"):
    """(loss [rows], m, log s, W = sum_j w_j [rows], total, count)."""
    z = np.asarray(z, np.float64)
    w = prob_weights(t, eps)
    loss, m, ls, W = weighted_rows(z, w)
    counted = np.ones(z.shape[0], bool)
    total, count = reduce(loss, counted, reduction)
    return loss, m, ls, W, total, count


def grad_probs(z, t, g, eps=0.0, reduction="none"):
    z = np.asarray(z, np.float64)
    w = prob_weights(t, eps)
    counted = np.ones(z.shape[0], bool)
    gi = row_upstream(g, counted, reduction, z.shape[0])
    return weighted_grad(z, w, gi, counted)
