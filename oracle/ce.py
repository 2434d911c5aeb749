"""Float64 oracle for softmax cross-entropy: loss, log-sum-exp and gradient.

TEST INFRASTRUCTURE: imported only by tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg.

Definitions (the pages' notation; z is one row of logits, y its target):

* loss = logsumexp(z) - z_y.  Source: Ineshin, "A fused linear cross-entropy
  forward kernel for Apple GPUs", section 1 "Streaming the loss without full
  logits".
* The row max is shifted out before the target score is taken, so
  loss = (m - z_y) + log sum_j exp(z_j - m), with m = max_j z_j.  Source: MLX
  PR #4188 "Shift by the max in cross_entropy", Proposed changes.  The shift
  leaves the exact value unchanged and keeps the gap between the logits from
  being absorbed into a large magnitude.
* The gradient of loss_i scaled by the upstream g_i is
  g_i * (softmax(z_i) - onehot(y_i)): the vector-Jacobian product of the
  per-row loss.

All arithmetic is float64 on the exact stored inputs.  Rows are processed as
plain NumPy reductions, in row chunks for large batches.  The oracle knows
nothing about strides: callers slice views with NumPy before passing rows.

Readings where the pages say nothing:

* A target outside [0, V) gives a NaN loss and a NaN gradient row.
* -inf entries carry zero probability.  A row that holds only -inf, or holds
  +inf or NaN, gives NaN, as the plain formula does.
"""

from __future__ import annotations

import numpy as np

CHUNK_ROWS = 1 << 22  # rows per chunk, as in the reference check of MLX PR #4776


def decode(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of stored logits (bf16 given as uint16 bit patterns)."""
    if dtype == "f32":
        return np.asarray(x, np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(x, np.float16).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(x, np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def row_max(z: np.ndarray) -> np.ndarray:
    return z.max(axis=1)


def row_log_sum(z: np.ndarray, m: np.ndarray) -> np.ndarray:
    """log sum_j exp(z_j - m) per row (the scaled sum of the online state)."""
    with np.errstate(invalid="ignore", over="ignore"):
        return np.log(np.exp(z - m[:, None]).sum(axis=1))


def target_logit(z: np.ndarray, y: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    V = z.shape[1]
    y = np.asarray(y, np.int64)
    ok = (y >= 0) & (y < V)
    zy = z[np.arange(z.shape[0]), np.where(ok, y, 0)]
    return np.where(ok, zy, np.nan), ok


def forward(z: np.ndarray, y: np.ndarray):
    """Per-row (loss, m, log_s) for float64 logits z [rows, V]; lse = m + log_s."""
    z = np.asarray(z, np.float64)
    m = row_max(z)
    ls = row_log_sum(z, m)
    zy, _ = target_logit(z, y)
    with np.errstate(invalid="ignore"):
        loss = (m - zy) + ls
    return loss, m, ls


def grad(z: np.ndarray, y: np.ndarray, g: np.ndarray, m=None, ls=None) -> np.ndarray:
    """g_i * (softmax(z_i) - onehot(y_i)) in float64, from the row statistics."""
    z = np.asarray(z, np.float64)
    if m is None or ls is None:
        m = row_max(z)
        ls = row_log_sum(z, m)
    with np.errstate(invalid="ignore", over="ignore"):
        p = np.exp((z - m[:, None]) - ls[:, None])
    onehot = np.zeros_like(p)
    _, ok = target_logit(z, y)
    rows = np.flatnonzero(ok)
    onehot[rows, np.asarray(y, np.int64)[rows]] = 1.0
    with np.errstate(invalid="ignore"):
        d = np.asarray(g, np.float64)[:, None] * (p - onehot)
    d[~ok] = np.nan
    return d


def forward_stored(x: np.ndarray, dtype: str, y: np.ndarray, chunk: int = CHUNK_ROWS):
    """forward() over stored rows [rows, V], decoded chunk by chunk."""
    R = x.shape[0]
    loss = np.empty(R)
    m = np.empty(R)
    ls = np.empty(R)
    for r0 in range(0, R, chunk):
        r1 = min(R, r0 + chunk)
        loss[r0:r1], m[r0:r1], ls[r0:r1] = forward(decode(x[r0:r1], dtype), y[r0:r1])
    return loss, m, ls


def grad_stored(x: np.ndarray, dtype: str, y: np.ndarray, g: np.ndarray) -> np.ndarray:
    return grad(decode(x, dtype), y, g)
