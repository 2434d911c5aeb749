"""Float64 oracle for the linear cross-entropy forward and its gradients.

TEST INFRASTRUCTURE: imported only by tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg.

Definition: Ineshin, "A fused linear cross-entropy forward kernel for Apple
GPUs", section 1 "Streaming the loss without full logits".  With hidden states
H (N x D) and output projection W (V x D), the logits are Z = H W^T and
loss_i = logsumexp(Z_i) - Z_{i, y_i}.

The streaming kernel on that page reaches the same value as the materialised
definition, up to rounding order.  The oracle therefore does not stream: it
builds each row block of Z in float64 with one matrix product (bf16 inputs
are exact in float64, and each product of two bf16 values is exact too), then
applies the softmax cross-entropy oracle to those rows.

The gradients follow the same page, section 1: training saves the forward's
log-sum-exp, and the backward regenerates the logits it needs.  For the
objective sum_i g_i loss_i, the derivative with respect to the logits row Z_i
is g_i (softmax(Z_i) - onehot(y_i)) (the softmax cross-entropy gradient), and
the chain rule through Z = H W^T gives dH = dZ W and dW = dZ^T H.  ``grad64``
writes exactly that out on float64 inputs, one row block of Z at a time.
"""

from __future__ import annotations

import numpy as np

from . import ce

BLOCK_ROWS = 512


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    return ce.decode(bits, "bf16")


def logits(H64: np.ndarray, W64: np.ndarray) -> np.ndarray:
    """Z = H W^T for float64 H [n, D] and W [V, D]."""
    return H64 @ W64.T


def forward(H_bits: np.ndarray, W_bits: np.ndarray, y: np.ndarray, rows=None,
            block: int = BLOCK_ROWS, W64: np.ndarray | None = None):
    """Per-row (loss, m, log_s) for the selected rows (all rows by default)."""
    if rows is None:
        rows = np.arange(H_bits.shape[0])
    rows = np.asarray(rows)
    if W64 is None:
        W64 = decode_bf16(W_bits)
    n = rows.shape[0]
    loss = np.empty(n)
    m = np.empty(n)
    ls = np.empty(n)
    for b0 in range(0, n, block):
        b1 = min(n, b0 + block)
        sel = rows[b0:b1]
        Z = logits(decode_bf16(H_bits[sel]), W64)
        loss[b0:b1], m[b0:b1], ls[b0:b1] = ce.forward(Z, np.asarray(y)[sel])
    return loss, m, ls


def grad64(H64: np.ndarray, W64: np.ndarray, y: np.ndarray, g: np.ndarray, m=None, ls=None,
           block: int = BLOCK_ROWS, bounds: bool = False):
    """(dH, dW) of sum_i g_i loss_i for float64 H [N, D] and W [V, D].

    dZ = diag(g) (softmax(Z) - onehot(y)) row block by row block, then dH = dZ W and
    dW += dZ^T H.  When the saved row statistics (m, ls) are given, softmax(Z_i) is
    exp((Z_i - m_i) - ls_i), as a backward that reuses the forward's log-sum-exp forms
    it; otherwise they are computed from Z.  With bounds=True it also returns
    |dZ| |W| and |dZ|^T |H|, the sums of magnitudes that bound how far a rounding of dZ
    can move each entry of dH and dW.
    """
    H64 = np.asarray(H64, np.float64)
    W64 = np.asarray(W64, np.float64)
    y = np.asarray(y)
    g = np.asarray(g, np.float64)
    N = H64.shape[0]
    dH = np.zeros((N, H64.shape[1]))
    dW = np.zeros(W64.shape)
    if bounds:
        bH = np.zeros_like(dH)
        bW = np.zeros_like(dW)
    for b0 in range(0, N, block):
        b1 = min(N, b0 + block)
        Z = logits(H64[b0:b1], W64)
        dZ = ce.grad(Z, y[b0:b1], g[b0:b1],
                     None if m is None else np.asarray(m, np.float64)[b0:b1],
                     None if ls is None else np.asarray(ls, np.float64)[b0:b1])
        dH[b0:b1] = dZ @ W64
        dW += dZ.T @ H64[b0:b1]
        if bounds:
            aZ = np.abs(dZ)
            bH[b0:b1] = aZ @ np.abs(W64)
            bW += aZ.T @ np.abs(H64[b0:b1])
    if bounds:
        return dH, dW, bH, bW
    return dH, dW


def grad(H_bits: np.ndarray, W_bits: np.ndarray, y: np.ndarray, g: np.ndarray, m=None, ls=None,
         block: int = BLOCK_ROWS, bounds: bool = False):
    """grad64 on bf16 H and W (exact in float64)."""
    return grad64(decode_bf16(H_bits), decode_bf16(W_bits), y, g, m, ls, block, bounds)


def grad_columns(H_bits: np.ndarray, W_bits: np.ndarray, y: np.ndarray, g: np.ndarray, m: np.ndarray,
                 ls: np.ndarray, cols, block: int = BLOCK_ROWS):
    """Rows `cols` of dW (dW[v] = sum_i dZ_iv H_i) from the saved (m, ls), with dZ
    formed only for those vocabulary columns: the full-size check of dW needs every
    row of H but only a few columns of Z."""
    cols = np.asarray(cols)
    H64 = decode_bf16(H_bits)
    Wc = decode_bf16(W_bits[cols])
    y = np.asarray(y, np.int64)
    g = np.asarray(g, np.float64)
    m = np.asarray(m, np.float64)
    ls = np.asarray(ls, np.float64)
    out = np.zeros((cols.shape[0], H64.shape[1]))
    for b0 in range(0, H64.shape[0], block):
        b1 = min(H64.shape[0], b0 + block)
        Z = H64[b0:b1] @ Wc.T
        with np.errstate(invalid="ignore", over="ignore"):
            P = np.exp((Z - m[b0:b1, None]) - ls[b0:b1, None])
        onehot = (y[b0:b1, None] == cols[None, :]).astype(np.float64)
        dZ = g[b0:b1, None] * (P - onehot)
        out += dZ.T @ H64[b0:b1]
    return out
