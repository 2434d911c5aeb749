"""Float64 oracle for the linear cross-entropy forward.

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
