"""GPU parity of lce_backward against the float64 oracle.

The gradient of the logits, dZ = g (softmax(Z) - onehot(y)), is rounded to bf16 before
the two products (round to nearest even with an 8-bit significand: at most 2^-8
relative per entry), and the products accumulate in fp32.  An entry of dH = dZ W can
therefore move by at most 2^-8 (|dZ| |W|) from the exact value, and an entry of
dW = dZ^T H by 2^-8 (|dZ|^T |H|); the fp32 parts (the regenerated logits, the saved
log-sum-exp, the accumulation) add far less.  The tests allow twice that bound,
2^-7 (|dZ| |W|), plus 1e-7, with the bounds computed by the oracle from the exact dZ.
"""

import numpy as np
import pytest
import torch

from oracle import lce as olce
from softmax_cross_entropy_amd import abi, inputs
from tests.conftest import full_lce_oracle

pytestmark = pytest.mark.gpu

REL = 2.0 ** -7
FLOOR = 1e-7


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def gpu_backward(H, W, y, g, one_pass=False):
    Hd, Wd = dev_bf16(H), dev_bf16(W)
    yd = torch.from_numpy(np.ascontiguousarray(y, np.int32)).cuda()
    _, lse = abi.lce_forward(Hd, Wd, yd)
    dH, dW = abi.lce_backward(Hd, Wd, yd, lse, torch.from_numpy(np.asarray(g, np.float32)).cuda(), one_pass=one_pass)
    torch.cuda.synchronize()
    return dH.cpu().numpy().astype(np.float64), dW.cpu().numpy().astype(np.float64)


def within(got, ref, bound, what):
    err = np.abs(got - ref)
    lim = REL * bound + FLOOR
    bad = err > lim
    assert not bad.any(), (f"{what}: {bad.sum()} entries outside the bound; worst excess "
                           f"{(err - lim).max():.3e} at {np.unravel_index(np.argmax(err - lim), err.shape)}")
    return float((err / (bound + 1e-30)).max())


def upstream(N, seed):
    return np.random.default_rng(seed).uniform(0.25, 2.0, N)


@pytest.mark.parametrize("N,D,V", [
    (1, 8, 1), (3, 8, 5), (37, 40, 127), (300, 72, 1000), (257, 520, 2049), (64, 256, 513),
    (100, 64, 20000), (513, 128, 8193),
    # 3, 5 and 6 K stages in the regenerated logits (the three-buffer W ring ends in each
    # of its states), and in the products over the tokens
    (129, 136, 700), (260, 192, 1300), (70, 320, 257), (300, 384, 900),
])
def test_small_shapes(N, D, V):
    H, W, y = inputs.linear_ce(N, D, V, seed_stream=N * 11 + D + V)
    g = upstream(N, N + V)
    dH, dW = gpu_backward(H, W, y, g)
    rH, rW, bH, bW = olce.grad(H, W, y, g, bounds=True)
    eH = within(dH, rH, bH, "dH")
    eW = within(dW, rW, bW, "dW")
    print(f"N={N} D={D} V={V}: max |error| / bound: dH {eH:.2e}, dW {eW:.2e}")


def test_zero_weights():
    """W = 0: dH = dZ W is exactly 0, dW = dZ^T H with the uniform softmax."""
    N, D, V = 300, 64, 1000
    H, W, y = inputs.linear_ce(N, D, V, seed_stream=5)
    W[:] = 0
    g = upstream(N, 1)
    dH, dW = gpu_backward(H, W, y, g)
    assert np.all(dH == 0.0)
    rH, rW, bH, bW = olce.grad(H, W, y, g, bounds=True)
    within(dW, rW, bW, "dW")


def test_invalid_target_rows_are_nan_and_zero_g_rows_are_zero():
    N, D, V = 260, 96, 700
    H, W, y = inputs.linear_ce(N, D, V, seed_stream=2)
    g = upstream(N, 3)
    g[[10, 11]] = 0.0
    dH, dW = gpu_backward(H, W, y, g)
    assert np.all(dH[[10, 11]] == 0.0)
    y2 = y.copy()
    y2[7] = V
    dH2, dW2 = gpu_backward(H, W, y2, g)
    assert np.isnan(dH2[7]).all()
    assert np.isnan(dW2).all()
    ok = np.setdiff1d(np.arange(N), [7])
    assert np.isfinite(dH2[ok]).all()


def test_repeat_is_bitwise_stable():
    N, D, V = 300, 128, 9000
    H, W, y = inputs.linear_ce(N, D, V, seed_stream=9)
    g = upstream(N, 4)
    a = gpu_backward(H, W, y, g)
    b = gpu_backward(H, W, y, g)
    assert np.array_equal(a[0].view(np.uint64), b[0].view(np.uint64))
    assert np.array_equal(a[1].view(np.uint64), b[1].view(np.uint64))


def test_empty_batch_writes_zero_dw():
    D, V = 64, 1000
    W = dev_bf16(inputs.linear_ce(1, D, V, seed_stream=1)[1])
    H = torch.empty(0, D, dtype=torch.bfloat16, device="cuda")
    dW = torch.full((V, D), float("nan"), device="cuda")
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    abi.lce_backward(H, W, e, torch.empty(0, 2, device="cuda"), torch.empty(0, device="cuda"), dW=dW)
    torch.cuda.synchronize()
    assert torch.all(dW == 0).item()


def test_full_vocab_and_width_one_row_tile():
    """N = 256 at the full V = 151,936 and D = 4096: every chunk, including the
    4480-column tail; dH everywhere and dW on sampled vocabulary rows."""
    N, D, V = 256, 4096, 151936
    H, W, y = inputs.linear_ce(N, D, V, seed_stream=12)
    g = upstream(N, 12)
    dH, dW = gpu_backward(H, W, y, g)
    W64 = olce.decode_bf16(W)
    _, m, ls = olce.forward(H, W, y, W64=W64)
    rng = np.random.default_rng(0)
    cols = np.unique(np.concatenate([rng.integers(0, V, 24), y[:8], [0, 8191, 8192, V - 4480, V - 1]]))
    rW = olce.grad_columns(H, W, y, g, m, ls, cols)
    rows = np.unique(np.concatenate([rng.integers(0, N, 6), [0, N - 1]]))
    H64 = olce.decode_bf16(H)
    rH, _, bH, _ = olce.grad64(H64[rows], W64, y[rows], g[rows], bounds=True)
    within(dH[rows], rH, bH, "dH rows")
    # |dZ|^T |H| for the sampled columns, from the exact dZ of those columns
    Wc = olce.decode_bf16(W[cols])
    Z = H64 @ Wc.T
    dZc = g[:, None] * (np.exp((Z - m[:, None]) - ls[:, None]) - (y[:, None] == cols[None, :]))
    within(dW[cols], rW, np.abs(dZc).T @ np.abs(H64), "dW columns")


@pytest.mark.parametrize("N,D,V", [(100, 64, 20000), (513, 128, 8193), (37, 40, 16385), (300, 72, 24577)])
def test_one_pass_matches_chunks(N, D, V):
    """A workspace of lce_backward_workspace_size_one_pass bytes runs the whole vocabulary
    as one chunk: dH written once, one launch of each product.  Its dH and dW equal the
    chunked call's bit for bit, and the oracle's within the bound."""
    H, W, y = inputs.linear_ce(N, D, V, seed_stream=N * 7 + D + V)
    g = upstream(N, N + 2 * V)
    assert abi.lce_backward_workspace_size_one_pass(N, D, V) > abi.lce_backward_workspace_size(N, D, V)
    cH, cW = gpu_backward(H, W, y, g)
    oH, oW = gpu_backward(H, W, y, g, one_pass=True)
    assert np.array_equal(cH, oH) and np.array_equal(cW, oW)
    rH, rW, bH, bW = olce.grad(H, W, y, g, bounds=True)
    within(oH, rH, bH, "dH")
    within(oW, rW, bW, "dW")


def test_bench_size_sampled_rows_columns_and_column_sum(full_lce):
    """N = 8192, D = 4096, V = 151,936 as bench.py runs it:
    * the call in chunks of 8192 columns and in one chunk (bench.py's layout), bit for bit;
    * dH on 64 sampled rows against the oracle, entry by entry;
    * dW on 72 sampled vocabulary rows against the oracle, entry by entry: the first and
      last columns of every 8192-column chunk boundary they touch, targets, and 24
      columns of the 4480-column tail chunk;
    * every row of dW summing to zero (every row of dZ sums to zero; the bf16 rounding
      of dZ leaves at most 2^-8 sum_v |dZ_iv| <= 2^-7 g_i per row; twice that allowed)."""
    H, W, y, W64 = full_lce["H"], full_lce["W"], full_lce["y"], full_lce["W64"]
    N, D = H.shape
    V = W.shape[0]
    g = upstream(N, 8192)
    Hd, Wd = dev_bf16(H), dev_bf16(W)
    yd = torch.from_numpy(np.ascontiguousarray(y, np.int32)).cuda()
    _, lse = abi.lce_forward(Hd, Wd, yd)
    gd = torch.from_numpy(g.astype(np.float32)).cuda()
    dHd, dWd = abi.lce_backward(Hd, Wd, yd, lse, gd)
    # one chunk over the whole vocabulary (the layout bench.py times) gives the same bits
    oH, oW = abi.lce_backward(Hd, Wd, yd, lse, gd, one_pass=True)
    torch.cuda.synchronize()
    assert torch.equal(oH.view(torch.int32), dHd.view(torch.int32))
    assert torch.equal(oW.view(torch.int32), dWd.view(torch.int32))
    del oH, oW
    dH = dHd.cpu().numpy().astype(np.float64)
    assert np.isfinite(dH).all() and torch.isfinite(dWd).all().item()
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([rng.choice(N, 62, replace=False), [0, N - 1]]))
    H64 = olce.decode_bf16(H)
    rH, _, bH, _ = olce.grad64(H64[rows], W64, y[rows], g[rows], bounds=True)
    within(dH[rows], rH, bH, "dH rows")
    tail0 = V - V % 8192
    cols = np.unique(np.concatenate([[0, 8191, 8192, 16383, 16384, tail0 - 1, tail0, V - 1], y[:16],
                                     rng.integers(0, tail0, 24), rng.integers(tail0, V, 24)]))
    assert len(cols) >= 64 and np.sum(cols >= tail0) >= 24
    _, m, ls = full_lce_oracle(full_lce)
    rW = olce.grad_columns(H, W, y, g, m, ls, cols)
    dWc = dWd[torch.from_numpy(cols).cuda()].cpu().numpy().astype(np.float64)
    Z = H64 @ W64[cols].T
    dZc = g[:, None] * (np.exp((Z - m[:, None]) - ls[:, None]) - (y[:, None] == cols[None, :]))
    within(dWc, rW, np.abs(dZc).T @ np.abs(H64), "dW columns")
    colsum = dWd.sum(dim=0, dtype=torch.float64).cpu().numpy()
    lim = 2.0 ** -6 * (np.abs(g)[:, None] * np.abs(H64)).sum(axis=0) + 1e-3
    assert np.all(np.abs(colsum) <= lim), float((np.abs(colsum) / lim).max())


def test_deepest_reduction():
    """D = 2^22, the largest depth the call accepts: the regenerated logits take 65,536 K
    stages, H^T and the W chunk's transpose have 2^22 rows, and dH and dW 2^22 columns."""
    N, D, V = 3, 1 << 22, 5
    H, W, y = inputs.linear_ce(N, D, V, seed_stream=23)
    g = upstream(N, 3)
    dH, dW = gpu_backward(H, W, y, g)
    rH, rW, bH, bW = olce.grad(H, W, y, g, bounds=True)
    eH = within(dH, rH, bH, "dH")
    eW = within(dW, rW, bW, "dW")
    print(f"D = 2^22: max |error| / bound: dH {eH:.2e}, dW {eW:.2e}")
