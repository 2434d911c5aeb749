"""GPU: the torch.autograd wrappers give exactly what the library's own calls give.

Each loss is computed and differentiated through softmax_cross_entropy_amd.autograd, and
the loss and the gradient are compared bit for bit with the direct forward and VJP calls
(which the other GPU tests check against the float64 oracle).
"""

import numpy as np
import pytest
import torch

from softmax_cross_entropy_amd import abi, autograd, inputs
from tests.gpu_util import to_dev

pytestmark = pytest.mark.gpu


def leaf(x, dtype):
    return to_dev(x, dtype).requires_grad_()


def test_cross_entropy_plain_and_summed():
    b = inputs.normal_rows(64, 5000, "bf16", workload=60)
    x = leaf(b.logits, "bf16")
    y = torch.from_numpy(b.targets).cuda()
    g = torch.from_numpy(np.linspace(0.5, 1.5, 64).astype(np.float32)).cuda()
    loss = autograd.cross_entropy(x, y)
    loss.backward(g)
    l0, s0 = abi.ce_forward(x.detach(), y)
    d0 = abi.ce_vjp(x.detach(), y, s0, g)
    assert torch.equal(loss.detach(), l0) and torch.equal(x.grad, d0)
    # loss.sum(): the upstream gradient arrives expanded (stride 0)
    x.grad = None
    autograd.cross_entropy(x, y).sum().backward()
    assert torch.equal(x.grad, abi.ce_vjp(x.detach(), y, s0, torch.ones(64, device="cuda")))


def test_cross_entropy_options_mean():
    b = inputs.normal_rows(96, 3001, "f32", workload=61)
    x = leaf(b.logits, "f32")
    yv = b.targets.copy()
    yv[::5] = -100
    y = torch.from_numpy(yv).cuda()
    loss = autograd.cross_entropy(x, y, 0.1, -100, "mean")
    assert loss.dim() == 0
    (2.0 * loss).backward()
    l0, s0, t0, c0 = abi.ce_forward_ex(x.detach(), y, 0.1, -100, "mean")
    d0 = abi.ce_vjp_ex(x.detach(), y, s0, torch.tensor([2.0], device="cuda"), 0.1, -100, "mean", count=c0)
    assert torch.equal(loss.detach().view(1), t0) and torch.equal(x.grad, d0)
    assert torch.all(x.grad[::5] == 0).item()


def test_cross_entropy_strided_view():
    """The [B, L - 1, V] view of a leaf: the gradient lands in the leaf, zeros elsewhere."""
    B, L, V = 3, 7, 300
    b = inputs.normal_rows(B * L, V, "f32", workload=62)
    X = torch.from_numpy(b.logits.reshape(B, L, V).copy()).cuda().requires_grad_()
    yv = b.targets.reshape(B, L)[:, 1:].copy().reshape(-1)
    y = torch.from_numpy(yv).cuda()
    g = torch.from_numpy(np.linspace(1.0, 2.0, B * (L - 1)).astype(np.float32)).cuda()
    autograd.cross_entropy(X[:, :-1], y).backward(g)
    v = X.detach()[:, :-1]
    _, s0 = abi.ce_forward(v, y)
    d0 = abi.ce_vjp(v, y, s0, g)
    assert torch.equal(X.grad[:, :-1], d0) and torch.all(X.grad[:, -1] == 0).item()


def test_cross_entropy_probs_sum():
    x_np = inputs.normal_rows(40, 2000, "f32", workload=63).logits
    t_np = inputs.prob_targets(40, 2000, "f32", workload=63, stream=1)
    x = leaf(x_np, "f32")
    t = to_dev(t_np, "f32")
    loss = autograd.cross_entropy_probs(x, t, 0.1, "sum")
    loss.backward()
    l0, s0, w0, t0, c0 = abi.ce_forward_probs(x.detach(), t, 0.1, "sum")
    d0 = abi.ce_vjp_probs(x.detach(), t, s0, w0, torch.ones(1, device="cuda"), 0.1, "sum", count=c0)
    assert torch.equal(loss.detach().view(1), t0) and torch.equal(x.grad, d0)


@pytest.mark.parametrize("which", ["kl", "js"])
def test_divergences(which):
    q_np, p_np, _ = inputs.kl_pair(48, 3000, "f32", workload=64)
    q = leaf(q_np, "f32")
    p = to_dev(p_np, "f32")
    g = torch.from_numpy(np.linspace(0.5, 1.5, 48).astype(np.float32)).cuda()
    if which == "kl":
        out = autograd.kl_div(q, p)
        out.backward(g)
        o0, lq, lp = abi.kl_forward(q.detach(), p)
        d0 = abi.kl_vjp(q.detach(), p, lq, lp, g)
    else:
        out = autograd.js_div(q, p)
        out.backward(g)
        o0, lq, lp, hq = abi.js_forward(q.detach(), p)
        d0 = abi.js_vjp(q.detach(), p, lq, lp, hq, g)
    assert torch.equal(out.detach(), o0) and torch.equal(q.grad, d0)
