"""torch.autograd integration of the library's losses.

Each function's forward calls the library's forward through `abi` and saves what its VJP
needs (the logits, the (m, log s) pairs, the weight sums, the count of a mean); its
backward calls the library's VJP with the upstream gradient.  Nothing is computed here:
the only torch operation is making a strided upstream gradient contiguous.  The losses
and the VJP they differentiate:

  cross_entropy        ce_forward / ce_vjp, or ce_forward_ex / ce_vjp_ex with label
                       smoothing, ignore_index or a sum / mean reduction
  cross_entropy_probs  ce_forward_probs / ce_vjp_probs (probability targets; no gradient
                       for the targets)
  kl_div, js_div       kl_forward / kl_vjp and js_forward / js_vjp (gradient for the
                       student q only, as the pages' kernels define it)

MLX PR #4188 "Shift by the max in cross_entropy", Proposed changes (the options);
"One barrier short", Run it yourself (the divergences and their student gradient);
Ineshin, "A fused linear cross-entropy forward kernel for Apple GPUs", section 1 (the
backward reuses the forward's saved log-sum-exp).
"""

import torch

from . import abi


def _upstream(grad: torch.Tensor, reduced: bool) -> torch.Tensor:
    g = grad.reshape(1) if reduced else grad
    return g if g.is_contiguous() else g.contiguous()


class _CrossEntropy(torch.autograd.Function):
    @staticmethod
    def forward(ctx, logits, targets, label_smoothing, ignore_index, reduction):
        ctx.opts = (label_smoothing, ignore_index, reduction)
        ctx.plain = label_smoothing == 0.0 and ignore_index is None and reduction == "none"
        if ctx.plain:
            loss, lse = abi.ce_forward(logits, targets)
            ctx.save_for_backward(logits, targets, lse)
            return loss
        loss, lse, total, count = abi.ce_forward_ex(logits, targets, label_smoothing, ignore_index, reduction)
        ctx.save_for_backward(logits, targets, lse, count)
        return loss if reduction == "none" else total.view(())

    @staticmethod
    def backward(ctx, grad):
        label_smoothing, ignore_index, reduction = ctx.opts
        if ctx.plain:
            logits, targets, lse = ctx.saved_tensors
            d = abi.ce_vjp(logits, targets, lse, _upstream(grad, False))
        else:
            logits, targets, lse, count = ctx.saved_tensors
            d = abi.ce_vjp_ex(logits, targets, lse, _upstream(grad, reduction != "none"), label_smoothing,
                              ignore_index, reduction, count=count)
        return d, None, None, None, None


class _CrossEntropyProbs(torch.autograd.Function):
    @staticmethod
    def forward(ctx, logits, probs, label_smoothing, reduction):
        ctx.opts = (label_smoothing, reduction)
        loss, lse, wsum, total, count = abi.ce_forward_probs(logits, probs, label_smoothing, reduction)
        ctx.save_for_backward(logits, probs, lse, wsum, count)
        return loss if reduction == "none" else total.view(())

    @staticmethod
    def backward(ctx, grad):
        label_smoothing, reduction = ctx.opts
        logits, probs, lse, wsum, count = ctx.saved_tensors
        d = abi.ce_vjp_probs(logits, probs, lse, wsum, _upstream(grad, reduction != "none"), label_smoothing,
                             reduction, count=count)
        return d, None, None, None


class _KLDiv(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, p):
        kl, lq, lp = abi.kl_forward(q, p)
        ctx.save_for_backward(q, p, lq, lp)
        return kl

    @staticmethod
    def backward(ctx, grad):
        q, p, lq, lp = ctx.saved_tensors
        return abi.kl_vjp(q, p, lq, lp, _upstream(grad, False)), None


class _JSDiv(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, p):
        js, lq, lp, hq = abi.js_forward(q, p)
        ctx.save_for_backward(q, p, lq, lp, hq)
        return js

    @staticmethod
    def backward(ctx, grad):
        q, p, lq, lp, hq = ctx.saved_tensors
        return abi.js_vjp(q, p, lq, lp, hq, _upstream(grad, False)), None


def cross_entropy(logits: torch.Tensor, targets: torch.Tensor, label_smoothing: float = 0.0, ignore_index=None,
                  reduction: str = "none") -> torch.Tensor:
    """Per-row losses ([n], reduction 'none') or their sum or mean (0-dim) of a [rows, V]
    or [B, L, V] logits view with int32 class targets; differentiable in the logits."""
    return _CrossEntropy.apply(logits, targets, float(label_smoothing), ignore_index, reduction)


def cross_entropy_probs(logits: torch.Tensor, probs: torch.Tensor, label_smoothing: float = 0.0,
                        reduction: str = "none") -> torch.Tensor:
    """The loss with probability targets of the logits' dtype; differentiable in the logits."""
    return _CrossEntropyProbs.apply(logits, probs, float(label_smoothing), reduction)


def kl_div(q: torch.Tensor, p: torch.Tensor) -> torch.Tensor:
    """Per-row KL divergence of the teacher softmax(p) from the student softmax(q);
    differentiable in q."""
    return _KLDiv.apply(q, p)


def js_div(q: torch.Tensor, p: torch.Tensor) -> torch.Tensor:
    """Per-row Jensen-Shannon divergence of softmax(q) and softmax(p); differentiable in q."""
    return _JSDiv.apply(q, p)
