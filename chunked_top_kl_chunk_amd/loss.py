"""torch autograd wrapper of the fused chunked top-K KL loss.

``FusedChunkedKLLoss`` is the module the pages configure in place of a stock PyTorch
loss ("Configuring Fused Chunked KL Loss", getaibook.com): it takes the student's
final hidden states and LM head (the output projection is part of the loss,
"What actually changed?", calcaas.com) and the teacher's cached top-K logits and
indices.  Its forward pass is ``fckl_forward_ex`` and its backward pass
``fckl_backward_ex``; the upstream gradient stays on the device.  Both passes run in
the library's HIP kernels; nothing here computes any part of the loss.

Token masks (padding, ignored positions) and per-token weights enter through the
weighted mean sum_i w_i loss_i / sum_i w_i; a masked token has w = 0.

The library computes dH and dW in float32; autograd hands them to h and W in those
tensors' dtype (bf16), as it does for any gradient.  A caller that keeps an fp32
master copy of W can call ``chunked_top_kl_chunk_amd.backward`` with
``accumulate=True`` on that buffer instead.

With ``single_call=True`` the forward pass runs ``fckl_forward_backward`` (each chunk's
logits formed once, 6 N V H flop instead of 8) with an upstream gradient of 1 and keeps
dH and dW (float32, N H + V H values) until the backward pass, which scales them in
place by the upstream gradient with ``fckl_scale`` on the device.  The gradients are
those of the two-pass path up to the bf16 rounding of the kept exponentials.

``FullTeacherKLLoss`` is the same kind of module for online distillation against the
teacher's whole distribution (``fckl_full_forward_backward``): it takes the teacher's
final hidden states and LM head instead of a cache.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import backward as _backward
from . import forward as _forward
from . import forward_backward as _forward_backward
from . import full_forward_backward as _full_forward_backward
from . import scale_ as _scale_


class FusedChunkedKLFunction(torch.autograd.Function):
    """loss = weighted mean over tokens of T^2 KL(p_teacher || softmax(h W^T / T)) over the K cached entries."""

    @staticmethod
    def forward(ctx, h, W, topk_idx, topk_logit, weights, T: float, chunk: int):
        _, lse, mean = _forward(h.detach(), W.detach(), topk_idx, topk_logit, T=T, chunk=chunk, weights=weights)
        ctx.save_for_backward(h, W, topk_idx, topk_logit, lse)
        ctx.weights = weights
        ctx.T, ctx.chunk = T, chunk
        return mean.reshape(())

    @staticmethod
    def backward(ctx, grad_out):
        h, W, topk_idx, topk_logit, lse = ctx.saved_tensors
        if not (ctx.needs_input_grad[0] or ctx.needs_input_grad[1]):
            return None, None, None, None, None, None, None
        g = grad_out.detach().to(torch.float32).reshape(1).contiguous()
        dH, dW = _backward(h.detach(), W.detach(), topk_idx, topk_logit, lse, T=ctx.T, chunk=ctx.chunk,
                           weights=ctx.weights, grad_scale=1.0, grad_scale_dev=g)
        return (dH if ctx.needs_input_grad[0] else None, dW if ctx.needs_input_grad[1] else None,
                None, None, None, None, None)


class FusedChunkedKLSingleCallFunction(torch.autograd.Function):
    """The same loss with both passes in the forward call; backward only scales."""

    @staticmethod
    def forward(ctx, h, W, topk_idx, topk_logit, weights, T: float, chunk: int):
        _, _, mean, dH, dW = _forward_backward(h.detach(), W.detach(), topk_idx, topk_logit, T=T, grad_scale=1.0,
                                               weights=weights, chunk=chunk)
        ctx.dH, ctx.dW = dH, dW
        return mean.reshape(())

    @staticmethod
    def backward(ctx, grad_out):
        dH, dW = ctx.dH, ctx.dW
        ctx.dH = ctx.dW = None
        g = grad_out.detach().to(torch.float32).reshape(1).contiguous()
        if ctx.needs_input_grad[0]:
            _scale_(dH, g)
        if ctx.needs_input_grad[1]:
            _scale_(dW, g)
        return (dH if ctx.needs_input_grad[0] else None, dW if ctx.needs_input_grad[1] else None,
                None, None, None, None, None)


class FusedChunkedKLLoss(torch.nn.Module):
    """Fused chunked KL distillation loss against a cached top-K teacher.

    Args:
        temperature: T; student and teacher logits are divided by it and the loss is
            scaled by T^2.
        chunk: tokens per chunk (0 = the library's scheduler).
        ignore_index: topk_idx rows whose first entry equals this value are masked
            (their other entries are then not read as indices; they must still be in
            [0, V) or be replaced by the caller).  None = no such convention.
        single_call: form the gradients in the forward call (fckl_forward_backward)
            and only scale them in the backward call; for a loss whose backward
            follows its forward once (the usual training step).

    forward(hidden [.., H] bf16, lm_head_weight [V, H] bf16, topk_idx [.., K] int32,
            topk_logit [.., K] bf16/f32, mask [..] bool (True = keep) or None,
            weights [..] float or None) -> scalar loss (float32).

    At least one token is needed: an empty batch raises FCKLError (ERR_INVALID_ARG), as
    the library refuses N = 0.  A batch whose tokens are all masked gives a loss of 0
    and zero gradients.
    """

    def __init__(self, temperature: float = 1.0, chunk: int = 0, ignore_index: Optional[int] = None,
                 single_call: bool = False):
        super().__init__()
        if not temperature > 0:
            raise ValueError("temperature must be > 0")
        self.temperature = float(temperature)
        self.chunk = int(chunk)
        self.ignore_index = ignore_index
        self.single_call = bool(single_call)

    def forward(self, hidden, lm_head_weight, topk_idx, topk_logit, mask=None, weights=None):
        H = hidden.shape[-1]
        K = topk_idx.shape[-1]
        h = hidden.reshape(-1, H)
        N = h.shape[0]
        idx = topk_idx.reshape(N, K)
        tl = topk_logit.reshape(N, K)
        w = None
        if weights is not None:
            w = weights.reshape(N).to(torch.float32)
        if mask is not None:
            m = mask.reshape(N).to(torch.float32)
            w = m if w is None else w * m
        if self.ignore_index is not None:
            keep = idx[:, 0] != self.ignore_index
            w = keep.to(torch.float32) if w is None else w * keep.to(torch.float32)
            # ignored rows get a valid placeholder index row; their weight is 0
            idx = torch.where(keep[:, None], idx, torch.arange(K, device=idx.device, dtype=idx.dtype)[None, :])
        if w is not None:
            # masked and ignored rows get finite placeholder logits too (padding rows often
            # hold -inf or NaN there); with weight 0 they reach neither the mean nor a gradient
            tl = torch.where((w != 0)[:, None], tl, torch.zeros((), dtype=tl.dtype, device=tl.device))
        wants_grad = torch.is_grad_enabled() and (hidden.requires_grad or lm_head_weight.requires_grad)
        fn = FusedChunkedKLSingleCallFunction if self.single_call and wants_grad else FusedChunkedKLFunction
        return fn.apply(h.contiguous(), lm_head_weight.contiguous(), idx.contiguous(), tl.contiguous(),
                        None if w is None else w.contiguous(), self.temperature, self.chunk)


class FullTeacherKLFunction(torch.autograd.Function):
    """KL against the teacher's whole distribution; gradients formed in the forward call."""

    @staticmethod
    def forward(ctx, h, W, h_t, W_t, weights, T: float, chunk: int, want_grad: bool):
        _, _, mean, dH, dW = _full_forward_backward(h.detach(), W.detach(), h_t.detach(), W_t.detach(), T=T,
                                                    grad_scale=1.0, weights=weights, chunk=chunk)
        ctx.dH, ctx.dW = (dH, dW) if want_grad else (None, None)
        return mean.reshape(())

    @staticmethod
    def backward(ctx, grad_out):
        dH, dW = ctx.dH, ctx.dW
        ctx.dH = ctx.dW = None
        g = grad_out.detach().to(torch.float32).reshape(1).contiguous()
        if ctx.needs_input_grad[0]:
            _scale_(dH, g)
        if ctx.needs_input_grad[1]:
            _scale_(dW, g)
        return (dH if ctx.needs_input_grad[0] else None, dW if ctx.needs_input_grad[1] else None,
                None, None, None, None, None, None)


class FullTeacherKLLoss(torch.nn.Module):
    """Online distillation against the teacher's whole distribution (the setting the
    cached top-K teacher replaces, "The Distillation Bottleneck", getaibook.com):
    loss = weighted mean over tokens of T^2 KL(softmax(h_t W_t^T / T) || softmax(h W^T / T)).
    The teacher's final hidden states and LM head are inputs and get no gradient; the
    forward call runs fckl_full_forward_backward and keeps dH and dW, which the backward
    call scales by the upstream gradient on the device (fckl_scale).

    forward(hidden [.., H] bf16, lm_head_weight [V, H] bf16, teacher_hidden [.., Ht] bf16,
            teacher_lm_head_weight [V, Ht] bf16, mask [..] bool or None, weights [..] or None)
            -> scalar loss (float32).
    """

    def __init__(self, temperature: float = 1.0, chunk: int = 0):
        super().__init__()
        if not temperature > 0:
            raise ValueError("temperature must be > 0")
        self.temperature = float(temperature)
        self.chunk = int(chunk)

    def forward(self, hidden, lm_head_weight, teacher_hidden, teacher_lm_head_weight, mask=None, weights=None):
        H, Ht = hidden.shape[-1], teacher_hidden.shape[-1]
        h = hidden.reshape(-1, H)
        ht = teacher_hidden.reshape(-1, Ht)
        N = h.shape[0]
        w = None
        if weights is not None:
            w = weights.reshape(N).to(torch.float32)
        if mask is not None:
            m = mask.reshape(N).to(torch.float32)
            w = m if w is None else w * m
        want_grad = torch.is_grad_enabled() and (hidden.requires_grad or lm_head_weight.requires_grad)
        return FullTeacherKLFunction.apply(h.contiguous(), lm_head_weight.contiguous(), ht.contiguous(),
                                           teacher_lm_head_weight.contiguous(), None if w is None else w.contiguous(),
                                           self.temperature, self.chunk, want_grad)


__all__ = ["FusedChunkedKLFunction", "FusedChunkedKLSingleCallFunction", "FusedChunkedKLLoss",
           "FullTeacherKLFunction", "FullTeacherKLLoss"]
