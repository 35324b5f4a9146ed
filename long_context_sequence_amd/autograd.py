"""PyTorch autograd wrapper: ``vla_attention`` runs ``vla_forward`` and, on
``backward()``, ``vla_backward`` (both in the HIP library); nothing else."""
from __future__ import annotations

from ._binding import vla_backward, vla_forward


def _function():
    import torch

    class VLAFunction(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, u, lambda0, eps):
            ctx.save_for_backward(q, k, v, u)
            ctx.lambda0, ctx.eps = lambda0, eps
            return vla_forward(q, k, v, u, lambda0, eps)

        @staticmethod
        def backward(ctx, dO):
            q, k, v, u = ctx.saved_tensors
            dO = dO.to(torch.float32).contiguous()
            dq, dk, dv, du, _, _, _ = vla_backward(q, k, v, u, dO, ctx.lambda0, ctx.eps,
                                                   want_state_grads=False)
            # gradients in the inputs' dtype (computed in fp32)
            return dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), du.to(u.dtype), None, None

    return VLAFunction


_FN = None


def vla_attention(q, k, v, u, lambda0: float = 0.1, eps: float = 1e-4):
    """Differentiable VLA over [B, H, T, d_h] device tensors (float32 or
    bfloat16), from the default initial state; returns o (float32)."""
    global _FN
    if _FN is None:
        _FN = _function()
    return _FN.apply(q, k, v, u, float(lambda0), float(eps))
