"""Training through the IKBO LCE: a torch.autograd.Function over the library's forward and
backward, and a module that owns the projections.

The pages say the same kernels serve training once the ratio of candidates to users exceeds one
(aibriefing article, the paragraph on the three layers of the stack).  Forward and backward both
run in ``libikbo`` (``ikbo_lce_forward`` / ``ikbo_lce_backward``); the gradients are those of

    Y[b] = W_u . U[map[b]] + W_c . C[b]

(dC[b] = W_c^T dY[b], dU[u] = W_u^T S[u], dW_c = sum_b dY[b] C[b]^T, dW_u = sum_u S[u] U[u]^T with
S[u] the sum of dY over the candidates of user u).  The library returns dW_u and dW_c in float32;
autograd wants a gradient in its parameter's dtype, so they are rounded to it once (the only
step outside the library, a dtype conversion).

    lce = IkboLce(K_u, K_c, M, D).cuda()           # W_u, W_c: bf16 parameters
    Y = lce(U, C, map)                               # U, C may require grad
    Y.backward(dY)                                   # lce.W_u.grad, lce.W_c.grad, U.grad, C.grad
"""
from __future__ import annotations

from typing import Dict, Tuple

import torch

from . import FLAG_BACKWARD, LcePlan
from .rewrite import bucket_b_c, bucket_b_u


class _BackwardPlans:
    """Plans with the backward's workspace, keyed by (K_u, K_c, M, D), each sized to a batch range.

    A plan that a larger batch outgrows is dropped, not destroyed: autograd graphs recorded
    with it may still run their backward, and it is freed once none refers to it."""

    def __init__(self, make_plan=LcePlan):
        self._make = make_plan
        self._plans: Dict[Tuple[int, int, int, int], object] = {}

    def plan_for(self, B_u: int, B_c: int, K_u: int, K_c: int, M: int, D: int):
        key = (K_u, K_c, M, D)
        plan = self._plans.get(key)
        if plan is None or plan.max_B_u < B_u or plan.max_B_c < B_c:
            mu, mc = bucket_b_u(B_u), bucket_b_c(B_c)
            if plan is not None:
                mu, mc = max(mu, plan.max_B_u), max(mc, plan.max_B_c)
            plan = self._make(mu, mc, K_u, K_c, M, D, dtype="bf16", flags=FLAG_BACKWARD)
            self._plans[key] = plan
        return plan

    def close(self) -> None:
        for plan in self._plans.values():
            plan.close()
        self._plans.clear()


class LceFunction(torch.autograd.Function):
    """Y = W_u . U[map] + W_c . C with both directions in the library (bf16 tensors on the GPU)."""

    @staticmethod
    def forward(ctx, U, C, mp, W_u, W_c, plans: _BackwardPlans):
        B_u, K_u, D = U.shape
        B_c, K_c, _ = C.shape
        plan = plans.plan_for(B_u, B_c, K_u, K_c, W_u.shape[0], D)
        mp32 = mp.to(torch.int32).contiguous()
        U, C, W_u, W_c = (t.contiguous() for t in (U, C, W_u, W_c))
        Y = plan.forward(U, C, mp32, W_u, W_c)
        ctx.save_for_backward(U, C, mp32, W_u, W_c)
        ctx.plan = plan
        return Y

    @staticmethod
    def backward(ctx, dY):
        U, C, mp32, W_u, W_c = ctx.saved_tensors
        dU, dC, dW_u, dW_c = ctx.plan.backward(dY.contiguous(), U, C, mp32, W_u, W_c)
        need = ctx.needs_input_grad
        return (dU if need[0] else None, dC if need[1] else None, None,
                dW_u.to(W_u.dtype) if need[3] else None, dW_c.to(W_c.dtype) if need[4] else None, None)


class IkboLce(torch.nn.Module):
    """The LCE layer with trainable projections W_u [M, K_u] and W_c [M, K_c] (bf16).

    Initialised with standard deviation 1/sqrt(K_u + K_c), so that Y has about unit variance for
    unit-variance inputs."""

    def __init__(self, K_u: int, K_c: int, M: int, D: int, generator=None):
        super().__init__()
        std = (K_u + K_c) ** -0.5
        self.W_u = torch.nn.Parameter((torch.randn(M, K_u, generator=generator) * std).to(torch.bfloat16))
        self.W_c = torch.nn.Parameter((torch.randn(M, K_c, generator=generator) * std).to(torch.bfloat16))
        self.D = D
        self._plans = _BackwardPlans()

    def forward(self, U, C, mp):
        return LceFunction.apply(U, C, mp, self.W_u, self.W_c, self._plans)
