"""Training through the IKBO LCE (broadcast_gemm_amd.autograd): the plan cache on the CPU, and on
the GPU the gradients autograd delivers against the oracle's backward (aibriefing article, the
three-layers paragraph: the same kernels serve training).  GPU bar, per element:
|g - g_ref| <= 1e-3 + 1.6e-2 |g_ref| (the backward tests' bar; dW is rounded to bf16 once, 2^-9
relative, inside it)."""
import numpy as np
import pytest
import torch

from broadcast_gemm_amd import FLAG_BACKWARD
from broadcast_gemm_amd.autograd import IkboLce, _BackwardPlans


def test_backward_plans_are_sized_by_range_and_carry_the_backward_flag():
    made = []

    class FakePlan:
        def __init__(self, mu, mc, K_u, K_c, M, D, dtype, flags):
            self.max_B_u, self.max_B_c, self.flags, self.closed = mu, mc, flags, False
            made.append(self)

        def close(self):
            self.closed = True

    t = _BackwardPlans(make_plan=FakePlan)
    p = t.plan_for(15, 1000, 301, 197, 96, 160)
    assert (p.max_B_u, p.max_B_c, p.flags) == (16, 1024, FLAG_BACKWARD)
    assert t.plan_for(9, 300, 301, 197, 96, 160) is p
    q = t.plan_for(40, 4096, 301, 197, 96, 160)
    # an outgrown plan stays usable: a graph recorded with it may still run its backward
    assert not p.closed and (q.max_B_u, q.max_B_c) == (64, 4096)
    assert t.plan_for(4, 10, 64, 32, 48, 128) is not q and len(made) == 3
    t.close()
    assert q.closed


def test_module_parameters_and_init_scale():
    m = IkboLce(301, 197, 96, 160, generator=torch.Generator().manual_seed(0))
    assert m.W_u.dtype == torch.bfloat16 and tuple(m.W_u.shape) == (96, 301) and tuple(m.W_c.shape) == (96, 197)
    w = torch.cat([m.W_u.float(), m.W_c.float()], dim=1)
    assert abs(w.std().item() * (498 ** 0.5) - 1.0) < 0.03


@pytest.mark.gpu
@pytest.mark.parametrize("shape", [(5, 37, 40, 24, 48, 160, "random"), (15, 300, 301, 197, 96, 160, "sorted")])
def test_autograd_gradients_match_oracle(shape):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import oracle
    from broadcast_gemm_amd.inputs import LceConfig, make_inputs, make_upstream_grad
    from gpu_util import assert_close, log, to_dev, to_f64
    B_u, B_c, K_u, K_c, M, D, mp = shape
    log(f"[autograd] shape={shape}")
    cfg = LceConfig("autograd", B_u, B_c, K_u, K_c, M, D, "bf16", mp, 17)
    x = make_inputs(cfg)
    dY = make_upstream_grad(cfg)
    lce = IkboLce(K_u, K_c, M, D).cuda()
    with torch.no_grad():
        lce.W_u.copy_(to_dev(x.W_u))
        lce.W_c.copy_(to_dev(x.W_c))
    U = to_dev(x.U).requires_grad_(True)
    C = to_dev(x.C).requires_grad_(True)
    Y = lce(U, C, to_dev(x.map).long())
    Y.backward(to_dev(dY))
    torch.cuda.synchronize()
    assert_close(to_f64(Y.detach()), oracle.lce_f64(x.U, x.C, x.map, x.W_u, x.W_c), "Y")
    ref = oracle.lce_backward_f64(dY, x.U, x.C, x.map, x.W_u, x.W_c)
    for name, got, want in zip(("dU", "dC", "dW_u", "dW_c"), (U.grad, C.grad, lce.W_u.grad, lce.W_c.grad), ref):
        assert got.dtype == torch.bfloat16
        assert_close(to_f64(got), want, name)
    lce._plans.close()
