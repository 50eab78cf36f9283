"""The inference-time rewrite (broadcast_gemm_amd.rewrite): pattern matching and plan
ranges on the CPU, and the rewritten graph against the oracle on the GPU.

The pass swaps a materialised broadcast followed by one GEMM (IKBO recsys blog, the
co-design section and FAQ; aibriefing article, the three-layers paragraph: inference-time
transformation) for the IKBO forward; the GPU check holds it to the parity bar
|Y - Y_ref| <= 1e-3 + 1.6e-2 |Y_ref| against the fp64 oracle.
"""
import operator

import pytest
import torch
import torch.fx as fx

from broadcast_gemm_amd import rewrite as rw


class CatThenMatmul(torch.nn.Module):
    def __init__(self, W, gather="getitem", order="user_first", mm="matmul", dim=1):
        super().__init__()
        self.W = torch.nn.Parameter(W, requires_grad=False)
        self.gather, self.order, self.mm, self.dim = gather, order, mm, dim

    def forward(self, U, C, mp):
        if self.gather == "getitem":
            g = U[mp]
        elif self.gather == "index_select":
            g = torch.index_select(U, 0, mp)
        else:
            g = U.index_select(0, mp)
        parts = [g, C] if self.order == "user_first" else [C, g]
        X = torch.cat(parts, dim=self.dim)
        if self.mm == "matmul":
            return torch.matmul(self.W, X)
        if self.mm == "at":
            return self.W @ X
        return torch.bmm(self.W.expand(X.shape[0], -1, -1), X)


def small(order="user_first"):
    B_u, B_c, K_u, K_c, M, D = 3, 7, 5, 4, 6, 8
    g = torch.Generator().manual_seed(5)
    U, C = torch.randn(B_u, K_u, D, generator=g), torch.randn(B_c, K_c, D, generator=g)
    mp = torch.randint(0, B_u, (B_c,), generator=g)
    W = torch.randn(M, K_u + K_c, generator=g)
    return U, C, mp, W


def calls(gm, target):
    return [n for n in gm.graph.nodes if n.op == "call_function" and n.target is target]


@pytest.mark.parametrize("gather", ["getitem", "index_select", "method"])
@pytest.mark.parametrize("mm", ["matmul", "at", "bmm"])
@pytest.mark.parametrize("order", ["user_first", "candidate_first"])
def test_rewrite_replaces_the_materialised_pattern(gather, mm, order):
    U, C, mp, W = small()
    if order == "candidate_first":
        W = torch.cat([W[:, U.shape[1]:], W[:, :U.shape[1]]], dim=1)   # [W_c | W_u]
    m = CatThenMatmul(W, gather, order, mm)
    gm = fx.symbolic_trace(m)
    assert rw.rewrite_lce(gm, U, C, mp) == 1
    (node,) = calls(gm, rw.ikbo_lce)
    assert not calls(gm, torch.cat) and not calls(gm, torch.matmul) and not calls(gm, torch.bmm)
    assert not calls(gm, operator.matmul)
    # the new call takes (U, C, map, W_u, W_c) with W split at U's K
    u, c, p, wu, wc = node.args
    assert (u.target, c.target, p.target) == ("U", "C", "mp")
    K_u = U.shape[1]
    W_u, W_c = getattr(gm, wu.target), getattr(gm, wc.target)
    if order == "user_first":
        assert torch.equal(W_u, W[:, :K_u]) and torch.equal(W_c, W[:, K_u:])
    else:
        assert torch.equal(W_c, W[:, :C.shape[1]]) and torch.equal(W_u, W[:, C.shape[1]:])
    assert W_u.is_contiguous() and W_c.is_contiguous()


def test_rewritten_graph_computes_the_same_decomposition_on_cpu(monkeypatch):
    # With the library call swapped for the plain decomposed product (test only), the
    # rewritten graph reproduces the original module: the rewrite keeps the math.
    U, C, mp, W = small()
    m = CatThenMatmul(W)
    gm = fx.symbolic_trace(m)
    rw.rewrite_lce(gm, U, C, mp)
    ref = m(U, C, mp)
    for node in calls(gm, rw.ikbo_lce):
        node.target = lambda U_, C_, mp_, Wu, Wc: torch.matmul(Wu, U_[mp_]) + torch.matmul(Wc, C_)
    gm.recompile()
    assert torch.allclose(gm(U, C, mp), ref, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("case", ["cat_dim2", "both_gathered", "none_gathered", "w_on_right", "k_mismatch"])
def test_rewrite_leaves_other_graphs_alone(case):
    U, C, mp, W = small()

    M, K_u, K_c = W.shape[0], U.shape[1], C.shape[1]
    widths = {"cat_dim2": K_u, "both_gathered": 2 * K_u, "none_gathered": 2 * K_c, "w_on_right": K_u + K_c,
              "k_mismatch": K_u + K_c - 1}

    class Other(torch.nn.Module):
        def __init__(self):
            super().__init__()
            self.W = torch.nn.Parameter(torch.randn(M, widths[case]), requires_grad=False)

        def forward(self, U, C, mp):
            if case == "cat_dim2":
                return torch.matmul(self.W, torch.cat([U[mp], U[mp]], dim=2))
            if case == "both_gathered":
                return torch.matmul(self.W, torch.cat([U[mp], U[mp]], dim=1))
            if case == "none_gathered":
                return torch.matmul(self.W, torch.cat([C, C], dim=1))
            if case == "w_on_right":
                return torch.matmul(torch.cat([U[mp], C], dim=1).transpose(1, 2), self.W.t())
            return torch.matmul(self.W, torch.cat([U[mp], C], dim=1))

    gm = fx.symbolic_trace(Other())
    if case == "k_mismatch":
        with pytest.raises(RuntimeError):
            gm(U, C, mp)                      # the shapes do not even multiply: nothing to rewrite
        return
    assert rw.rewrite_lce(gm, U, C, mp) == 0
    assert not calls(gm, rw.ikbo_lce)


def test_plan_table_sizes_plans_by_shape_range():
    made = []

    class FakePlan:
        def __init__(self, mu, mc, K_u, K_c, M, D, dtype, variant):
            self.max_B_u, self.max_B_c, self.closed = mu, mc, False
            made.append(self)

        def close(self):
            self.closed = True

    t = rw.PlanTable(make_plan=FakePlan)
    p1 = t.plan_for(15, 1000, 301, 197, 96, 160, "bf16")
    assert (p1.max_B_u, p1.max_B_c) == (16, 1024)
    assert t.plan_for(12, 1024, 301, 197, 96, 160, "bf16") is p1           # same range: reused
    p2 = t.plan_for(40, 300, 301, 197, 96, 160, "bf16")                    # more users: regrow
    assert p1.closed and (p2.max_B_u, p2.max_B_c) == (64, 1024)
    p3 = t.plan_for(2, 20000, 509, 251, 128, 128, "bf16")                  # another shape: own plan
    assert (p3.max_B_u, p3.max_B_c) == (16, 20480) and not p2.closed
    assert [rw.bucket_b_c(b) for b in (1, 256, 257, 4096, 4097)] == [256, 256, 512, 4096, 8192]


@pytest.mark.gpu
def test_rewritten_module_matches_oracle_on_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import numpy as np

    import oracle
    from broadcast_gemm_amd.inputs import CONFIG_BY_NAME, make_inputs
    from gpu_util import assert_close, to_dev, to_f64
    x = make_inputs(CONFIG_BY_NAME["small-10to1"])
    U, C, mp, W_u, W_c = to_dev(x.U), to_dev(x.C), to_dev(x.map), to_dev(x.W_u), to_dev(x.W_c)
    m = CatThenMatmul(torch.cat([W_u, W_c], dim=1)).cuda()
    gm = fx.symbolic_trace(m)
    assert rw.rewrite_lce(gm, U, C, mp.long()) == 1
    Y = gm(U, C, mp.long())
    assert rw.plan_table().check_all() == 0
    assert_close(to_f64(Y), oracle.lce_f64(x.U, x.C, x.map, x.W_u, x.W_c), "rewritten module")
