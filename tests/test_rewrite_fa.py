"""The inference-time rewrite of target attention over a broadcast K/V
(broadcast_gemm_amd.rewrite.rewrite_attention): matching on the CPU, and the rewritten
module against the oracle on the GPU (IKBO recsys blog, "Deep Dive: Flash Attention";
aibriefing article, the three-layers paragraph: inference-time transformation).  GPU bar:
|O - O_ref| <= 1e-3 + 1.6e-2 |O_ref| + 2^-8 sum_k w_k |V_k| (the attention bar)."""
import pytest
import torch
import torch.fx as fx
import torch.nn.functional as F

from broadcast_gemm_amd import rewrite as rw


class TargetAttention(torch.nn.Module):
    def __init__(self, gather="getitem", scale=None, variant="plain"):
        super().__init__()
        self.gather, self.scale, self.variant = gather, scale, variant

    def forward(self, Q, K, V, mp):
        if self.gather == "getitem":
            Kb, Vb = K[mp], V[mp]
        else:
            Kb, Vb = torch.index_select(K, 0, mp), torch.index_select(V, 0, mp)
        if self.variant == "causal":
            return F.scaled_dot_product_attention(Q, Kb, Vb, is_causal=True)
        if self.variant == "mask":
            return F.scaled_dot_product_attention(Q, Kb, Vb, attn_mask=torch.ones(1, dtype=torch.bool))
        if self.variant == "k_only":
            return F.scaled_dot_product_attention(Q, Kb, V[torch.zeros_like(mp)])
        if self.scale is None:
            return F.scaled_dot_product_attention(Q, Kb, Vb)
        return F.scaled_dot_product_attention(Q, Kb, Vb, scale=self.scale)


def small(dtype=torch.bfloat16, hd=64, L_q=16):
    g = torch.Generator().manual_seed(9)
    B_u, B_c, H, L_kv = 3, 7, 2, 40
    Q = torch.randn(B_c, H, L_q, hd, generator=g).to(dtype)
    K = torch.randn(B_u, H, L_kv, hd, generator=g).to(dtype)
    V = torch.randn(B_u, H, L_kv, hd, generator=g).to(dtype)
    mp = torch.randint(0, B_u, (B_c,), generator=g)
    return Q, K, V, mp


def calls(gm, target):
    return [n for n in gm.graph.nodes if n.op == "call_function" and n.target is target]


@pytest.mark.parametrize("gather", ["getitem", "index_select"])
@pytest.mark.parametrize("scale", [None, 0.3])
def test_rewrite_replaces_sdpa_over_gathered_kv(gather, scale):
    Q, K, V, mp = small()
    gm = fx.symbolic_trace(TargetAttention(gather, scale))
    assert rw.rewrite_attention(gm, Q, K, V, mp) == 1
    (node,) = calls(gm, rw.ikbo_target_attention)
    assert not calls(gm, F.scaled_dot_product_attention)
    q, k, v, p, sc = node.args
    assert (q.target, k.target, v.target, p.target) == ("Q", "K", "V", "mp") and sc == scale


def test_rewritten_graph_keeps_the_math_on_cpu():
    # With the library call swapped for a plain attention over the gathered K/V (test only),
    # the rewritten graph reproduces the original module.
    Q, K, V, mp = small()
    m = TargetAttention()
    gm = fx.symbolic_trace(m)
    rw.rewrite_attention(gm, Q, K, V, mp)
    ref = m(Q, K, V, mp).float()

    def plain(Q_, K_, V_, mp_, scale):
        s = (Q_.float() @ K_[mp_].float().transpose(-2, -1)) * (scale or Q_.shape[-1] ** -0.5)
        return torch.softmax(s, dim=-1) @ V_[mp_].float()
    for node in calls(gm, rw.ikbo_target_attention):
        node.target = plain
    gm.recompile()
    assert torch.allclose(gm(Q, K, V, mp), ref, rtol=2e-2, atol=2e-2)


@pytest.mark.parametrize("case", ["causal", "mask", "k_only", "float32", "head_dim_32", "L_q_48", "scale_0"])
def test_rewrite_leaves_other_attention_alone(case):
    kw = {"float32": dict(dtype=torch.float32), "head_dim_32": dict(hd=32), "L_q_48": dict(L_q=48)}.get(case, {})
    Q, K, V, mp = small(**kw)
    variant = case if case in ("causal", "mask", "k_only") else "plain"
    gm = fx.symbolic_trace(TargetAttention(variant=variant, scale=0.0 if case == "scale_0" else None))
    try:
        n = rw.rewrite_attention(gm, Q, K, V, mp)
    except RuntimeError:
        return                                     # shape propagation itself rejects the graph
    assert n == 0 and not calls(gm, rw.ikbo_target_attention)


def test_fa_plan_table_sizes_plans_by_shape_range():
    made = []

    class FakePlan:
        def __init__(self, mu, mc, H, L_q, L_kv, hd):
            self.max_B_u, self.max_B_c, self.closed = mu, mc, False
            made.append(self)

        def close(self):
            self.closed = True

    t = rw.FaPlanTable(make_plan=FakePlan)
    p1 = t.plan_for(15, 1000, 4, 64, 1024, 128)
    assert (p1.max_B_u, p1.max_B_c) == (16, 1024)
    assert t.plan_for(15, 1024, 4, 64, 1024, 128) is p1
    p2 = t.plan_for(59, 4096, 4, 64, 1024, 128)
    assert p1.closed and (p2.max_B_u, p2.max_B_c) == (64, 4096)


@pytest.mark.gpu
def test_rewritten_attention_matches_oracle_on_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import numpy as np

    import oracle
    from broadcast_gemm_amd.inputs import FA_CONFIG_BY_NAME, make_fa_inputs
    from gpu_util import assert_close, to_dev, to_f64
    x = make_fa_inputs(FA_CONFIG_BY_NAME["fa-10to1"])
    Q, K, V, mp = to_dev(x.Q), to_dev(x.K), to_dev(x.V), to_dev(x.map).long()
    gm = fx.symbolic_trace(TargetAttention())
    assert rw.rewrite_attention(gm, Q, K, V, mp) == 1
    O = to_f64(gm(Q, K, V, mp))
    assert rw.fa_plan_table().check_all() == 0
    rng = np.random.default_rng(3)
    rows = [(int(b), int(h), int(q)) for b in rng.integers(0, x.cfg.B_c, 24) for h in (0, 3) for q in (0, 63)]
    assert_close(np.stack([O[r] for r in rows]), oracle.fa_f64(x.Q, x.K, x.V, x.map, rows=rows),
                 "rewritten attention", oracle.fa_weight_bound(x.Q, x.K, x.V, x.map, rows=rows))
