"""Inference-time rewrite of a materialised-broadcast LCE into the IKBO forward.

The pages describe two ways to adopt the kernels: write them into the model, or let
an inference-time pass swap the standard operators for the IKBO ones without touching
the model (IKBO recsys blog, the section on how the IKBO co-design is built and its
FAQ; aibriefing article, the paragraph on the three layers of the stack).  The same
passages say the compiler needs each operator's dynamic shape range to pick the kernel.

This module is that pass for torch.fx graphs, for the pages' two kernels.  For the LCE it finds

    X = cat([U[map], C], dim=1)        (U[map] as indexing or index_select along dim 0;
    Y = W @ X                           the blocks in either order; @ as matmul, or bmm
                                        of W expanded over the batch)

with W a 2-D [M, K_u + K_c] matrix, and replaces Y by ``ikbo_lce(U, C, map, W_u, W_c)``,
where W_u and W_c are W's column blocks (split where U's K ends; copies are taken once
at rewrite time when W is a module attribute).  ``ikbo_lce`` runs the HIP forward with
a plan from ``PlanTable``, which sizes plans by shape range: candidate batches are rounded
up to the pages' 256..4096 range (then to multiples of 4096), user batches to powers of
two, and a plan is replaced by a larger one when a call outgrows it.

For target attention (IKBO recsys blog, "Deep Dive: Flash Attention") it finds

    O = scaled_dot_product_attention(Q, K[map], V[map])   (K and V gathered by the same index,
                                                           no mask, no dropout, not causal)

with bf16 Q [B_c, H, L_q, hd] and K, V [B_u, H, L_kv, hd] in the shapes the library serves
(hd 64 or 128, L_q 16, 32 or 64), and replaces O by ``ikbo_target_attention(Q, K, V, map,
scale)``, which never replicates K and V; plans come from ``FaPlanTable``, sized by the same
batch ranges.

Only the graph is rewritten; every forward runs in the HIP library (no CPU fallback).
"""
from __future__ import annotations

import operator
from typing import Dict, Optional, Tuple

from . import FaPlan, LcePlan

B_C_BUCKETS = (256, 512, 1024, 2048, 4096)   # candidate batch range (the pages' practical advice)


def bucket_b_c(b: int) -> int:
    for x in B_C_BUCKETS:
        if b <= x:
            return x
    return -(-b // B_C_BUCKETS[-1]) * B_C_BUCKETS[-1]


def bucket_b_u(b: int) -> int:
    n = 16
    while n < b:
        n *= 2
    return n


class PlanTable:
    """Plans keyed by (K_u, K_c, M, D, dtype), each sized to a shape range."""

    def __init__(self, variant: str = "auto", make_plan=LcePlan):
        self.variant = variant
        self._make = make_plan
        self._plans: Dict[Tuple, object] = {}

    def plan_for(self, B_u: int, B_c: int, K_u: int, K_c: int, M: int, D: int, dtype: str):
        key = (K_u, K_c, M, D, dtype)
        plan = self._plans.get(key)
        if plan is None or plan.max_B_u < B_u or plan.max_B_c < B_c:
            mu, mc = bucket_b_u(B_u), bucket_b_c(B_c)
            if plan is not None:
                mu, mc = max(mu, plan.max_B_u), max(mc, plan.max_B_c)
                plan.close()
            plan = self._make(mu, mc, K_u, K_c, M, D, dtype=dtype, variant=self.variant)
            self._plans[key] = plan
        return plan

    def check_all(self) -> int:
        """Device status of every plan (synchronises); the first non-zero status, else 0."""
        for plan in self._plans.values():
            st = plan.check()
            if st != 0:
                return st
        return 0

    def close(self) -> None:
        for plan in self._plans.values():
            plan.close()
        self._plans.clear()


_TABLE: Optional[PlanTable] = None


def plan_table() -> PlanTable:
    global _TABLE
    if _TABLE is None:
        _TABLE = PlanTable()
    return _TABLE


def ikbo_lce(U, C, mp, W_u, W_c):
    """Y = W_u . U[map] + W_c . C through the plan table (the rewritten graph's call)."""
    import torch
    dtype = "bf16" if U.dtype == torch.bfloat16 else "f32"
    B_u, K_u, D = U.shape
    B_c, K_c, _ = C.shape
    plan = plan_table().plan_for(B_u, B_c, K_u, K_c, W_u.shape[0], D, dtype)
    return plan.forward(U.contiguous(), C.contiguous(), mp, W_u.contiguous(), W_c.contiguous())


class FaPlanTable:
    """Attention plans keyed by (H, L_q, L_kv, head_dim), each sized to a batch range."""

    def __init__(self, make_plan=FaPlan):
        self._make = make_plan
        self._plans: Dict[Tuple, object] = {}

    def plan_for(self, B_u: int, B_c: int, H: int, L_q: int, L_kv: int, hd: int):
        key = (H, L_q, L_kv, hd)
        plan = self._plans.get(key)
        if plan is None or plan.max_B_u < B_u or plan.max_B_c < B_c:
            mu, mc = bucket_b_u(B_u), bucket_b_c(B_c)
            if plan is not None:
                mu, mc = max(mu, plan.max_B_u), max(mc, plan.max_B_c)
                plan.close()
            plan = self._make(mu, mc, H, L_q, L_kv, hd)
            self._plans[key] = plan
        return plan

    def check_all(self) -> int:
        for plan in self._plans.values():
            st = plan.check()
            if st != 0:
                return st
        return 0

    def close(self) -> None:
        for plan in self._plans.values():
            plan.close()
        self._plans.clear()


_FA_TABLE: Optional[FaPlanTable] = None


def fa_plan_table() -> FaPlanTable:
    global _FA_TABLE
    if _FA_TABLE is None:
        _FA_TABLE = FaPlanTable()
    return _FA_TABLE


def ikbo_target_attention(Q, K, V, mp, scale=None):
    """softmax(scale Q K[map]^T) V[map] per head through the plan table (the rewritten graph's call)."""
    B_c, H, L_q, hd = Q.shape
    B_u, _, L_kv, _ = K.shape
    plan = fa_plan_table().plan_for(B_u, B_c, H, L_q, L_kv, hd)
    return plan.forward(Q.contiguous(), K.contiguous(), V.contiguous(), mp, scale=0.0 if scale is None else scale)


# ---- pattern matching on an fx graph --------------------------------------------------

def _is_call(node, targets) -> bool:
    return node.op == "call_function" and node.target in targets


def _gather_of(node):
    """(U, map) if node is U[map] or U.index_select(0, map), else None."""
    import torch
    if _is_call(node, (operator.getitem,)):
        src, idx = node.args
        if hasattr(idx, "op"):                 # a tensor index, not a slice or an int
            return src, idx
    if _is_call(node, (torch.index_select,)) or (node.op == "call_method" and node.target == "index_select"):
        src, dim, idx = (list(node.args) + [node.kwargs.get("dim"), node.kwargs.get("index")])[:3]
        if dim == 0:
            return src, idx
    return None


def _cat_parts(node):
    """The two parts of a cat along dim 1 (of 3-D tensors), else None."""
    import torch
    if not _is_call(node, (torch.cat, torch.concat)):
        return None
    parts = node.args[0]
    dim = node.args[1] if len(node.args) > 1 else node.kwargs.get("dim", 0)
    if not isinstance(parts, (list, tuple)) or len(parts) != 2 or dim not in (1, -2):
        return None
    return parts


def _matmul_operands(node):
    """(W, X) of W @ X or bmm(W.expand(...), X), else None."""
    import torch
    if _is_call(node, (torch.matmul, operator.matmul)):
        return node.args[0], node.args[1]
    if node.op == "call_method" and node.target == "matmul":
        return node.args[0], node.args[1]
    if _is_call(node, (torch.bmm,)):
        w = node.args[0]
        if w.op == "call_method" and w.target == "expand":
            return w.args[0], node.args[1]
    return None


def _shape(node):
    tm = node.meta.get("tensor_meta")
    return tuple(tm.shape) if tm is not None else None


def rewrite_lce(gm, *example_inputs) -> int:
    """Replace every materialised-broadcast LCE in gm (a torch.fx.GraphModule) by ikbo_lce.

    example_inputs (any device, dtype of the model) give the shapes the split of W needs.
    Returns the number of rewrites; gm is recompiled in place."""
    import torch
    from torch.fx.passes.shape_prop import ShapeProp

    ShapeProp(gm).propagate(*example_inputs)
    count = 0
    for node in list(gm.graph.nodes):
        ops = _matmul_operands(node)
        if ops is None:
            continue
        w_node, x_node = ops
        parts = _cat_parts(x_node) if hasattr(x_node, "op") else None
        if parts is None:
            continue
        g0, g1 = _gather_of(parts[0]), _gather_of(parts[1])
        if (g0 is None) == (g1 is None):
            continue                                   # exactly one block must be U[map]
        user_first = g0 is not None
        (U, mp), C = (g0, parts[1]) if user_first else (g1, parts[0])
        su, sc, sw = _shape(U), _shape(C), _shape(w_node)
        if su is None or sc is None or sw is None or len(su) != 3 or len(sc) != 3 or len(sw) != 2:
            continue
        K_u, K_c = su[1], sc[1]
        if sw[1] != K_u + K_c or su[2] != sc[2]:
            continue
        lo = K_u if user_first else K_c                # columns of W's first block
        with gm.graph.inserting_before(node):
            if w_node.op == "get_attr":
                W = operator.attrgetter(w_node.target)(gm).detach()
                first, second = W[:, :lo].contiguous(), W[:, lo:].contiguous()
                names = []
                for part, tag in ((first, "a"), (second, "b")):
                    name = f"_ikbo_w{count}{tag}"
                    gm.register_buffer(name, part)
                    names.append(gm.graph.get_attr(name))
                n_first, n_second = names
            else:
                n_first = gm.graph.call_method("contiguous", (gm.graph.call_function(
                    operator.getitem, (w_node, (slice(None), slice(None, lo)))),))
                n_second = gm.graph.call_method("contiguous", (gm.graph.call_function(
                    operator.getitem, (w_node, (slice(None), slice(lo, None)))),))
            W_u, W_c = (n_first, n_second) if user_first else (n_second, n_first)
            new = gm.graph.call_function(ikbo_lce, (U, C, mp, W_u, W_c))
        node.replace_all_uses_with(new)
        gm.graph.erase_node(node)
        count += 1
    if count:
        gm.graph.eliminate_dead_code()
        gm.graph.lint()
        gm.recompile()
    return count


def _sdpa_args(node):
    """(Q, K, V, scale) of an unmasked, non-causal, dropout-free SDPA call, else None."""
    import torch.nn.functional as F
    if not _is_call(node, (F.scaled_dot_product_attention,)):
        return None
    names = ["query", "key", "value", "attn_mask", "dropout_p", "is_causal", "scale"]
    got = dict(zip(names, node.args))
    got.update(node.kwargs)
    if got.get("attn_mask") is not None or got.get("dropout_p", 0.0) not in (0, 0.0) or got.get("is_causal", False):
        return None
    if any(k not in names for k in node.kwargs):   # enable_gqa and the like: leave alone
        return None
    scale = got.get("scale")
    if scale is not None and not (isinstance(scale, (int, float)) and 0 < scale < float("inf")):
        return None                                    # the library reads 0 as 1/sqrt(head_dim)
    return got["query"], got["key"], got["value"], scale


def rewrite_attention(gm, *example_inputs) -> int:
    """Replace every target attention over a gathered (broadcast) K/V in gm by
    ikbo_target_attention.  Returns the number of rewrites; gm is recompiled in place."""
    import torch
    from torch.fx.passes.shape_prop import ShapeProp

    ShapeProp(gm).propagate(*example_inputs)
    count = 0
    for node in list(gm.graph.nodes):
        got = _sdpa_args(node)
        if got is None:
            continue
        q, k, v, scale = got
        gk, gv = (_gather_of(x) if hasattr(x, "op") else None for x in (k, v))
        if gk is None or gv is None or gk[1] is not gv[1]:
            continue                                   # K and V gathered by one index
        (K, mp), (V, _) = gk, gv
        tq, tk, tv = (x.meta.get("tensor_meta") for x in (q, K, V))
        if tq is None or tk is None or tv is None:
            continue
        sq, sk = tuple(tq.shape), tuple(tk.shape)
        if (len(sq) != 4 or len(sk) != 4 or tuple(tv.shape) != sk or sq[1] != sk[1] or sq[3] != sk[3]
                or any(t.dtype != torch.bfloat16 for t in (tq, tk, tv))
                or sq[3] not in (64, 128) or sq[2] not in (16, 32, 64)):
            continue
        with gm.graph.inserting_before(node):
            new = gm.graph.call_function(ikbo_target_attention, (q, K, V, mp, scale))
        node.replace_all_uses_with(new)
        gm.graph.erase_node(node)
        count += 1
    if count:
        gm.graph.eliminate_dead_code()
        gm.graph.lint()
        gm.recompile()
    return count

