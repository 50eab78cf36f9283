"""Self + target attention in one launch (IKBO recsys blog, "Self + Target Attention
Fusion"), through the C ABI.  The users' own queries attend over the same K/V as their
candidates' queries; the oracle's attention with the users as their own candidates
(identity map) is the reference for the self part.  Checks: the target part of a fused
launch is bit-identical to a target-only launch, the self part of a fused launch is
bit-identical to a self-only launch (B_c = 0) and within the attention bar of the oracle
(|O - O_ref| <= 1e-3 + 1.6e-2 |O_ref| + 2^-8 sum_k w_k |V_k|)."""
import numpy as np
import pytest

import broadcast_gemm_amd as bga
from broadcast_gemm_amd.inputs import FA_CONFIG_BY_NAME, FaConfig, f32_to_bf16_bits, make_fa_inputs
from gpu_util import assert_close, log, to_dev, to_f64, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch().cuda.is_available():
        pytest.skip("no GPU")
    bga.lib()


def q_self_for(cfg, L_self, seed):
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(rng.standard_normal((cfg.B_u, cfg.H, L_self, cfg.hd), dtype=np.float32))


CASES = [
    # (B_u, B_c, H, L_q, L_kv, hd, L_self, map kind)
    (3, 10, 2, 32, 130, 128, 64, "random"),
    (5, 7, 1, 64, 256, 128, 192, "gaps"),      # users 1 and 3 have no candidate but their own queries
    (2, 6, 2, 16, 40, 64, 48, "sorted"),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}x{c[1]}-Lq{c[3]}-Lkv{c[4]}-hd{c[5]}-self{c[6]}-{c[7]}" for c in CASES])
def test_fused_matches_separate_and_oracle(case):
    import oracle
    B_u, B_c, H, L_q, L_kv, hd, L_self, kind = case
    log(f"[fa-fused] case={case}")
    cfg = FaConfig("fa-fused", B_u, B_c, H, L_q, L_kv, hd, "bf16", "sorted" if kind == "sorted" else "random", 71)
    x = make_fa_inputs(cfg)
    if kind == "gaps":
        x.map = np.random.default_rng(4).choice(np.array([0, 2, 4], np.int32), B_c).astype(np.int32)
    Qs = q_self_for(cfg, L_self, 72)
    plan = bga.FaPlan(B_u, B_c, H, L_q, L_kv, hd)
    try:
        Q, K, V, mp, Qsd = (to_dev(a) for a in (x.Q, x.K, x.V, x.map, Qs))
        O_f, Os_f = plan.forward_fused(Q, K, V, mp, Qsd)
        O_t = plan.forward(Q, K, V, mp)
        O_s = torch().empty_like(Qsd)
        st = plan.forward_fused_ptrs(0, K.data_ptr(), V.data_ptr(), 0, 0, Qsd.data_ptr(), O_s.data_ptr(), B_u, 0, L_self)
        assert st == bga.IKBO_OK, bga.status_str(st)
        assert plan.check() == bga.IKBO_OK
        O_f, Os_f, O_t, O_s = (to_f64(t) for t in (O_f, Os_f, O_t, O_s))
    finally:
        plan.close()
    assert np.array_equal(O_f, O_t), "target part of the fused launch differs from a target-only launch"
    assert np.array_equal(Os_f, O_s), "self part of the fused launch differs from a self-only launch"
    ident = np.arange(B_u, dtype=np.int32)
    ref = oracle.fa_f64(Qs, x.K, x.V, ident)
    assert_close(Os_f, ref, f"{case} self part", oracle.fa_weight_bound(Qs, x.K, x.V, ident))
    assert_close(O_f, oracle.fa_f64(x.Q, x.K, x.V, x.map), f"{case} target part",
                 oracle.fa_weight_bound(x.Q, x.K, x.V, x.map))


def test_fused_full_size_sampled():
    import oracle
    cfg = FA_CONFIG_BY_NAME["fa-70to1"]
    L_self = 1024
    log("[fa-fused] fa-70to1 with the users' 1024-token sequences as self queries")
    x = make_fa_inputs(cfg)
    Qs = q_self_for(cfg, L_self, 73)
    plan = bga.FaPlan(cfg.B_u, cfg.B_c, cfg.H, cfg.L_q, cfg.L_kv, cfg.hd)
    try:
        O_f, Os_f = plan.forward_fused(*(to_dev(a) for a in (x.Q, x.K, x.V, x.map, Qs)))
        assert plan.check() == bga.IKBO_OK
        O_f, Os_f = to_f64(O_f), to_f64(Os_f)
    finally:
        plan.close()
    rng = np.random.default_rng(5)
    rows = [(int(u), int(h), int(q)) for u in (0, cfg.B_u - 1, 7) for h in (0, cfg.H - 1) for q in (0, 511, 1023, int(rng.integers(0, 1024)))]
    ident = np.arange(cfg.B_u, dtype=np.int32)
    assert_close(np.stack([Os_f[r] for r in rows]), oracle.fa_f64(Qs, x.K, x.V, ident, rows=rows), "self rows",
                 oracle.fa_weight_bound(Qs, x.K, x.V, ident, rows=rows))
    trows = [(int(b), 1, 5) for b in (0, 500, 1023)]
    assert_close(np.stack([O_f[r] for r in trows]), oracle.fa_f64(x.Q, x.K, x.V, x.map, rows=trows), "target rows",
                 oracle.fa_weight_bound(x.Q, x.K, x.V, x.map, rows=trows))
