"""The HIP backward against the CPU oracle, through the C ABI.

Gradients of L = <dY, Y> for the LCE forward (IKBO recsys blog, "Deep Dive: Linear
Compression", stage 1; the pages give no training formulas, so the oracle is the
chain rule of their definition).  Small shapes that span several tiles with ragged
tails are compared element by element; the four bf16 configurations at full size are
compared on sampled rows the oracle computes one by one (dC rows, dU rows, dW
elements).  Bar, per element of each gradient: |g - g_ref| <= 1e-3 + 1.6e-2 |g_ref|
(the forward's bar: bf16 inputs, fp32 accumulation; dU and dC are rounded to bf16
once, dW stays fp32).
"""
import numpy as np
import pytest

import broadcast_gemm_amd as bga
from broadcast_gemm_amd.inputs import CONFIG_BY_NAME, LceConfig, make_inputs, make_upstream_grad
from gpu_util import assert_close, log, to_dev, to_f64, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch().cuda.is_available():
        pytest.skip("no GPU")
    bga.lib()


def gpu_backward(x, dY, plan_B=None):
    cfg = x.cfg
    mu, mc = plan_B or (cfg.B_u, cfg.B_c)
    plan = bga.LcePlan(mu, mc, cfg.K_u, cfg.K_c, cfg.M, cfg.D, dtype="bf16", flags=bga.FLAG_BACKWARD)
    try:
        out = plan.backward(to_dev(dY), to_dev(x.U), to_dev(x.C), to_dev(x.map), to_dev(x.W_u), to_dev(x.W_c))
        st = plan.check()
        assert st == bga.IKBO_OK, bga.status_str(st)
        return tuple(to_f64(t) for t in out)
    finally:
        plan.close()


SMALL = [
    # (B_u, B_c, K_u, K_c, M, D, map): what it covers
    (5, 70, 301, 197, 96, 160, "sorted"),     # the 70:1 dimensions at a small batch; ragged K tails
    (3, 50, 120, 77, 64, 32, "random"),       # D = 32
    (9, 130, 120, 77, 112, 128, "random"),    # D = 128, 7 row blocks, more chunks than candidates per user
    (2, 40, 509, 251, 128, 128, "sorted"),    # the 10000:1 dimensions
    (7, 33, 64, 40, 48, 192, "random"),       # D = 192, M = 48 (one row tile)
    (6, 64, 301, 197, 90, 160, "gaps"),       # users 1 and 4 have no candidate; ragged M
    (4, 300, 64, 40, 80, 64, "sorted"),       # D = 64; runs of 75 span several chunks
]


@pytest.mark.parametrize("shape", SMALL, ids=[f"{s[0]}x{s[1]}-K{s[2]}_{s[3]}-M{s[4]}-D{s[5]}-{s[6]}" for s in SMALL])
def test_backward_small_elementwise(shape):
    import oracle
    B_u, B_c, K_u, K_c, M, D, kind = shape
    log(f"[backward] small shape={shape}")
    cfg = LceConfig("bwd", B_u, B_c, K_u, K_c, M, D, "bf16", "random" if kind == "gaps" else kind, 77)
    x = make_inputs(cfg)
    if kind == "gaps":
        mp = np.random.default_rng(5).choice(np.array([0, 2, 3, 5], np.int32), B_c).astype(np.int32)
        x = x.__class__(cfg, x.U, x.C, x.W_u, x.W_c, mp)
    dY = make_upstream_grad(cfg)
    got = gpu_backward(x, dY)
    ref = oracle.lce_backward_f64(dY, x.U, x.C, x.map, x.W_u, x.W_c)
    for name, g, r in zip(("dU", "dC", "dW_u", "dW_c"), got, ref):
        assert g.shape == r.shape, name
        assert_close(g, r, f"{shape} {name}")
    if kind == "gaps":
        assert np.all(got[0][[1, 4]] == 0.0), "users without candidates must get dU = 0 exactly"


def _samples(cfg, mp, rng):
    B_u, B_c, K_u, K_c, M = cfg.B_u, cfg.B_c, cfg.K_u, cfg.K_c, cfg.M
    bs = np.unique(np.concatenate([[0, 1, B_c // 2, B_c - 2, B_c - 1], rng.integers(0, B_c, 11)]))
    dc = [(int(b), int(k)) for b in bs for k in (0, K_c - 1, int(rng.integers(0, K_c)))]
    counts = np.bincount(mp, minlength=B_u)
    users = np.unique([0, B_u - 1, int(np.argmax(counts)), int(rng.integers(0, B_u))])
    du = [(int(u), int(k)) for u in users for k in (0, K_u - 1)]
    ms = np.unique([0, M - 1, int(rng.integers(0, M))])
    kks = np.unique([0, K_u - 1, K_u, K_u + K_c - 1, int(rng.integers(0, K_u)), int(rng.integers(K_u, K_u + K_c))])
    dw = [(int(m), int(k)) for m in ms for k in kks]
    return dc, du, dw


@pytest.mark.parametrize("name", ["default-70to1", "small-10to1", "large-unsorted", "extreme-10000to1"])
def test_backward_full_size_sampled(name):
    import oracle
    cfg = CONFIG_BY_NAME[name]
    log(f"[backward] full size {name}")
    x = make_inputs(cfg)
    dY = make_upstream_grad(cfg)
    dU, dC, dW_u, dW_c = gpu_backward(x, dY)
    dc, du, dw = _samples(cfg, x.map, np.random.default_rng(31))
    oc, ou, ow = oracle.lce_backward_rows_f64(dY, x.U, x.C, x.map, x.W_u, x.W_c, dc, du, dw)
    assert_close(np.stack([dC[b, k] for b, k in dc]), oc, f"{name} dC rows")
    assert_close(np.stack([dU[u, k] for u, k in du]), ou, f"{name} dU rows")
    K_u = cfg.K_u
    gw = np.array([dW_u[m, k] if k < K_u else dW_c[m, k - K_u] for m, k in dw])
    assert_close(gw, ow, f"{name} dW elements")
    assert np.all(np.isfinite(dU)) and np.all(np.isfinite(dC)) and np.all(np.isfinite(dW_u)) and np.all(np.isfinite(dW_c))


def test_backward_repeats_bit_exactly_and_plan_reuse():
    """Fixed summation orders that depend on the inputs only: the same call twice on one
    plan, and on a plan sized for larger batches, gives the same bits."""
    cfg = CONFIG_BY_NAME["default-70to1"]
    log("[backward] determinism and plan reuse")
    x = make_inputs(cfg)
    dY = make_upstream_grad(cfg)
    plan = bga.LcePlan(cfg.B_u, cfg.B_c, cfg.K_u, cfg.K_c, cfg.M, cfg.D, dtype="bf16", flags=bga.FLAG_BACKWARD)
    try:
        args = tuple(to_dev(a) for a in (dY, x.U, x.C, x.map, x.W_u, x.W_c))
        a = tuple(to_f64(t) for t in plan.backward(*args))
        a2 = tuple(to_f64(t) for t in plan.backward(*args))
        assert plan.check() == bga.IKBO_OK
    finally:
        plan.close()
    b = gpu_backward(x, dY, plan_B=(cfg.B_u + 9, cfg.B_c + 500))
    for name, p, q, r in zip(("dU", "dC", "dW_u", "dW_c"), a, a2, b):
        assert np.array_equal(p, q), f"{name}: second call differs"
        assert np.array_equal(p, r), f"{name}: larger plan differs"


def test_backward_outputs_ordered_on_the_callers_stream():
    """The call's kernels run on streams of the plan as well as the caller's; whatever the
    caller enqueues on its stream after the call must see the finished outputs.  Three calls
    on a user stream write the same output tensors, each with a different dY, and each is
    copied on that stream right after its call, with no synchronisation in between; every
    copy must equal the same call made alone."""
    t = torch()
    cfg = CONFIG_BY_NAME["default-70to1"].with_batch(8, 300)
    log("[backward] outputs ordered on the caller's stream")
    x = make_inputs(cfg)
    dYs = [make_upstream_grad(cfg, seed=s) for s in (501, 502, 503)]
    plan = bga.LcePlan(cfg.B_u, cfg.B_c, cfg.K_u, cfg.K_c, cfg.M, cfg.D, dtype="bf16", flags=bga.FLAG_BACKWARD)
    try:
        ins = tuple(to_dev(a) for a in (x.U, x.C, x.map, x.W_u, x.W_c))
        dev_dY = [to_dev(d) for d in dYs]
        alone = [tuple(to_f64(g) for g in plan.backward(d, *ins)) for d in dev_dY]
        st = t.cuda.Stream()
        st.wait_stream(t.cuda.current_stream())
        with t.cuda.stream(st):
            out = plan.backward(dev_dY[0], *ins)
            copies = [tuple(g.clone() for g in out)]
            for d in dev_dY[1:]:
                plan.backward(d, *ins, out=out)
                copies.append(tuple(g.clone() for g in out))
        st.synchronize()
        assert plan.check() == bga.IKBO_OK
    finally:
        plan.close()
    for i, (c, a) in enumerate(zip(copies, alone)):
        for name, g, r in zip(("dU", "dC", "dW_u", "dW_c"), c, a):
            assert np.array_equal(to_f64(g), r), f"call {i}: {name} copied before the call finished"
    assert not np.array_equal(alone[0][1], alone[1][1])


def test_backward_edge_cases():
    """B_c = 0 zeroes dU and dW (outputs are overwritten, not accumulated); a map entry out
    of range is reported; a plan made without the backward flag is refused."""
    t = torch()
    cfg = LceConfig("bwd-edge", 3, 40, 64, 40, 48, 64, "bf16", "random", 5)
    log("[backward] edge cases")
    x = make_inputs(cfg)
    dY = make_upstream_grad(cfg)
    plan = bga.LcePlan(3, 40, 64, 40, 48, 64, dtype="bf16", flags=bga.FLAG_BACKWARD)
    try:
        U, C, mp, W_u, W_c, g = (to_dev(a) for a in (x.U, x.C, x.map, x.W_u, x.W_c, dY))
        outs = (t.full((3, 64, 64), float("nan"), dtype=t.bfloat16, device="cuda"),
                t.full((0, 40, 64), float("nan"), dtype=t.bfloat16, device="cuda"),
                t.full((48, 64), float("nan"), dtype=t.float32, device="cuda"),
                t.full((48, 40), float("nan"), dtype=t.float32, device="cuda"))
        plan.backward(g[:0].contiguous(), U, C[:0].contiguous(), mp[:0].contiguous(), W_u, W_c, out=outs)
        assert plan.check() == bga.IKBO_OK
        for o in (outs[0], outs[2], outs[3]):
            assert bool((o == 0).all()), "B_c = 0 must give zero gradients"
        bad = mp.clone()
        bad[7] = 3
        plan.backward(g, U, C, bad, W_u, W_c)
        assert plan.check() == bga.IKBO_ERR_MAP_RANGE
        plan.backward(g, U, C, mp, W_u, W_c)
        assert plan.check() == bga.IKBO_OK
    finally:
        plan.close()
    fwd_only = bga.LcePlan(3, 40, 64, 40, 48, 64, dtype="bf16")
    try:
        with pytest.raises(bga.IkboError):
            fwd_only.backward(g, U, C, mp, W_u, W_c)
    finally:
        fwd_only.close()


ONE_PASS = [
    # (B_u, B_c, K_u, K_c, M, D, map): the one-pass dC + dW_c launch at its edges
    (3, 300, 40, 13, 96, 160, "random"),      # one K_c block: three waves own none; 300 > 256 chunks
    (2, 257, 33, 256, 128, 128, "sorted"),    # sixteen K_c blocks (four per wave); chunks of 2 and 1
    (4, 9, 50, 49, 33, 160, "random"),        # M = 33: two 32-row steps, the second mostly zero rows
    (1, 1, 20, 70, 1, 128, "sorted"),         # M = 1, one candidate
    (5, 520, 64, 100, 112, 160, "sorted"),    # M = 112 on the 128-row kernel, ragged K_c
]


@pytest.mark.parametrize("shape", ONE_PASS, ids=[f"{s[0]}x{s[1]}-K{s[2]}_{s[3]}-M{s[4]}-D{s[5]}" for s in ONE_PASS])
def test_backward_one_pass_elementwise(shape):
    """dC and dW_c from the one-pass launch (dY read once for both) against the oracle,
    element by element, at shapes on its edges."""
    import oracle
    B_u, B_c, K_u, K_c, M, D, kind = shape
    log(f"[backward] one pass shape={shape}")
    cfg = LceConfig("bwd1", B_u, B_c, K_u, K_c, M, D, "bf16", kind, 91)
    x = make_inputs(cfg)
    dY = make_upstream_grad(cfg)
    plan = bga.LcePlan(B_u, B_c, K_u, K_c, M, D, dtype="bf16", flags=bga.FLAG_BACKWARD)
    try:
        assert plan.info()["bwd_cand_chunks"] > 0
        out = plan.backward(to_dev(dY), to_dev(x.U), to_dev(x.C), to_dev(x.map), to_dev(x.W_u), to_dev(x.W_c))
        st = plan.check()
        assert st == bga.IKBO_OK, bga.status_str(st)
        got = tuple(to_f64(t) for t in out)
    finally:
        plan.close()
    ref = oracle.lce_backward_f64(dY, x.U, x.C, x.map, x.W_u, x.W_c)
    for name, g, r in zip(("dU", "dC", "dW_u", "dW_c"), got, ref):
        assert g.shape == r.shape, name
        assert_close(g, r, f"{shape} {name}")


def test_backward_separate_launches_still_match(monkeypatch):
    """With the one-pass launch switched off (IKBO_BWD_FUSED=0, read when the plan is made),
    dC and dW_c come from the row-tile engine and the weight-gradient kernel, as for shapes the
    one-pass launch does not take; both routes meet the bar at the 70:1 dimensions."""
    import oracle
    monkeypatch.setenv("IKBO_BWD_FUSED", "0")
    cfg = LceConfig("bwd0", 5, 70, 301, 197, 96, 160, "bf16", "sorted", 78)
    log("[backward] separate launches")
    x = make_inputs(cfg)
    dY = make_upstream_grad(cfg)
    plan = bga.LcePlan(cfg.B_u, cfg.B_c, cfg.K_u, cfg.K_c, cfg.M, cfg.D, dtype="bf16", flags=bga.FLAG_BACKWARD)
    try:
        assert plan.info()["bwd_cand_chunks"] == 0
        out = plan.backward(to_dev(dY), to_dev(x.U), to_dev(x.C), to_dev(x.map), to_dev(x.W_u), to_dev(x.W_c))
        assert plan.check() == bga.IKBO_OK
        got = tuple(to_f64(t) for t in out)
    finally:
        plan.close()
    ref = oracle.lce_backward_f64(dY, x.U, x.C, x.map, x.W_u, x.W_c)
    for name, g, r in zip(("dU", "dC", "dW_u", "dW_c"), got, ref):
        assert_close(g, r, f"separate {name}")


def test_backward_one_pass_forced_long_chunks(monkeypatch):
    """The one-pass launch forced (IKBO_BWD_FUSED=2) on the 4096-candidate random-map workload,
    where the plan would not take it: chunks of 16 candidates per CU, sampled rows and weight
    elements against the oracle."""
    import oracle
    monkeypatch.setenv("IKBO_BWD_FUSED", "2")
    cfg = CONFIG_BY_NAME["large-unsorted"]
    log("[backward] one pass forced, large-unsorted")
    x = make_inputs(cfg)
    dY = make_upstream_grad(cfg)
    dU, dC, dW_u, dW_c = gpu_backward(x, dY)
    dc, du, dw = _samples(cfg, x.map, np.random.default_rng(47))
    oc, ou, ow = oracle.lce_backward_rows_f64(dY, x.U, x.C, x.map, x.W_u, x.W_c, dc, du, dw)
    assert_close(np.stack([dC[b, k] for b, k in dc]), oc, "forced one pass dC rows")
    assert_close(np.stack([dU[u, k] for u, k in du]), ou, "forced one pass dU rows")
    K_u = cfg.K_u
    gw = np.array([dW_u[m, k] if k < K_u else dW_c[m, k - K_u] for m, k in dw])
    assert_close(gw, ow, "forced one pass dW elements")
