"""HIP path against the CPU oracle, through the C ABI, on the seeded configurations.

Bar: per element |Y_gpu - Y_ref| <= 1e-3 + 1.6e-2*|Y_ref| (bf16 inputs, fp32
accumulation, one bf16 rounding), with map/gather indexing bit-exact (tag and
integer tests).  The largest configuration is checked on sampled candidates.
"""
import numpy as np
import pytest

import broadcast_gemm_amd as bga
from broadcast_gemm_amd.inputs import (CONFIG_BY_NAME, LceConfig, make_inputs, make_integer_inputs,
                                       make_tag_inputs)
from gpu_util import (CONFIG_NAMES, SAMPLED_ROWS, VARIANTS, assert_close, cached_inputs, cached_oracle,
                      dev_inputs, log, to_dev, to_f64, torch)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    bga.lib()


def run(x, variant, plan=None, check=True):
    cfg = x.cfg
    U, C, mp, W_u, W_c = dev_inputs(x)
    own = plan is None
    if own:
        plan = bga.LcePlan(cfg.B_u, cfg.B_c, cfg.K_u, cfg.K_c, cfg.M, cfg.D, dtype=cfg.dtype, variant=variant)
    try:
        Y = plan.forward(U, C, mp, W_u, W_c)
        if check:
            st = plan.check()
            assert st == bga.IKBO_OK, bga.status_str(st)
        return Y
    finally:
        if own:
            plan.close()


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("name", CONFIG_NAMES)
def test_config_parity(name, variant):
    log(f"[parity] config={name} variant={variant}")
    x = cached_inputs(name)
    Y = to_f64(run(x, variant))
    ref, rows = cached_oracle(name)
    if rows is not None:
        Y = Y[rows]
    assert_close(Y, ref, f"{name}/{variant}")


RAGGED = [
    # (B_u, B_c, K_u, K_c, M, D, dtype): ragged column tails, K tails, M not a multiple of 16
    (3, 37, 45, 33, 40, 24, "bf16"),
    (1, 1, 1, 1, 1, 8, "bf16"),
    (5, 11, 64, 32, 16, 8, "bf16"),
    (7, 50, 301, 197, 96, 160, "bf16"),
    (2, 19, 70, 9, 72, 200, "bf16"),
    (4, 13, 13, 11, 8, 16, "f32"),
    (3, 29, 37, 5, 20, 12, "f32"),
    (1, 1, 1, 1, 1, 4, "f32"),
]


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("shape", RAGGED, ids=[f"{s[0]}x{s[1]}-K{s[2]}_{s[3]}-M{s[4]}-D{s[5]}-{s[6]}" for s in RAGGED])
def test_ragged_shapes(shape, variant):
    import oracle
    B_u, B_c, K_u, K_c, M, D, dt = shape
    log(f"[ragged] shape={shape} variant={variant}")
    cfg = LceConfig("ragged", B_u, B_c, K_u, K_c, M, D, dt, "random", 77)
    x = make_inputs(cfg)
    Y = to_f64(run(x, variant))
    assert_close(Y, oracle.lce_f64(x.U, x.C, x.map, x.W_u, x.W_c), f"{shape}/{variant}")


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("name", ["default-70to1", "large-unsorted", "extreme-10000to1", "tiny"])
def test_integer_inputs_bit_exact(name, variant):
    """Inputs and weights in {-1, 0, 1}: every partial sum is an exact small integer,
    so any summation order gives the oracle's value bit for bit."""
    import oracle
    log(f"[exact] config={name} variant={variant}")
    cfg = CONFIG_BY_NAME[name]
    if name == "extreme-10000to1":
        cfg = cfg.with_batch(2, 2000)
    x = make_integer_inputs(cfg)
    Y = to_f64(run(x, variant))
    rows = list(range(0, cfg.B_c, max(1, cfg.B_c // 64)))
    ref = oracle.lce_f64(x.U, x.C, x.map, x.W_u, x.W_c, rows=rows)
    assert np.array_equal(Y[rows], ref)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("name", ["default-70to1", "small-10to1", "large-unsorted", "extreme-10000to1"])
def test_gather_tag(name, variant):
    """Y[b, m, d] must equal map[b] + 1 exactly: the gather reads the right user."""
    log(f"[tag] config={name} variant={variant}")
    cfg = CONFIG_BY_NAME[name]
    x = make_tag_inputs(cfg, mp=cached_inputs(name).map if name == "large-unsorted" else None)
    Y = to_f64(run(x, variant))
    assert np.array_equal(Y, np.broadcast_to((x.map + 1.0)[:, None, None], Y.shape))


@pytest.mark.parametrize("variant", VARIANTS)
def test_power_of_two_scaling_is_exact(variant):
    log(f"[scale] variant={variant}")
    x = make_inputs(CONFIG_BY_NAME["small-10to1"])
    Y1 = run(x, variant)
    t = torch()
    U, C, mp, W_u, W_c = dev_inputs(x)
    cfg = x.cfg
    with bga.LcePlan(cfg.B_u, cfg.B_c, cfg.K_u, cfg.K_c, cfg.M, cfg.D, dtype=cfg.dtype, variant=variant) as p:
        Y2 = p.forward((U.float() * 2).to(t.bfloat16), (C.float() * 2).to(t.bfloat16), mp, W_u, W_c)
        assert p.check() == bga.IKBO_OK
    assert t.equal((Y1.float() * 2).to(t.bfloat16).view(t.int16), Y2.view(t.int16))


@pytest.mark.parametrize("variant", VARIANTS)
def test_variants_identical_on_repeat_and_resize(variant):
    """One plan, back-to-back forwards with different batch sizes inside its range."""
    import oracle
    log(f"[repeat] variant={variant}")
    base = CONFIG_BY_NAME["default-70to1"]
    plan = bga.LcePlan(20, 1024, base.K_u, base.K_c, base.M, base.D, dtype="bf16", variant=variant)
    try:
        outs = []
        for (B_u, B_c) in [(15, 1024), (3, 100), (20, 1000), (15, 1024), (1, 1)]:
            x = make_inputs(base.with_batch(B_u, B_c))
            Y = run(x, variant, plan=plan)
            rows = list(range(0, B_c, max(1, B_c // 40)))
            assert_close(to_f64(Y)[rows], oracle.lce_f64(x.U, x.C, x.map, x.W_u, x.W_c, rows=rows),
                         f"{variant} B_u={B_u} B_c={B_c}")
            outs.append(Y)
        assert torch().equal(outs[0].view(torch().int16), outs[3].view(torch().int16))
    finally:
        plan.close()


@pytest.mark.parametrize("engine", ["rows", "stream"])
def test_s4_alternating_inputs_every_element(engine, monkeypatch):
    """One one-launch (S4) plan at the 70:1 workload fed two input sets in turn, A, B, A, B:
    every element of every output against the oracle, and the repeats bit-identical.  A
    candidate that read a user partial left by the previous forward (a stale flag or a stale
    cache line) would carry the other set's user term and fail."""
    import dataclasses
    import oracle
    monkeypatch.setenv("IKBO_STREAM", "1" if engine == "stream" else "0")
    base = CONFIG_BY_NAME["default-70to1"]
    xa = cached_inputs("default-70to1")
    xb = make_inputs(dataclasses.replace(base, seed=base.seed + 101))
    ref_a, _ = cached_oracle("default-70to1")
    ref_b = oracle.lce_f64(xb.U, xb.C, xb.map, xb.W_u, xb.W_c)
    plan = bga.LcePlan(base.B_u, base.B_c, base.K_u, base.K_c, base.M, base.D, dtype="bf16", variant="S4")
    try:
        assert plan.info()["engine"] == engine
        outs = []
        for k, (x, ref) in enumerate([(xa, ref_a), (xb, ref_b), (xa, ref_a), (xb, ref_b)]):
            log(f"[abab] engine={engine} forward {k} set {'AB'[k % 2]}")
            Y = run(x, "S4", plan=plan)
            assert_close(to_f64(Y), ref, f"S4/{engine} forward {k}")
            outs.append(Y)
        t = torch()
        assert t.equal(outs[0].view(t.int16), outs[2].view(t.int16))
        assert t.equal(outs[1].view(t.int16), outs[3].view(t.int16))
    finally:
        plan.close()


@pytest.mark.parametrize("variant", VARIANTS)
def test_zero_candidates_is_a_noop(variant):
    cfg = CONFIG_BY_NAME["tiny"]
    t = torch()
    with bga.LcePlan(2, 8, cfg.K_u, cfg.K_c, cfg.M, cfg.D, dtype="f32", variant=variant) as p:
        x = make_inputs(cfg)
        U, C, mp, W_u, W_c = dev_inputs(x)
        Y = t.full((0, cfg.M, cfg.D), 7.0, device="cuda")
        st = p.forward_ptrs(U.data_ptr(), C.data_ptr(), mp.data_ptr(), W_u.data_ptr(), W_c.data_ptr(),
                            Y.data_ptr(), 2, 0)
        assert st == bga.IKBO_OK
        assert p.check() == bga.IKBO_OK


@pytest.mark.parametrize("variant", VARIANTS)
def test_isolation_and_guard_zones(variant):
    """NaN in candidate b+1 or in rows after user u never reaches Y[b]; bytes just
    outside Y stay untouched; users with no candidates are fine."""
    log(f"[isolation] variant={variant}")
    t = torch()
    cfg = LceConfig("iso", 4, 9, 33, 21, 40, 24, "bf16", "explicit", 5, explicit_map=(0, 0, 1, 1, 1, 3, 3, 3, 3))
    x = make_inputs(cfg)
    U, C, mp, W_u, W_c = dev_inputs(x)
    Y_ref = to_f64(run(x, variant))
    C2 = C.clone()
    C2[4] = float("nan")                 # candidate 4 only
    U2 = U.clone()
    U2[2] = float("inf")                 # user 2 has no candidates
    guard = 64
    buf = t.full((cfg.B_c * cfg.M * cfg.D + 2 * guard,), 3.0, dtype=t.bfloat16, device="cuda")
    Y = buf[guard:guard + cfg.B_c * cfg.M * cfg.D].view(cfg.B_c, cfg.M, cfg.D)
    with bga.LcePlan(cfg.B_u, cfg.B_c, cfg.K_u, cfg.K_c, cfg.M, cfg.D, dtype="bf16", variant=variant) as p:
        p.forward(U2, C2, mp, W_u, W_c, out=Y)
        assert p.check() == bga.IKBO_OK
    Yn = to_f64(Y)
    assert np.isnan(Yn[4]).all()
    others = [b for b in range(cfg.B_c) if b != 4]
    assert np.array_equal(Yn[others], Y_ref[others])
    assert (buf[:guard] == 3.0).all() and (buf[-guard:] == 3.0).all()


@pytest.mark.parametrize("variant", VARIANTS)
def test_map_out_of_range_is_reported(variant):
    t = torch()
    cfg = CONFIG_BY_NAME["tiny"]
    x = make_inputs(cfg)
    U, C, mp, W_u, W_c = dev_inputs(x)
    bad = mp.clone()
    bad[5] = 7
    with bga.LcePlan(2, 8, cfg.K_u, cfg.K_c, cfg.M, cfg.D, dtype="f32", variant=variant) as p:
        p.set_spin_limit(2000)
        p.forward(U, C, bad, W_u, W_c)
        assert p.check() == bga.IKBO_ERR_MAP_RANGE
        p.forward(U, C, mp, W_u, W_c)     # error word was cleared
        assert p.check() == bga.IKBO_OK


def test_host_validation_on_device():
    cfg = CONFIG_BY_NAME["tiny"]
    x = make_inputs(cfg)
    U, C, mp, W_u, W_c = dev_inputs(x)
    t = torch()
    Y = t.empty((8, 8, 16), device="cuda")
    with bga.LcePlan(2, 8, cfg.K_u, cfg.K_c, cfg.M, cfg.D, dtype="f32", variant="S4") as p:
        L = bga.lib()
        args = [U.data_ptr(), C.data_ptr(), mp.data_ptr(), W_u.data_ptr(), W_c.data_ptr(), Y.data_ptr()]
        assert L.ikbo_lce_forward(p.handle, *args, 3, 8, 13, 11, 8, 16, None) == bga.IKBO_ERR_INVALID_ARG
        assert L.ikbo_lce_forward(p.handle, *args, 2, 9, 13, 11, 8, 16, None) == bga.IKBO_ERR_INVALID_ARG
        assert L.ikbo_lce_forward(p.handle, *args, 2, 8, 12, 11, 8, 16, None) == bga.IKBO_ERR_INVALID_ARG
        assert L.ikbo_lce_forward(p.handle, *args, 0, 8, 13, 11, 8, 16, None) == bga.IKBO_ERR_INVALID_ARG
        mis = list(args)
        mis[1] += 4
        assert L.ikbo_lce_forward(p.handle, *mis, 2, 8, 13, 11, 8, 16, None) == bga.IKBO_ERR_ALIGNMENT
        info = p.info()
        assert info["variant"] == "S4" and info["K_u_pad"] % 32 == 0
        assert p.check() == bga.IKBO_OK


def test_s4_delayed_user_tiles_still_correct():
    import oracle
    log("[s4-delay]")
    cfg = CONFIG_BY_NAME["small-10to1"]
    x = cached_inputs("small-10to1")
    U, C, mp, W_u, W_c = dev_inputs(x)
    with bga.LcePlan(cfg.B_u, cfg.B_c, cfg.K_u, cfg.K_c, cfg.M, cfg.D, variant="S4",
                     flags=bga.FLAG_DEBUG_DELAY_USER) as p:
        Y = p.forward(U, C, mp, W_u, W_c)
        assert p.check() == bga.IKBO_OK
    assert_close(to_f64(Y), oracle.lce_f64(x.U, x.C, x.map, x.W_u, x.W_c), "S4 delayed users")


@pytest.mark.parametrize("engine", ["rows", "stream"])
@pytest.mark.parametrize("name", ["default-70to1", "small-10to1"])
@pytest.mark.parametrize("delay", [False, True])
def test_s4_poisoned_user_partials(name, engine, delay, monkeypatch):
    """Each forward first fills the user partials with NaN (and, with delay, the user units
    also sleep before computing): a candidate that read P_u before this forward's user
    product had published it would carry a NaN into Y.  Two forwards in a row, every element
    against the oracle."""
    log(f"[s4-poison] config={name} engine={engine} delay={delay}")
    monkeypatch.setenv("IKBO_STREAM", "1" if engine == "stream" else "0")
    cfg = CONFIG_BY_NAME[name]
    x = cached_inputs(name)
    ref, rows = cached_oracle(name)
    flags = bga.FLAG_DEBUG_POISON_USER | (bga.FLAG_DEBUG_DELAY_USER if delay else 0)
    with bga.LcePlan(cfg.B_u, cfg.B_c, cfg.K_u, cfg.K_c, cfg.M, cfg.D, variant="S4", flags=flags) as p:
        assert p.info()["engine"] == engine
        for k in range(2):
            Y = run(x, "S4", plan=p)
            assert p.check() == bga.IKBO_OK
            Yf = to_f64(Y)
            assert not np.isnan(Yf).any(), f"forward {k}: NaN from a poisoned user partial"
            assert_close(Yf if rows is None else Yf[rows], ref, f"S4/{engine} poisoned forward {k}")


def test_s4_poison_reaches_the_user_partials():
    """The poisoning itself: with the user units skipped, every candidate times out and then
    adds the poisoned partials, so every output is NaN and the plan reports the timeout."""
    log("[s4-poison-skip]")
    cfg = CONFIG_BY_NAME["small-10to1"]
    x = cached_inputs("small-10to1")
    with bga.LcePlan(cfg.B_u, cfg.B_c, cfg.K_u, cfg.K_c, cfg.M, cfg.D, variant="S4",
                     flags=bga.FLAG_DEBUG_POISON_USER | bga.FLAG_DEBUG_SKIP_USER) as p:
        p.set_spin_limit(200)
        Y = run(x, "S4", plan=p, check=False)
        assert p.check() == bga.IKBO_ERR_TIMEOUT
        assert np.isnan(to_f64(Y)).all()


def test_s4_skipped_user_tiles_time_out():
    """No user tile publishes: every candidate wave gives up after the poll limit,
    the kernel exits, and the plan reports IKBO_ERR_TIMEOUT."""
    log("[s4-skip]")
    cfg = CONFIG_BY_NAME["small-10to1"]
    x = cached_inputs("small-10to1")
    U, C, mp, W_u, W_c = dev_inputs(x)
    with bga.LcePlan(cfg.B_u, cfg.B_c, cfg.K_u, cfg.K_c, cfg.M, cfg.D, variant="S4",
                     flags=bga.FLAG_DEBUG_SKIP_USER) as p:
        p.set_spin_limit(200)
        p.forward(U, C, mp, W_u, W_c)
        assert p.check() == bga.IKBO_ERR_TIMEOUT
        p.forward(U, C, mp, W_u, W_c)
        assert p.check() == bga.IKBO_ERR_TIMEOUT


def test_s4_plan_on_sampled_full_size_rows_again():
    """Second forward on the same S4 plan at the largest configuration (epoch and
    ticket reset path at scale), checked on sampled candidates."""
    name = "extreme-10000to1"
    log(f"[s4-repeat] {name}")
    cfg = CONFIG_BY_NAME[name]
    x = cached_inputs(name)
    U, C, mp, W_u, W_c = dev_inputs(x)
    ref, rows = cached_oracle(name)
    with bga.LcePlan(cfg.B_u, cfg.B_c, cfg.K_u, cfg.K_c, cfg.M, cfg.D, variant="S4") as p:
        for _ in range(3):
            Y = p.forward(U, C, mp, W_u, W_c)
            assert p.check() == bga.IKBO_OK
            assert_close(to_f64(Y)[rows], ref, "S4 repeat")
