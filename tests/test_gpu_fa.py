"""IKBO target attention on the GPU against the CPU oracle, through the C ABI.

O[b,h] = softmax(scale Q[b,h] K[map[b],h]^T) V[map[b],h] (IKBO recsys blog, "Deep Dive:
Flash Attention").  Small shapes with ragged key counts, partial candidate groups, users
without candidates and both head sizes are compared element by element; the attention
configurations at full size on sampled query rows.  Bar, per element:
|O - O_ref| <= 1e-3 + 1.6e-2 |O_ref| + 2^-8 sum_k w_k |V_k|: the LCE bar (bf16 inputs and
output, fp32 accumulation) plus twice what bf16 rounding of the softmax weights w (at most
2^-9 of each weight) can move an output; the pages fix no precision for attention, and the
last term matters only when few keys carry the weight.
"""
import numpy as np
import pytest

import broadcast_gemm_amd as bga
from broadcast_gemm_amd.inputs import FA_CONFIG_BY_NAME, FaConfig, make_fa_inputs
from gpu_util import assert_close, log, to_dev, to_f64, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch().cuda.is_available():
        pytest.skip("no GPU")
    bga.lib()


def gpu_fa(x, mp=None, plan_B=None):
    c = x.cfg
    mp = x.map if mp is None else mp
    mu, mc = plan_B or (c.B_u, c.B_c)
    plan = bga.FaPlan(mu, mc, c.H, c.L_q, c.L_kv, c.hd)
    try:
        O = plan.forward(to_dev(x.Q), to_dev(x.K), to_dev(x.V), to_dev(mp))
        st = plan.check()
        assert st == bga.IKBO_OK, bga.status_str(st)
        return to_f64(O)
    finally:
        plan.close()


SMALL = [
    # (B_u, B_c, H, L_q, L_kv, hd, map): what it covers
    (2, 6, 2, 16, 40, 64, "sorted"),        # one partial key block; groups of 3 candidates
    (3, 10, 2, 32, 130, 128, "random"),     # three key blocks, the last with 2 keys
    (5, 23, 3, 64, 256, 128, "random"),     # the attention configuration's L_q and hd; partial groups
    (4, 9, 1, 64, 64, 64, "sorted"),        # exactly one key block, hd = 64
    (6, 17, 2, 16, 1, 128, "random"),       # a single key: O = V[map[b], h, 0]
    (6, 30, 2, 64, 200, 128, "gaps"),       # users 1, 3 and 4 have no candidate
]


@pytest.mark.parametrize("shape", SMALL, ids=[f"{s[0]}x{s[1]}-H{s[2]}-Lq{s[3]}-Lkv{s[4]}-hd{s[5]}-{s[6]}" for s in SMALL])
def test_fa_small_elementwise(shape):
    import oracle
    B_u, B_c, H, L_q, L_kv, hd, kind = shape
    log(f"[fa] small shape={shape}")
    cfg = FaConfig("fa-test", B_u, B_c, H, L_q, L_kv, hd, "bf16", "sorted" if kind == "sorted" else "random", 61)
    x = make_fa_inputs(cfg)
    if kind == "gaps":
        x.map = np.random.default_rng(3).choice(np.array([0, 2, 5], np.int32), B_c).astype(np.int32)
    O = gpu_fa(x)
    ref = oracle.fa_f64(x.Q, x.K, x.V, x.map)
    assert_close(O, ref, f"fa {shape}", oracle.fa_weight_bound(x.Q, x.K, x.V, x.map))


def _rows(cfg, mp, rng):
    B_c = cfg.B_c
    bs = np.unique(np.concatenate([[0, 1, B_c // 2, B_c - 1], rng.integers(0, B_c, 12),
                                   [int(np.argmax(mp == mp.max()))]]))
    return [(int(b), int(h), int(q)) for b in bs for h in {0, cfg.H - 1, int(rng.integers(0, cfg.H))}
            for q in (0, cfg.L_q - 1, int(rng.integers(0, cfg.L_q)))]


@pytest.mark.parametrize("name", ["fa-70to1", "fa-10to1", "fa-large-unsorted"])
def test_fa_full_size_sampled(name):
    import oracle
    cfg = FA_CONFIG_BY_NAME[name]
    log(f"[fa] full size {name}")
    x = make_fa_inputs(cfg)
    O = gpu_fa(x)
    rows = _rows(cfg, x.map, np.random.default_rng(41))
    ref = oracle.fa_f64(x.Q, x.K, x.V, x.map, rows=rows)
    assert_close(np.stack([O[r] for r in rows]), ref, f"{name} sampled rows",
                 oracle.fa_weight_bound(x.Q, x.K, x.V, x.map, rows=rows))
    assert np.all(np.isfinite(O))


def test_fa_shared_user_and_determinism():
    """Candidates of one user with equal queries get equal outputs, bit for bit; a second
    call (also on a plan sized for more) repeats every bit."""
    cfg = FaConfig("fa-dup", 3, 40, 2, 64, 300, 128, "bf16", "random", 62)
    log("[fa] shared user / determinism")
    x = make_fa_inputs(cfg)
    src = 5
    same = np.nonzero(x.map == x.map[src])[0]
    x.Q[same] = x.Q[src]
    a = gpu_fa(x)
    for b in same:
        assert np.array_equal(a[b], a[src]), f"candidate {b} differs from {src} with the same user and queries"
    b2 = gpu_fa(x, plan_B=(9, 100))
    assert np.array_equal(a, b2)


def test_fa_map_out_of_range_reported():
    cfg = FaConfig("fa-bad", 3, 12, 1, 16, 64, 64, "bf16", "random", 63)
    log("[fa] map out of range")
    x = make_fa_inputs(cfg)
    bad = x.map.copy()
    bad[4] = 3
    plan = bga.FaPlan(3, 12, 1, 16, 64, 64)
    try:
        plan.forward(to_dev(x.Q), to_dev(x.K), to_dev(x.V), to_dev(bad))
        assert plan.check() == bga.IKBO_ERR_MAP_RANGE
        plan.forward(to_dev(x.Q), to_dev(x.K), to_dev(x.V), to_dev(x.map))
        assert plan.check() == bga.IKBO_OK
    finally:
        plan.close()


def test_fa_rescale_after_first_block():
    """A key in the last key block whose score exceeds the running maximum by far more than
    the kernel's 8 (log2) of headroom: O must be rescaled after block 0 (L_kv = 1024, 16
    key blocks).  Each candidate gets such a key for one of its queries, aligned with it."""
    import oracle
    from broadcast_gemm_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits
    cfg = FaConfig("fa-rescale", 2, 6, 2, 64, 1024, 128, "bf16", "sorted", 64)
    log("[fa] rescale after block 0")
    x = make_fa_inputs(cfg)
    Q = bf16_bits_to_f32(x.Q)
    K = bf16_bits_to_f32(x.K)
    for b in range(cfg.B_c):
        u = int(x.map[b])
        for h in range(cfg.H):
            q = (7 * b + h) % cfg.L_q
            # score = |Q|^2 * 1.5 / sqrt(128): about 17 against a running maximum near 4
            K[u, h, cfg.L_kv - 1 - 3 * b - h] = 1.5 * Q[b, h, q]
    x.K = f32_to_bf16_bits(K)
    O = gpu_fa(x)
    ref = oracle.fa_f64(x.Q, x.K, x.V, x.map)
    assert_close(O, ref, "fa rescale", oracle.fa_weight_bound(x.Q, x.K, x.V, x.map))
    assert np.all(np.isfinite(O))
