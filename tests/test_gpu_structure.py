"""Structural properties of the HIP path, through the C ABI, at the 70:1 workload's shapes.

Each candidate's output depends only on its own C[b], its user's U row and the two
projections (the definition in the IKBO recsys blog, "Deep Dive: Linear Compression",
stage 1), so:

* permuting the candidates (C and map together) permutes the rows of Y;
* relabelling the users (U permuted, map renamed to match) leaves Y unchanged;
* an IEEE special value reaches exactly the outputs that read it: a NaN in one element
  of U[u] turns that column of every candidate of u into NaN, an Inf in a row of C[b]
  turns that column of Y[b] into +-Inf, and nothing else changes.  Specials sit in the
  last K row of one candidate and the first K row of the next, so a K tail that read
  past its own candidate (0 x Inf = NaN) would show up in the neighbour.

Where every unit accumulates in the same order (S0..S3) the permuted and relabelled
results are bit-identical; S4 adds the user product at the end for a wave's first two
units and starts its other units from it, so its results are held to the parity bar
(|Y - Y_ref| <= 1e-3 + 1.6e-2 |Y_ref|) instead.  Specials are compared by position and
sign against the fp64 oracle, finite elements at the parity bar.
"""
import numpy as np
import pytest

import broadcast_gemm_amd as bga
from gpu_util import VARIANTS, assert_close, cached_inputs, cached_oracle, dev_inputs, log, to_dev, to_f64, torch

pytestmark = pytest.mark.gpu

NAME = "default-70to1"
BF16_NAN, BF16_POS_INF, BF16_NEG_INF = 0x7FC0, 0x7F80, 0xFF80


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch().cuda.is_available():
        pytest.skip("no GPU")
    bga.lib()


def forward(x_arrays, cfg, variant):
    U, C, mp, W_u, W_c = (to_dev(a) for a in x_arrays)
    plan = bga.LcePlan(cfg.B_u, cfg.B_c, cfg.K_u, cfg.K_c, cfg.M, cfg.D, dtype=cfg.dtype, variant=variant)
    try:
        Y = plan.forward(U, C, mp, W_u, W_c)
        st = plan.check()
        assert st == bga.IKBO_OK, bga.status_str(st)
        return to_f64(Y)
    finally:
        plan.close()


def compare(Y_a, Y_b, variant, what):
    if variant == "S4":
        assert_close(Y_a, Y_b, what)
    else:
        diff = int(np.count_nonzero(Y_a != Y_b))
        assert diff == 0, f"{what}: {diff} elements differ"


@pytest.mark.parametrize("variant", VARIANTS)
def test_permuted_candidates_permute_outputs(variant):
    x = cached_inputs(NAME)
    cfg = x.cfg
    log(f"[structure] permuted candidates variant={variant}")
    Y = forward((x.U, x.C, x.map, x.W_u, x.W_c), cfg, variant)
    perm = np.random.default_rng(11).permutation(cfg.B_c)
    Yp = forward((x.U, np.ascontiguousarray(x.C[perm]), np.ascontiguousarray(x.map[perm]), x.W_u, x.W_c), cfg, variant)
    compare(Yp, Y[perm], variant, f"{variant} permuted candidates")


@pytest.mark.parametrize("variant", VARIANTS)
def test_relabelled_users_leave_outputs_unchanged(variant):
    x = cached_inputs(NAME)
    cfg = x.cfg
    log(f"[structure] relabelled users variant={variant}")
    Y = forward((x.U, x.C, x.map, x.W_u, x.W_c), cfg, variant)
    sigma = np.random.default_rng(12).permutation(cfg.B_u)        # user u becomes sigma[u]
    U2 = np.ascontiguousarray(x.U[np.argsort(sigma)])             # U2[sigma[u]] = U[u]
    map2 = sigma[x.map].astype(np.int32)
    Y2 = forward((U2, x.C, map2, x.W_u, x.W_c), cfg, variant)
    compare(Y2, Y, variant, f"{variant} relabelled users")


@pytest.mark.parametrize("variant", VARIANTS)
def test_ieee_specials_reach_exactly_their_outputs(variant):
    import oracle
    x = cached_inputs(NAME)
    cfg = x.cfg
    log(f"[structure] NaN/Inf propagation variant={variant}")
    U = x.U.copy()
    C = x.C.copy()
    u0 = int(x.map[700])
    U[u0, cfg.K_u - 1, 17] = BF16_NAN            # last K row of a user, a group-1 column
    C[500, cfg.K_c - 1, 150] = BF16_POS_INF      # last K row of candidate 500, a group-2 column
    C[501, 0, 3] = BF16_NEG_INF                  # first K row of the next candidate
    C[64, cfg.K_c - 1, 128] = BF16_NAN           # last row of a candidate inside a sorted run
    Y = forward((U, C, x.map, x.W_u, x.W_c), cfg, variant)
    Y_ref = oracle.lce_f64(U, C, x.map, x.W_u, x.W_c)
    nan_ref, nan_gpu = np.isnan(Y_ref), np.isnan(Y)
    assert nan_ref.any() and np.array_equal(nan_gpu, nan_ref), (
        f"{variant}: NaN at {int(nan_gpu.sum())} outputs, expected {int(nan_ref.sum())}; first extra "
        f"{np.argwhere(nan_gpu & ~nan_ref)[:3].tolist()}, first missing {np.argwhere(nan_ref & ~nan_gpu)[:3].tolist()}")
    inf_ref, inf_gpu = np.isinf(Y_ref), np.isinf(Y)
    assert inf_ref.any() and np.array_equal(inf_gpu, inf_ref), (
        f"{variant}: Inf at {int(inf_gpu.sum())} outputs, expected {int(inf_ref.sum())}")
    assert np.array_equal(np.sign(Y[inf_ref]), np.sign(Y_ref[inf_ref])), f"{variant}: Inf signs differ"
    fin = np.isfinite(Y_ref)
    assert_close(np.where(fin, Y, 0.0), np.where(fin, Y_ref, 0.0), f"{variant} finite outputs beside specials")
