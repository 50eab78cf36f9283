"""HIP path against the CPU oracle on shapes chosen for the persistent schedule's
edge cases: partial last rounds split into row-block sub-units (with a ragged last
row chunk), waves left with a single candidate unit, more user units than waves
(the one-launch stage falls back to two launches), and every column layout of the
row-tile engine (D = 32, 64, 128, 160, 192).

Bar: per element |Y_gpu - Y_ref| <= 1e-3 + 1.6e-2*|Y_ref|, as in test_gpu_parity.
"""
import pytest

import broadcast_gemm_amd as bga
from broadcast_gemm_amd.inputs import LceConfig, make_inputs
from gpu_util import VARIANTS, assert_close, dev_inputs, log, to_f64, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch().cuda.is_available():
        pytest.skip("no GPU")
    bga.lib()


SHAPES = [
    # (B_u, B_c, K_u, K_c, M, D, map): comment
    (15, 1000, 301, 197, 90, 160, "sorted"),     # partial last round -> sub-units; ragged last row chunk
    (15, 600, 301, 197, 96, 160, "random"),      # fewer units than waves: some waves hold one candidate
    (200, 400, 64, 40, 96, 160, "random"),       # more user units than waves: S4 takes two launches
    (9, 700, 120, 77, 64, 32, "sorted"),         # D = 32 (two 2-column slots per lane group)
    (9, 700, 120, 77, 80, 64, "random"),         # D = 64
    (9, 700, 120, 77, 112, 128, "sorted"),       # D = 128
    (9, 700, 120, 77, 48, 192, "random"),        # D = 192
]


@pytest.mark.parametrize("variant", ["S0", "S2", "S3", "S4"])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{s[0]}x{s[1]}-K{s[2]}_{s[3]}-M{s[4]}-D{s[5]}-{s[6]}" for s in SHAPES])
def test_schedule_shapes(shape, variant):
    import oracle
    B_u, B_c, K_u, K_c, M, D, mp = shape
    log(f"[schedule] shape={shape} variant={variant}")
    cfg = LceConfig("schedule", B_u, B_c, K_u, K_c, M, D, "bf16", mp, 91)
    x = make_inputs(cfg)
    plan = bga.LcePlan(B_u, B_c, K_u, K_c, M, D, dtype="bf16", variant=variant)
    try:
        assert plan.info()["engine"] == "rows"
        Y = plan.forward(*dev_inputs(x))
        st = plan.check()
        assert st == bga.IKBO_OK, bga.status_str(st)
        Y = to_f64(Y)
    finally:
        plan.close()
    assert_close(Y, oracle.lce_f64(x.U, x.C, x.map, x.W_u, x.W_c), f"{shape}/{variant}")
