"""HIP path against the CPU oracle on shapes chosen for the persistent schedule's
edge cases: partial last rounds split into row-block sub-units (with a ragged last
row chunk), waves left with a single candidate unit, more user units than waves
(the one-launch stage falls back to two launches), every column layout of the
row-tile engine (D = 32, 64, 128, 160, 192) with both activation load widths (S1
loads 4 bytes per lane, the other stages 16), and projections too large to sit in
LDS together (the one-launch stage then holds them one after the other).

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
    (2, 300, 509, 251, 128, 128, "sorted"),      # W_u + W_c exceed LDS: S4 copies W_c over W_u after users
    (7, 500, 509, 251, 128, 128, "random"),      # same, with a partial user block and a random map
]


def _cases():
    for sh in SHAPES:
        sid = f"{sh[0]}x{sh[1]}-K{sh[2]}_{sh[3]}-M{sh[4]}-D{sh[5]}-{sh[6]}"
        for v in ["S0", "S1", "S2", "S3", "S4"]:
            # S0's packed [W_u | W_c] (M x (K_u + K_c)) must fit LDS for the rows engine.
            if v == "S0" and sh[4] * (sh[2] + sh[3]) * 2 > 150 * 1024:
                continue
            # the gather-add stages run on both engines (the streaming one and the row-tile one)
            for eng in (["stream", "rows"] if v in ("S3", "S4") else ["rows"]):
                yield pytest.param(sh, v, eng, id=f"{sid}-{v}-{eng}")


@pytest.mark.parametrize("shape,variant,engine", list(_cases()))
def test_schedule_shapes(shape, variant, engine, monkeypatch):
    import oracle
    B_u, B_c, K_u, K_c, M, D, mp = shape
    log(f"[schedule] shape={shape} variant={variant} engine={engine}")
    cfg = LceConfig("schedule", B_u, B_c, K_u, K_c, M, D, "bf16", mp, 91)
    x = make_inputs(cfg)
    if variant in ("S3", "S4"):
        monkeypatch.setenv("IKBO_STREAM", "1" if engine == "stream" else "0")
    plan = bga.LcePlan(B_u, B_c, K_u, K_c, M, D, dtype="bf16", variant=variant)
    try:
        assert plan.info()["engine"] == engine
        Y = plan.forward(*dev_inputs(x))
        st = plan.check()
        assert st == bga.IKBO_OK, bga.status_str(st)
        Y = to_f64(Y)
    finally:
        plan.close()
    assert_close(Y, oracle.lce_f64(x.U, x.C, x.map, x.W_u, x.W_c), f"{shape}/{variant}")


TAIL_SHAPES = [
    # (B_u, B_c, K_u, K_c, M, D, map): units left for a partial last round, at most a quarter of the
    # waves, so that each is cut along K over the four waves of one block
    (9, 1100, 120, 130, 64, 32, "sorted"),       # D = 32, 112 units left (S3's candidate launch: 76)
    (9, 1100, 120, 130, 64, 64, "random"),       # D = 64
    (9, 600, 120, 130, 128, 128, "sorted"),      # D = 128, four row blocks per unit (128 KB of partials)
    (9, 1100, 120, 130, 48, 192, "random"),      # D = 192, one row block per unit
    (15, 1000, 301, 197, 90, 160, "sorted"),     # 42 units left, ragged last row chunk
    (7, 1150, 509, 251, 128, 128, "random"),     # projections taking turns in LDS (S4); S3 leaves 252 units
]


@pytest.mark.parametrize("variant", ["S3", "S4"])
@pytest.mark.parametrize("shape", TAIL_SHAPES,
                         ids=[f"{s[0]}x{s[1]}-K{s[2]}_{s[3]}-M{s[4]}-D{s[5]}-{s[6]}" for s in TAIL_SHAPES])
def test_tail_pieces(shape, variant, monkeypatch):
    """The partial last round's units cut along K into four pieces on the waves of one block,
    their partial sums added in LDS (the gather-add stages on the rows engine), against the
    oracle; a second forward on the same plan as well."""
    import oracle
    B_u, B_c, K_u, K_c, M, D, mp = shape
    log(f"[tail] shape={shape} variant={variant}")
    cfg = LceConfig("tail", B_u, B_c, K_u, K_c, M, D, "bf16", mp, 97)
    x = make_inputs(cfg)
    monkeypatch.setenv("IKBO_STREAM", "0")
    plan = bga.LcePlan(B_u, B_c, K_u, K_c, M, D, dtype="bf16", variant=variant)
    try:
        info = plan.info()
        assert info["engine"] == "rows" and info["rows_tail_split"] == 1
        for _ in range(2):
            Y = plan.forward(*dev_inputs(x))
            st = plan.check()
            assert st == bga.IKBO_OK, bga.status_str(st)
        Y = to_f64(Y)
    finally:
        plan.close()
    assert_close(Y, oracle.lce_f64(x.U, x.C, x.map, x.W_u, x.W_c), f"{shape}/{variant} tail pieces")
