"""The forward without a plan or any device allocation (ikbo_lce_forward_noalloc), called
through the C ABI, against the plan-based entry point (ikbo_lce_forward) on the same
kernels: two calls in a row, the second with a smaller input, each bit-identical to the
plan's output and within the oracle bar (|Y_gpu - Y_ref| <= 1e-3 + 1.6e-2*|Y_ref|).
Sizes past the scratch array, and unsupported widths, are refused before anything runs."""
import ctypes

import pytest

import broadcast_gemm_amd as bga
from broadcast_gemm_amd.inputs import LceConfig, make_inputs
from gpu_util import assert_close, dev_inputs, log, to_f64, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch().cuda.is_available():
        pytest.skip("no GPU")
    bga.lib()


def _noalloc(x, Y):
    U, C, mp, W_u, W_c = x
    B_u, K_u, D = U.shape
    B_c, K_c = C.shape[0], C.shape[1]
    M = W_u.shape[0]
    return bga.forward_noalloc_ptrs(U.data_ptr(), C.data_ptr(), mp.data_ptr(), W_u.data_ptr(), W_c.data_ptr(),
                                    Y.data_ptr(), B_u, B_c, K_u, K_c, M, D,
                                    torch().cuda.current_stream().cuda_stream)


def test_noalloc_matches_plan_two_calls(monkeypatch):
    import oracle
    monkeypatch.delenv("IKBO_STREAM", raising=False)
    t = torch()
    shapes = [("first", 15, 1024, 301, 197, 96, 160, "sorted"),     # the 70:1 workload
              ("second", 5, 37, 40, 24, 48, 160, "random")]         # smaller, after it
    for name, B_u, B_c, K_u, K_c, M, D, mp in shapes:
        log(f"[noalloc] {name} B_u={B_u} B_c={B_c} K_u={K_u} K_c={K_c} M={M} D={D}")
        x = make_inputs(LceConfig("noalloc", B_u, B_c, K_u, K_c, M, D, "bf16", mp, 17))
        d = dev_inputs(x)
        Y_na = t.full((B_c, M, D), float("nan"), dtype=t.bfloat16, device="cuda")
        st = _noalloc(d, Y_na)
        assert st == bga.IKBO_OK, bga.status_str(st) + " " + bga.last_error_message()
        plan = bga.LcePlan(B_u, B_c, K_u, K_c, M, D, dtype="bf16", variant="S3")
        try:
            assert plan.info()["engine"] == "stream"
            Y_pl = plan.forward(*d)
            assert plan.check() == bga.IKBO_OK
        finally:
            plan.close()
        t.cuda.synchronize()
        assert t.equal(Y_na.view(t.int16), Y_pl.view(t.int16)), f"{name}: differs from ikbo_lce_forward"
        assert_close(to_f64(Y_na), oracle.lce_f64(x.U, x.C, x.map, x.W_u, x.W_c), f"noalloc/{name}")


def test_noalloc_refuses_beyond_scratch():
    t = torch()
    B_u, B_c, K_u, K_c, M, D = 200, 4, 32, 32, 96, 160      # P_u: 200*96*160*4 bytes > 8 MiB - 256
    U = t.zeros((B_u, K_u, D), dtype=t.bfloat16, device="cuda")
    C = t.zeros((B_c, K_c, D), dtype=t.bfloat16, device="cuda")
    mp = t.zeros((B_c,), dtype=t.int32, device="cuda")
    W_u = t.zeros((M, K_u), dtype=t.bfloat16, device="cuda")
    W_c = t.zeros((M, K_c), dtype=t.bfloat16, device="cuda")
    Y = t.zeros((B_c, M, D), dtype=t.bfloat16, device="cuda")
    st = _noalloc((U, C, mp, W_u, W_c), Y)
    assert st == bga.IKBO_ERR_UNSUPPORTED
    assert "scratch" in bga.last_error_message()
    assert float(Y.float().abs().sum()) == 0.0           # nothing was enqueued
    U48 = t.zeros((1, K_u, 48), dtype=t.bfloat16, device="cuda")
    C48 = t.zeros((B_c, K_c, 48), dtype=t.bfloat16, device="cuda")
    Y48 = t.zeros((B_c, M, 48), dtype=t.bfloat16, device="cuda")
    assert _noalloc((U48, C48, mp, W_u, W_c), Y48) == bga.IKBO_ERR_UNSUPPORTED
