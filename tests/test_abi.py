"""libikbo's C ABI on the CPU: the library loads, exports every symbol that
include/ikbo.h declares, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

import broadcast_gemm_amd as bga

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ikbo.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ikbo_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(bga.LIB_PATH):
        from broadcast_gemm_amd import build
        build.build()
    return bga.lib()


def test_header_declares_the_binding_surface():
    assert declared_functions() == sorted(bga.EXPORTED)


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), f"libikbo.so does not export {name}"
        assert isinstance(getattr(L, name), ctypes._CFuncPtr)


def test_status_strings(L):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert bga.status_str(code) not in ("", "unknown status")
    assert bga.status_str(12345) == "unknown status"


def test_plan_rejects_bad_arguments_before_hip(L):
    h = ctypes.c_void_p()
    bad = [
        (-1, 8, 13, 11, 8, 16, 1, 0, 0),     # max_B_u < 1
        (2, -1, 13, 11, 8, 16, 1, 0, 0),     # max_B_c < 0
        (2, 8, 0, 11, 8, 16, 1, 0, 0),       # K_u < 1
        (2, 8, 13, 0, 8, 16, 1, 0, 0),       # K_c < 1
        (2, 8, 13, 11, 0, 16, 1, 0, 0),      # M < 1
        (2, 8, 13, 11, 8, 0, 1, 0, 0),       # D < 1
        (2, 8, 13, 11, 8, 16, 7, 0, 0),      # dtype
        (2, 8, 13, 11, 8, 16, 1, 9, 0),      # variant
        (2, 8, 13, 11, 8, 16, 1, 0, 1),      # unknown flag bit
    ]
    for args in bad:
        assert L.ikbo_lce_plan(ctypes.byref(h), *args) == bga.IKBO_ERR_INVALID_ARG, args
        assert h.value is None
    assert L.ikbo_lce_plan(None, 2, 8, 13, 11, 8, 16, 1, 0, 0) == bga.IKBO_ERR_INVALID_ARG


def test_plan_rejects_unaligned_rows_before_hip(L):
    h = ctypes.c_void_p()
    # bf16 rows of D=12 elements are 24 bytes: not whole 16-byte chunks.
    assert L.ikbo_lce_plan(ctypes.byref(h), 2, 8, 13, 11, 8, 12, 0, 0, 0) == bga.IKBO_ERR_UNSUPPORTED
    # fp32 rows of D=6 elements are 24 bytes.
    assert L.ikbo_lce_plan(ctypes.byref(h), 2, 8, 13, 11, 8, 6, 1, 0, 0) == bga.IKBO_ERR_UNSUPPORTED


def test_null_plan_calls(L):
    assert L.ikbo_lce_forward(None, None, None, None, None, None, None, 1, 1, 1, 1, 1, 8, None) == \
        bga.IKBO_ERR_INVALID_ARG
    assert L.ikbo_lce_check(None, None) == bga.IKBO_ERR_INVALID_ARG
    assert L.ikbo_lce_plan_info(None, None, 0) == bga.IKBO_ERR_INVALID_ARG
    assert L.ikbo_lce_plan_set_spin_limit(None, 5) == bga.IKBO_ERR_INVALID_ARG
    assert L.ikbo_lce_plan_destroy(None) == bga.IKBO_OK


def test_product_package_does_not_reach_the_oracle():
    """The HIP path's sources never import, load or name the CPU oracle."""
    pkg = os.path.join(ROOT, "broadcast_gemm_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "ikbo_oracle" not in text and "libikbo_oracle" not in text, f


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(bga, "_lib", None)
    monkeypatch.setattr(bga, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(ImportError):
        bga.lib()


def test_backward_rejects_bad_arguments_before_hip(L):
    h = ctypes.c_void_p()
    # The backward's workspace exists for bf16 row-tile layouts only.
    assert L.ikbo_lce_plan(ctypes.byref(h), 2, 8, 13, 11, 8, 16, 1, 0, bga.FLAG_BACKWARD) == bga.IKBO_ERR_UNSUPPORTED
    assert L.ikbo_lce_plan(ctypes.byref(h), 2, 8, 13, 11, 8, 48, 0, 0, bga.FLAG_BACKWARD) == bga.IKBO_ERR_UNSUPPORTED
    assert h.value is None
    # No plan: rejected before any HIP call.
    assert L.ikbo_lce_backward(None, *([None] * 10), 1, 1, 13, 11, 8, 16, None) == bga.IKBO_ERR_INVALID_ARG


def test_fa_rejects_bad_arguments_before_hip(L):
    h = ctypes.c_void_p()
    bad_args = [(0, 8, 4, 64, 100, 128, 0, 0), (2, 8, 4, 64, 100, 128, 0, 1), (2, 8, 0, 64, 100, 128, 0, 0)]
    for args in bad_args:
        assert L.ikbo_fa_plan(ctypes.byref(h), *args) == bga.IKBO_ERR_INVALID_ARG, args
    unsupported = [(2, 8, 4, 64, 100, 96, 0, 0), (2, 8, 4, 48, 100, 128, 0, 0), (2, 8, 4, 64, 100, 128, 1, 0)]
    for args in unsupported:
        assert L.ikbo_fa_plan(ctypes.byref(h), *args) == bga.IKBO_ERR_UNSUPPORTED, args
    assert h.value is None
    assert L.ikbo_fa_forward(None, None, None, None, None, None, 1, 1, 4, 64, 100, 128, 0.0, None) == \
        bga.IKBO_ERR_INVALID_ARG


def test_noalloc_rejects_bad_arguments_before_hip(L):
    f = L.ikbo_lce_forward_noalloc
    p = 1 << 20   # stand-in addresses: every check below returns before any HIP call
    assert f(None, p, p, p, p, p, 2, 8, 32, 32, 16, 32, None) == bga.IKBO_ERR_INVALID_ARG
    assert f(p, p, p, p, p, p, 0, 8, 32, 32, 16, 32, None) == bga.IKBO_ERR_INVALID_ARG
    assert f(p, p, p, p, p, p, 2, 0, 32, 32, 16, 32, None) == bga.IKBO_OK            # no candidates: no-op
    assert f(p + 8, p, p, p, p, p, 2, 8, 32, 32, 16, 32, None) == bga.IKBO_ERR_ALIGNMENT
    assert f(p, p, p + 2, p, p, p, 2, 8, 32, 32, 16, 32, None) == bga.IKBO_ERR_ALIGNMENT
    assert f(p, p, p, p, p, p, 2, 8, 32, 32, 16, 48, None) == bga.IKBO_ERR_UNSUPPORTED  # width
    assert f(p, p, p, p, p, p, 200, 8, 32, 32, 96, 160, None) == bga.IKBO_ERR_UNSUPPORTED  # P_u > scratch
    assert "scratch" in bga.last_error_message()
