"""The CPU oracle against its pins (see ``tests/pins.py``), plus mutation tests:
slips planted in copies of the oracle's C source must each fail some pin."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import pins
from broadcast_gemm_amd.inputs import CONFIGS, make_inputs, make_tag_inputs

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "ikbo_oracle.c")


@pytest.fixture(scope="module")
def f(oracle_mod):
    return lambda U, C, mp, W_u, W_c: oracle_mod.lce_f64(U, C, mp, W_u, W_c)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("name,pin", pins.ALL_PINS, ids=[n for n, _ in pins.ALL_PINS])
def test_pin(f, dtype, name, pin):
    pin(f, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_pin_bruteforce(f, dtype):
    pins.pin_bruteforce(f, np.random.default_rng(3 if dtype == "bf16" else 4), dtype)


def test_tiny_config_bruteforce(f):
    """The tiny configuration itself against the exact rational value."""
    x = make_inputs(CONFIGS[0])
    Y = f(x.U, x.C, x.map, x.W_u, x.W_c)
    Yx, S = pins.fraction_bruteforce(x.U, x.C, x.map, x.W_u, x.W_c)
    from fractions import Fraction
    err = np.vectorize(lambda y, e: float(abs(Fraction(float(y)) - e)), otypes=[float])(Y, Yx)
    assert np.all(err <= 1e-12 * S)


def test_map_out_of_range_rejected(oracle_mod):
    x = make_inputs(CONFIGS[0])
    bad = x.map.copy()
    bad[3] = 2
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.lce_f64(x.U, x.C, bad, x.W_u, x.W_c)
    bad[3] = -1
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.lce_f64(x.U, x.C, bad, x.W_u, x.W_c)


def test_row_subset_matches_full(oracle_mod):
    x = make_inputs(CONFIGS[2])
    rows = [0, 5, 255, 17, 17]
    full = oracle_mod.lce_f64(x.U, x.C, x.map, x.W_u, x.W_c)
    sub = oracle_mod.lce_f64(x.U, x.C, x.map, x.W_u, x.W_c, rows=rows)
    assert np.array_equal(sub, full[rows])


def test_thread_count_does_not_change_bits(oracle_mod):
    x = make_inputs(CONFIGS[2].with_batch(7, 33))
    a = oracle_mod.lce_f64(x.U, x.C, x.map, x.W_u, x.W_c, threads=1)
    b = oracle_mod.lce_f64(x.U, x.C, x.map, x.W_u, x.W_c, threads=5)
    assert np.array_equal(a, b)


def test_tag_on_full_config_maps(oracle_mod):
    """The gather tag at the real batch sizes and maps of the bf16 configurations."""
    for cfg in CONFIGS[1:4]:
        small = cfg.with_batch(cfg.B_u, cfg.B_c)
        small = small.__class__(**{**small.__dict__, "K_u": 3, "K_c": 2, "M": 2, "D": 8})
        x = make_tag_inputs(small)
        Y = oracle_mod.lce_f64(x.U, x.C, x.map, x.W_u, x.W_c)
        assert np.array_equal(Y, np.broadcast_to((x.map + 1.0)[:, None, None], Y.shape))


def test_output_scale_is_unit_normal(oracle_mod):
    """Fan-in scaling of W makes each Y element about N(0, 1)."""
    x = make_inputs(CONFIGS[2])
    Y = oracle_mod.lce_f64(x.U, x.C, x.map, x.W_u, x.W_c)
    assert 0.95 < Y.std() < 1.05 and abs(Y.mean()) < 0.02


# ----------------------------------------------------------------------------------
# Mutation tests: each planted slip must be caught by at least one pin.
# ----------------------------------------------------------------------------------
MUTANTS = {
    "gather_by_candidate_index": (
        "const int64_t u = map[b];", "const int64_t u = b % B_u;"),
    "map_read_backwards": (
        "const int64_t u = map[b];", "const int64_t u = map[B_c - 1 - b];"),
    "W_u_transposed": (
        "W[m * K + k] = widen(W_u, m * K_u + k, dtype);",
        "W[m * K + k] = widen(W_u, (k * M + m) % (M * K_u), dtype);"),
    "W_c_transposed": (
        "W[m * K + K_u + k] = widen(W_c, m * K_c + k, dtype);",
        "W[m * K + K_u + k] = widen(W_c, (k * M + m) % (M * K_c), dtype);"),
    "first_k_dropped": (
        "for (int64_t k = 0; k < K; ++k) {", "for (int64_t k = 1; k < K; ++k) {"),
    "last_k_dropped": (
        "for (int64_t k = 0; k < K; ++k) {", "for (int64_t k = 0; k + 1 < K; ++k) {"),
    "user_term_dropped": (
        "X[k * D + d] = widen(U, (u * K_u + k) * D + d, dtype);", "X[k * D + d] = 0.0;"),
    "candidate_rows_shifted": (
        "X[(K_u + k) * D + d] = widen(C, (b * K_c + k) * D + d, dtype);",
        "X[(K_u + k) * D + d] = widen(C, (b * K_c + (k + 1) % K_c) * D + d, dtype);"),
    "columns_reversed": (
        "for (int64_t d = 0; d < D; ++d) acc[d] += w * x[d];",
        "for (int64_t d = 0; d < D; ++d) acc[d] += w * x[D - 1 - d];"),
    "sign_flipped_on_candidates": (
        "const double w = W[m * K + k];", "const double w = (k < K_u) ? W[m * K + k] : -W[m * K + k];"),
    "bf16_widening_wrong": (
        "uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;",
        "uint32_t bits = ((uint32_t)((const uint16_t *)base)[i] << 16) | 0x8000u;"),
    "single_precision_accumulation": (
        "for (int64_t d = 0; d < D; ++d) acc[d] += w * x[d];",
        "for (int64_t d = 0; d < D; ++d) acc[d] = (float)(acc[d] + (float)(w * x[d]));"),
}


def _build_mutant(tmp_path, name, old, new):
    src = open(ORACLE_SRC).read()
    # The forward's slips are planted in the forward function only (the backward follows it).
    cut = src.index("int ikbo_oracle_lce_backward_f64(")
    fwd, rest = src[:cut], src[cut:]
    assert fwd.count(old) == 1, f"mutant {name}: anchor not found once in the oracle's forward"
    path = tmp_path / f"{name}.c"
    path.write_text(fwd.replace(old, new) + rest)
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                    "-o", str(so), str(path)], check=True)
    lib = ctypes.CDLL(str(so))
    fn = lib.ikbo_oracle_lce_f64
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int64] * 6 + [ctypes.c_int, ctypes.c_void_p,
                                                                   ctypes.c_int64, ctypes.c_int]

    def call(U, C, mp, W_u, W_c):
        U, C, W_u, W_c = (np.ascontiguousarray(a) for a in (U, C, W_u, W_c))
        mp = np.ascontiguousarray(mp, dtype=np.int32)
        code = 0 if U.dtype == np.uint16 else 1
        B_u, K_u, D = U.shape
        B_c, K_c, _ = C.shape
        M = W_u.shape[0]
        Y = np.empty((B_c, M, D))
        st = fn(U.ctypes.data, C.ctypes.data, mp.ctypes.data, W_u.ctypes.data, W_c.ctypes.data,
                Y.ctypes.data, B_u, B_c, K_u, K_c, M, D, code, None, B_c, 1)
        if st != 0:
            raise AssertionError(f"mutant returned {st}")
        return Y
    return call


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_oracle_mutants(tmp_path, name):
    old, new = MUTANTS[name]
    f = _build_mutant(tmp_path, name, old, new)
    failed = pins.run_all(f, "bf16", with_bruteforce=False) + pins.run_all(f, "f32", with_bruteforce=False)
    if not failed:
        try:
            pins.pin_bruteforce(f, np.random.default_rng(3), "f32")
        except AssertionError:
            failed.append("bruteforce")
    assert failed, f"planted slip '{name}' passed every pin"
