"""The oracle's backward against its pins (``tests/pins_bwd.py``), plus mutation tests:
slips planted in copies of the backward's C source must each fail some pin."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import pins_bwd
from broadcast_gemm_amd.inputs import CONFIGS, make_inputs

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "ikbo_oracle.c")


@pytest.fixture(scope="module")
def g(oracle_mod):
    return oracle_mod.lce_backward_f64


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("name,pin", pins_bwd.ALL_PINS, ids=[n for n, _ in pins_bwd.ALL_PINS])
def test_pin(g, dtype, name, pin):
    pin(g, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_pin_bruteforce(g, dtype):
    pins_bwd.pin_bwd_bruteforce(g, np.random.default_rng(5 if dtype == "bf16" else 6), dtype)


def test_thread_count_does_not_change_bits(oracle_mod):
    x = make_inputs(CONFIGS[2].with_batch(7, 33))
    dY = np.random.default_rng(9).standard_normal((33, x.cfg.M, x.cfg.D)).astype(np.float32)
    from broadcast_gemm_amd.inputs import f32_to_bf16_bits
    dY = f32_to_bf16_bits(dY)
    a = oracle_mod.lce_backward_f64(dY, x.U, x.C, x.map, x.W_u, x.W_c, threads=1)
    b = oracle_mod.lce_backward_f64(dY, x.U, x.C, x.map, x.W_u, x.W_c, threads=5)
    for p, q in zip(a, b):
        assert np.array_equal(p, q)


def test_sampled_rows_match_full(oracle_mod):
    """The sampled entry point returns exactly the requested rows of the full gradients."""
    x = make_inputs(CONFIGS[2].with_batch(5, 21))
    from broadcast_gemm_amd.inputs import f32_to_bf16_bits
    dY = f32_to_bf16_bits(np.random.default_rng(8).standard_normal((21, x.cfg.M, x.cfg.D)).astype(np.float32))
    dU, dC, dW_u, dW_c = oracle_mod.lce_backward_f64(dY, x.U, x.C, x.map, x.W_u, x.W_c)
    K_u = x.cfg.K_u
    pc, pu, pw = [(3, 0), (20, 196), (3, 0)], [(int(x.map[7]), 300), (0, 5)], [(0, 0), (95, K_u), (4, K_u + 196)]
    oc, ou, ow = oracle_mod.lce_backward_rows_f64(dY, x.U, x.C, x.map, x.W_u, x.W_c, pc, pu, pw)
    assert np.array_equal(oc, np.stack([dC[b, k] for b, k in pc]))
    assert np.array_equal(ou, np.stack([dU[u, k] for u, k in pu]))
    assert np.array_equal(ow, [dW_u[0, 0], dW_c[95, 0], dW_c[4, 196]])
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.lce_backward_rows_f64(dY, x.U, x.C, x.map, x.W_u, x.W_c, dc_rows=[(21, 0)])


def test_map_out_of_range_rejected(oracle_mod):
    x = make_inputs(CONFIGS[0])
    dY = np.ones((8, 8, 16), np.float32)
    bad = x.map.copy()
    bad[5] = 2
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.lce_backward_f64(dY, x.U, x.C, bad, x.W_u, x.W_c)


# ----------------------------------------------------------------------------------
# Mutation tests: each planted slip in the backward must be caught by a pin.
# ----------------------------------------------------------------------------------
MUTANTS = {
    "dC_reads_user_rows": (
        "const int64_t b = dc_rows[2 * i], k = K_u + dc_rows[2 * i + 1];",
        "const int64_t b = dc_rows[2 * i], k = dc_rows[2 * i + 1];"),
    "dU_own_index": (
        "if (map[b] != u) continue;", "if (b % B_u != u) continue;"),
    "dU_first_candidate_only": (
        "for (int64_t d = 0; d < D; ++d) acc[d] += x[d];",
        "for (int64_t d = 0; d < D; ++d) acc[d] = x[d];"),
    "dU_reads_candidate_rows": (
        "const int64_t u = du_rows[2 * i], k = du_rows[2 * i + 1];",
        "const int64_t u = du_rows[2 * i], k = du_rows[2 * i + 1] % (K_c > 0 ? K_c : 1) + K_u;"),
    "dX_uses_W_not_W_T": (
        "const double w = W[m * K + k];\n                        for (int64_t d = 0; d < D; ++d) x[d]",
        "const double w = W[(k % M) * K + (m % K)];\n                        for (int64_t d = 0; d < D; ++d) x[d]"),
    "dC_column_reversed": (
        "for (int64_t d = 0; d < D; ++d) out[d] += w * widen(dY, (b * M + m) * D + d, dtype);",
        "for (int64_t d = 0; d < D; ++d) out[d] += w * widen(dY, (b * M + m) * D + (D - 1 - d), dtype);"),
    "dW_user_by_candidate_index": (
        "? widen(U, ((int64_t)map[b] * K_u + k) * D + d, dtype)",
        "? widen(U, ((int64_t)(b % B_u) * K_u + k) * D + d, dtype)"),
    "dW_candidate_rows_shifted": (
        ": widen(C, (b * K_c + (k - K_u)) * D + d, dtype);",
        ": widen(C, (b * K_c + (k - K_u + 1) % K_c) * D + d, dtype);"),
    "dW_last_candidate_dropped": (
        "for (int64_t b = 0; b < B_c; ++b) {\n            for (int64_t d = 0; d < D; ++d) {",
        "for (int64_t b = 0; b + 1 < B_c; ++b) {\n            for (int64_t d = 0; d < D; ++d) {"),
    "dW_sign_on_users": (
        "dW[i] = acc;", "dW[i] = k < K_u ? -acc : acc;"),
    "dW_row_shifted": (
        "const int64_t m = dw_elems[2 * i], k = dw_elems[2 * i + 1];",
        "const int64_t m = (dw_elems[2 * i] + 1) % M, k = dw_elems[2 * i + 1];"),
    "dY_rows_shifted": (
        "for (int64_t d = 0; d < D; ++d) x[d] += w * widen(dY, (b * M + m) * D + d, dtype);",
        "for (int64_t d = 0; d < D; ++d) x[d] += w * widen(dY, (b * M + (m + 1) % M) * D + d, dtype);"),
}


def _build_mutant(tmp_path, name, old, new):
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, f"mutant {name}: anchor not found once in the oracle source"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                    "-o", str(so), str(path)], check=True)
    lib = ctypes.CDLL(str(so))
    fn = lib.ikbo_oracle_lce_backward_f64
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int64] * 6 + [ctypes.c_int] + [
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p] * 3 + [ctypes.c_int]

    def call(dY, U, C, mp, W_u, W_c):
        dY, U, C, W_u, W_c = (np.ascontiguousarray(a) for a in (dY, U, C, W_u, W_c))
        mp = np.ascontiguousarray(mp, dtype=np.int32)
        code = 0 if U.dtype == np.uint16 else 1
        B_u, K_u, D = U.shape
        B_c, K_c, _ = C.shape
        M = W_u.shape[0]
        grid = lambda a, b: np.ascontiguousarray(
            np.stack(np.meshgrid(np.arange(a), np.arange(b), indexing="ij"), -1).reshape(-1, 2).astype(np.int64))
        pc, pu, pw = grid(B_c, K_c), grid(B_u, K_u), grid(M, K_u + K_c)
        oc, ou, ow = np.empty((len(pc), D)), np.empty((len(pu), D)), np.empty(len(pw))
        st = fn(dY.ctypes.data, U.ctypes.data, C.ctypes.data, mp.ctypes.data, W_u.ctypes.data,
                W_c.ctypes.data, B_u, B_c, K_u, K_c, M, D, code, pc.ctypes.data, len(pc), oc.ctypes.data,
                pu.ctypes.data, len(pu), ou.ctypes.data, pw.ctypes.data, len(pw), ow.ctypes.data, 1)
        if st != 0:
            raise AssertionError(f"mutant returned {st}")
        dW = ow.reshape(M, K_u + K_c)
        return ou.reshape(B_u, K_u, D), oc.reshape(B_c, K_c, D), dW[:, :K_u].copy(), dW[:, K_u:].copy()
    return call


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_backward_mutants(tmp_path, name):
    old, new = MUTANTS[name]
    f = _build_mutant(tmp_path, name, old, new)
    failed = pins_bwd.run_all(f, "bf16", with_bruteforce=False) + pins_bwd.run_all(f, "f32", with_bruteforce=False)
    if not failed:
        try:
            pins_bwd.pin_bwd_bruteforce(f, np.random.default_rng(5), "f32")
        except AssertionError:
            failed.append("bruteforce")
    assert failed, f"planted slip '{name}' passed every pin"
