"""The oracle's IKBO target attention against its pins (``tests/pins_fa.py``), plus
mutation tests: slips planted in copies of its C source must each fail some pin."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import pins_fa

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "ikbo_oracle.c")


@pytest.fixture(scope="module")
def f(oracle_mod):
    return lambda Q, K, V, mp, scale=None: oracle_mod.fa_f64(Q, K, V, mp, scale=scale)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("name,pin", pins_fa.ALL_PINS, ids=[n for n, _ in pins_fa.ALL_PINS])
def test_pin(f, dtype, name, pin):
    pin(f, dtype)


def test_sampled_rows_match_full(oracle_mod):
    from broadcast_gemm_amd.inputs import FA_CONFIGS, make_fa_inputs
    x = make_fa_inputs(FA_CONFIGS[0])
    full = oracle_mod.fa_f64(x.Q, x.K, x.V, x.map)
    rows = [(5, 1, 15), (0, 0, 0), (3, 1, 7)]
    assert np.array_equal(oracle_mod.fa_f64(x.Q, x.K, x.V, x.map, rows=rows), np.stack([full[r] for r in rows]))
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.fa_f64(x.Q, x.K, x.V, x.map, rows=[(6, 0, 0)])
    bad = x.map.copy()
    bad[2] = 2
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.fa_f64(x.Q, x.K, x.V, bad)


MUTANTS = {
    "user_by_candidate_index": ("const int64_t u = map[b];\n                for (int64_t k = 0; k < L_kv; ++k)",
                                "const int64_t u = b % B_u;\n                for (int64_t k = 0; k < L_kv; ++k)"),
    "scale_dropped": ("sc[k] = scale * t;", "sc[k] = t;"),
    "keys_shifted": ("Kb[k * hd + d] = widen(K, ((u * H + h) * L_kv + k) * hd + d, dtype);",
                     "Kb[k * hd + d] = widen(K, ((u * H + h) * L_kv + (k + 1) % L_kv) * hd + d, dtype);"),
    "values_from_keys": ("Vb[k * hd + d] = widen(V, ((u * H + h) * L_kv + k) * hd + d, dtype);",
                         "Vb[k * hd + d] = widen(K, ((u * H + h) * L_kv + k) * hd + d, dtype);"),
    "head_ignored_for_kv": ("Vb[k * hd + d] = widen(V, ((u * H + h) * L_kv + k) * hd + d, dtype);",
                            "Vb[k * hd + d] = widen(V, ((u * H + 0) * L_kv + k) * hd + d, dtype);"),
    "not_normalised": ("for (int64_t d = 0; d < hd; ++d) out[d] /= l;", "for (int64_t d = 0; d < hd; ++d) out[d] /= L_kv;"),
    "last_key_dropped": ("    sc[k] = exp(sc[k] - mx);\n                    l += sc[k];\n                }\n                double *out = O + i * hd;\n                for (int64_t d = 0; d < hd; ++d) out[d] = 0.0;\n                for (int64_t k = 0; k < L_kv; ++k)",
                         "    sc[k] = exp(sc[k] - mx);\n                    l += sc[k];\n                }\n                double *out = O + i * hd;\n                for (int64_t d = 0; d < hd; ++d) out[d] = 0.0;\n                for (int64_t k = 0; k + 1 < L_kv; ++k)"),
    "query_row_swapped": ("qv[d] = widen(Q, ((b * H + h) * L_q + q) * hd + d, dtype);",
                          "qv[d] = widen(Q, ((b * H + h) * L_q + (L_q - 1 - q)) * hd + d, dtype);"),
    "exp_without_max_sign": ("sc[k] = exp(sc[k] - mx);", "sc[k] = exp(mx - sc[k]);"),
    "columns_reversed": ("for (int64_t d = 0; d < hd; ++d) out[d] += sc[k] * Vb[k * hd + d];",
                         "for (int64_t d = 0; d < hd; ++d) out[d] += sc[k] * Vb[k * hd + (hd - 1 - d)];"),
}


def _build_mutant(tmp_path, name, old, new):
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, f"mutant {name}: anchor not found once in the oracle source"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                    "-o", str(so), str(path), "-lm"], check=True)
    fn = ctypes.CDLL(str(so)).ikbo_oracle_fa_f64
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64] * 6 + [ctypes.c_double, ctypes.c_int, ctypes.c_void_p,
                                                                   ctypes.c_int64, ctypes.c_void_p, ctypes.c_int]

    def call(Q, K, V, mp, scale=None):
        Q, K, V = (np.ascontiguousarray(a) for a in (Q, K, V))
        mp = np.ascontiguousarray(mp, dtype=np.int32)
        B_c, H, L_q, hd = Q.shape
        B_u, _, L_kv, _ = K.shape
        rows = np.ascontiguousarray(np.stack(np.meshgrid(np.arange(B_c), np.arange(H), np.arange(L_q), indexing="ij"),
                                             -1).reshape(-1, 3).astype(np.int64))
        O = np.empty((len(rows), hd))
        st = fn(Q.ctypes.data, K.ctypes.data, V.ctypes.data, mp.ctypes.data, B_u, B_c, H, L_q, L_kv, hd,
                float(1.0 / np.sqrt(hd) if scale is None else scale), 0 if Q.dtype == np.uint16 else 1,
                rows.ctypes.data, len(rows), O.ctypes.data, 1)
        if st != 0:
            raise AssertionError(f"mutant returned {st}")
        return O.reshape(B_c, H, L_q, hd)
    return call


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_fa_mutants(tmp_path, name):
    old, new = MUTANTS[name]
    f = _build_mutant(tmp_path, name, old, new)
    failed = pins_fa.run_all(f, "bf16") + pins_fa.run_all(f, "f32")
    assert failed, f"planted slip '{name}' passed every pin"


def test_weight_bound_is_the_attention_of_abs_v(oracle_mod):
    """The attention bar's extra term: 2^-8 times the oracle's attention over |V|, which lies
    between the smallest and largest |V| row value and is zero for V = 0."""
    from broadcast_gemm_amd.inputs import FA_CONFIGS, make_fa_inputs
    from pins import _f
    x = make_fa_inputs(FA_CONFIGS[0])
    wb = oracle_mod.fa_weight_bound(x.Q, x.K, x.V, x.map)
    Va = np.abs(_f(x.V))[x.map]
    assert np.all(wb >= Va.min(axis=2, keepdims=True) * 2.0 ** -8 - 1e-15)
    assert np.all(wb <= Va.max(axis=2, keepdims=True) * 2.0 ** -8 + 1e-15)
    assert np.all(oracle_mod.fa_weight_bound(x.Q, x.K, np.zeros_like(x.V), x.map) == 0)
