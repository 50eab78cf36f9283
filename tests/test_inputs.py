"""The seeded input generator and the configurations against the pages' shape facts."""
import json
import os

import numpy as np
import pytest

from broadcast_gemm_amd.inputs import (CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits, make_inputs,
                                       make_integer_inputs, sorted_map)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_deterministic_per_seed():
    a = make_inputs(CONFIGS[2])
    b = make_inputs(CONFIGS[2])
    for n in ("U", "C", "W_u", "W_c", "map"):
        assert np.array_equal(getattr(a, n), getattr(b, n))
    c = make_inputs(CONFIGS[2], seed=99)
    assert not np.array_equal(a.C, c.C)


def test_sorted_run_lengths():
    assert sorted(np.bincount(sorted_map(15, 1024)).tolist()) == [68] * 11 + [69] * 4
    assert sorted(np.bincount(sorted_map(26, 256)).tolist()) == [9] * 4 + [10] * 22
    assert np.bincount(sorted_map(2, 20000)).tolist() == [10000, 10000]
    m = sorted_map(15, 1024)
    assert np.all(np.diff(m) >= 0) and m[0] == 0 and m[-1] == 14


def test_tiny_explicit_map_and_dtype():
    x = make_inputs(CONFIGS[0])
    assert x.map.tolist() == [0, 0, 0, 0, 1, 1, 1, 1]
    assert x.U.dtype == np.float32 and x.U.shape == (2, 13, 16) and x.C.shape == (8, 11, 16)
    assert x.W_u.shape == (8, 13) and x.W_c.shape == (8, 11)


def test_random_map_range():
    cfg = CONFIGS[3].with_batch(59, 4096)
    x = make_inputs(cfg.__class__(**{**cfg.__dict__, "K_u": 3, "K_c": 2, "M": 2, "D": 8}))
    assert x.map.min() >= 0 and x.map.max() < 59 and not np.all(np.diff(x.map) >= 0)


def test_bf16_rounding_is_rne():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: ties go to the even mantissa (1.0).
    vals = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -(1.0 + 2 ** -8), 3.0e38,
                     np.inf, -np.inf, 0.0, -0.0], dtype=np.float32)
    out = bf16_bits_to_f32(f32_to_bf16_bits(vals))
    want = np.array([1.0, 1.0 + 2 ** -6, 1.0, -1.0, np.float32(3.0e38), np.inf, -np.inf, 0.0, -0.0],
                    dtype=np.float32)
    assert np.array_equal(out[:4], want[:4])
    assert np.isinf(out[5]) and np.isinf(out[6]) and out[7] == 0
    assert np.signbit(out[8])
    assert abs(out[4] - 3.0e38) / 3.0e38 < 2 ** -8


def test_fast_rounding_path_agrees():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(200000).astype(np.float32) * 10
    from broadcast_gemm_amd.inputs import _round_bf16_fast
    assert np.array_equal(_round_bf16_fast(x), f32_to_bf16_bits(x))


def test_weight_scale():
    x = make_inputs(CONFIGS[1].with_batch(15, 16))
    w = bf16_bits_to_f32(x.W_c)
    assert abs(w.std() * np.sqrt(498) - 1.0) < 0.05


def test_integer_inputs_are_small_integers():
    x = make_integer_inputs(CONFIGS[1].with_batch(3, 5))
    for n in ("U", "C", "W_u", "W_c"):
        v = x.as_f32(n)
        assert set(np.unique(v).tolist()) <= {-1.0, 0.0, 1.0}


def test_configs_follow_page_facts():
    facts = json.load(open(os.path.join(GOLDEN, "pages_facts.json")))
    c1 = CONFIGS[1]
    assert c1.B_c == facts["candidates_per_request"]["value"]
    assert c1.B_u == facts["users_per_request_approx"]["value"]
    assert round(c1.B_c / c1.B_u) == pytest.approx(facts["candidate_user_ratio"]["value"], abs=2)
    # Decomposition runs the user product at B_u rows instead of B_c: share of user work left.
    assert 1.0 - c1.B_u / c1.B_c > facts["user_work_removed_min_fraction"]["value"]
    lo, hi = facts["batch_envelope"]["value"]
    rlo, rhi = facts["ratio_envelope"]["value"]
    for c in CONFIGS[1:]:
        ratio = c.B_c / c.B_u
        assert rlo * 0.9 <= ratio <= rhi * 1.01
    assert lo <= CONFIGS[2].B_c and CONFIGS[3].B_c <= hi


def test_golden_tiny_oracle_reproduces(oracle_mod):
    doc = json.load(open(os.path.join(GOLDEN, "tiny_oracle.json")))
    s = doc["shapes"]
    x = make_inputs(CONFIGS[0])
    assert np.array_equal(np.array(doc["U"], np.float32).reshape(x.U.shape), x.U)
    assert np.array_equal(np.array(doc["C"], np.float32).reshape(x.C.shape), x.C)
    Y = oracle_mod.lce_f64(x.U, x.C, x.map, x.W_u, x.W_c)
    want = np.array([float.fromhex(h) for h in doc["Y"]]).reshape(s["B_c"], s["M"], s["D"])
    assert np.array_equal(Y, want)
