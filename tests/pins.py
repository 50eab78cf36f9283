"""Pins for the CPU oracle: checks against facts the oracle cannot supply itself.

Each ``pin_*`` takes ``f(U, C, map, W_u, W_c) -> Y`` (numpy in, float64 out) and
raises AssertionError when ``f`` disagrees with the fact it pins.  The suite is
chosen so that a plausible slip anywhere in the oracle (a dropped or shifted
term, a transposed operand, the map read the wrong way, a wrong sign, a bad
bf16 widening) fails at least one pin; ``test_oracle_mutants`` plants such slips
in copies of the oracle source and checks exactly that.

Facts used (IKBO recsys blog, "Deep Dive: Linear Compression"; aibriefing
article, "kernel deep-dive case 1"; plus plain linear algebra):
  * exact value: bf16/fp32 numbers are dyadic rationals, so the operator's value
    is computable exactly with ``fractions.Fraction`` (brute force, tiny sizes);
  * orientation: a W with a single 1 at (m0, k0) copies input row k0 into output
    row m0 (closed form);
  * library special cases: identity map reduces to ``numpy.matmul`` of [W_u|W_c]
    with [U;C]; C = 0 reduces to gathering rows of ``W_u @ U``; U = 0 reduces
    to ``W_c @ C``;
  * stage 1: the decomposed form equals the materialised one (by linearity);
  * stage 2: zero K-padding leaves every output bit unchanged;
  * linearity in (U, C); power-of-two scaling is exact;
  * permutation structure: candidates permute rows; relabelling users is a no-op;
  * gather tag: Y[b, m, d] = map[b] + 1 for the tag inputs.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from broadcast_gemm_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits


def _f(a):
    """Exact float64 view of stored values (bf16 bit patterns or float32)."""
    return (bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)


def _store_like(x, like):
    x = np.asarray(x, dtype=np.float32)
    return f32_to_bf16_bits(x) if like.dtype == np.uint16 else x


def rand_case(rng, dtype, B_u, B_c, K_u, K_c, M, D, sorted_map=False, ints=False):
    def draw(shape):
        x = rng.integers(-3, 4, size=shape).astype(np.float32) if ints else \
            rng.standard_normal(shape).astype(np.float32)
        return f32_to_bf16_bits(x) if dtype == "bf16" else x
    U, C = draw((B_u, K_u, D)), draw((B_c, K_c, D))
    W_u, W_c = draw((M, K_u)), draw((M, K_c))
    mp = np.sort(rng.integers(0, B_u, B_c)) if sorted_map else rng.integers(0, B_u, B_c)
    return U, C, mp.astype(np.int32), W_u, W_c


def fraction_bruteforce(U, C, mp, W_u, W_c):
    """Exact value (decomposed form) and the sum of |terms| per element."""
    Uf, Cf, Wuf, Wcf = (_f(a) for a in (U, C, W_u, W_c))
    B_c, K_c, D = C.shape
    M, K_u = W_u.shape
    Y = np.empty((B_c, M, D), dtype=object)
    S = np.empty((B_c, M, D), dtype=np.float64)
    for b in range(B_c):
        u = int(mp[b])
        for m in range(M):
            for d in range(D):
                tot = Fraction(0)
                mag = 0.0
                for k in range(K_u):
                    t = Fraction(float(Wuf[m, k])) * Fraction(float(Uf[u, k, d]))
                    tot += t
                    mag += abs(float(t))
                for k in range(K_c):
                    t = Fraction(float(Wcf[m, k])) * Fraction(float(Cf[b, k, d]))
                    tot += t
                    mag += abs(float(t))
                Y[b, m, d] = tot
                S[b, m, d] = mag
    return Y, S


def pin_bruteforce(f, rng, dtype):
    shapes = [(1, 1, 1, 1, 1, 1), (2, 5, 3, 4, 2, 3), (3, 6, 9, 7, 5, 7), (1, 4, 8, 1, 3, 2),
              (3, 2, 1, 9, 4, 5), (2, 6, 5, 5, 5, 6)]
    for (B_u, B_c, K_u, K_c, M, D) in shapes:
        U, C, mp, W_u, W_c = rand_case(rng, dtype, B_u, B_c, K_u, K_c, M, D)
        Y = f(U, C, mp, W_u, W_c)
        Yx, S = fraction_bruteforce(U, C, mp, W_u, W_c)
        assert Y.shape == Yx.shape, (Y.shape, Yx.shape)
        err = np.array([[[abs(Fraction(float(Y[b, m, d])) - Yx[b, m, d]) for d in range(D)]
                         for m in range(M)] for b in range(B_c)], dtype=np.float64)
        assert np.all(err <= 1e-12 * S + 1e-300), f"brute force mismatch, max err {err.max()}"


def pin_orientation(f, dtype):
    rng = np.random.default_rng(7)
    B_u, B_c, K_u, K_c, M, D = 3, 5, 4, 6, 7, 9
    U0, C0, mp, _, _ = rand_case(rng, dtype, B_u, B_c, K_u, K_c, M, D)
    Uf, Cf = _f(U0), _f(C0)
    for (m0, k0) in [(0, 0), (6, 5), (2, 3)]:
        W_u = np.zeros((M, K_u), np.float32)
        W_c = np.zeros((M, K_c), np.float32)
        W_c[m0, k0] = 1.0
        Y = f(U0, C0, mp, _store_like(W_u, U0), _store_like(W_c, U0))
        want = np.zeros((B_c, M, D))
        want[:, m0, :] = Cf[:, k0, :]
        assert np.array_equal(Y, want), f"W_c orientation (m0={m0}, k0={k0})"
    for (m0, k0) in [(0, 0), (6, 3), (4, 1)]:
        W_u = np.zeros((M, K_u), np.float32)
        W_c = np.zeros((M, K_c), np.float32)
        W_u[m0, k0] = 1.0
        Y = f(U0, C0, mp, _store_like(W_u, U0), _store_like(W_c, U0))
        want = np.zeros((B_c, M, D))
        want[:, m0, :] = Uf[mp, k0, :]
        assert np.array_equal(Y, want), f"W_u orientation / gather (m0={m0}, k0={k0})"


def pin_library_special_cases(f, dtype):
    rng = np.random.default_rng(11)
    B, K_u, K_c, M, D = 6, 5, 7, 4, 8
    U, C, _, W_u, W_c = rand_case(rng, dtype, B, B, K_u, K_c, M, D)
    ident = np.arange(B, dtype=np.int32)
    Y = f(U, C, ident, W_u, W_c)
    W = np.concatenate([_f(W_u), _f(W_c)], axis=1)
    X = np.concatenate([_f(U), _f(C)], axis=1)
    ref = np.matmul(W, X)
    assert np.allclose(Y, ref, rtol=1e-12, atol=1e-12), "identity map != matmul([W_u|W_c], [U;C])"
    mp = rng.integers(0, B, B).astype(np.int32)
    Cz = _store_like(np.zeros(C.shape, np.float32), C)
    Y = f(U, Cz, mp, W_u, W_c)
    ref = np.take(np.matmul(_f(W_u), _f(U)), mp, axis=0)
    assert np.allclose(Y, ref, rtol=1e-12, atol=1e-12), "C=0 != index_select(W_u @ U, map)"
    Uz = _store_like(np.zeros(U.shape, np.float32), U)
    Y = f(Uz, C, mp, W_u, W_c)
    ref = np.matmul(_f(W_c), _f(C))
    assert np.allclose(Y, ref, rtol=1e-12, atol=1e-12), "U=0 != W_c @ C"


def pin_decomposed_equals_materialised(f, dtype):
    rng = np.random.default_rng(13)
    for ints in (False, True):
        U, C, mp, W_u, W_c = rand_case(rng, dtype, 4, 9, 11, 6, 5, 8, ints=ints)
        Y = f(U, C, mp, W_u, W_c)
        dec = np.take(np.matmul(_f(W_u), _f(U)), mp, axis=0) + np.matmul(_f(W_c), _f(C))
        if ints:
            assert np.array_equal(Y, dec), "integer data: decomposed != materialised"
        else:
            assert np.allclose(Y, dec, rtol=1e-12, atol=1e-12), "decomposed != materialised"


def pin_zero_padding(f, dtype):
    rng = np.random.default_rng(17)
    U, C, mp, W_u, W_c = rand_case(rng, dtype, 3, 7, 13, 11, 6, 8)
    Y = f(U, C, mp, W_u, W_c)
    pu, pc = 3, 5   # pad K_u 13 -> 16 and K_c 11 -> 16 with zeros

    def padk(a, p, axis):
        w = [(0, 0)] * a.ndim
        w[axis] = (0, p)
        return np.pad(a, w)
    Yp = f(padk(U, pu, 1), padk(C, pc, 1), mp, padk(W_u, pu, 1), padk(W_c, pc, 1))
    assert np.array_equal(Y, Yp), "zero K-padding changed the result"


def pin_linearity(f, dtype):
    rng = np.random.default_rng(19)
    U, C, mp, W_u, W_c = rand_case(rng, dtype, 3, 8, 7, 9, 5, 6)
    Y = f(U, C, mp, W_u, W_c)
    two = lambda a: _store_like(2.0 * _f(a).astype(np.float32), a)  # noqa: E731 (exact)
    Y2 = f(two(U), two(C), mp, W_u, W_c)
    assert np.array_equal(Y2, 2.0 * Y), "Y(2U, 2C) != 2 Y(U, C)"
    zU = _store_like(np.zeros(U.shape, np.float32), U)
    zC = _store_like(np.zeros(C.shape, np.float32), C)
    Ysum = f(U, zC, mp, W_u, W_c) + f(zU, C, mp, W_u, W_c)
    assert np.allclose(Y, Ysum, rtol=1e-12, atol=1e-12), "Y(U,C) != Y(U,0) + Y(0,C)"


def pin_permutations(f, dtype):
    rng = np.random.default_rng(23)
    U, C, mp, W_u, W_c = rand_case(rng, dtype, 4, 9, 6, 5, 4, 7)
    Y = f(U, C, mp, W_u, W_c)
    p = rng.permutation(C.shape[0])
    Yp = f(U, C[p], mp[p], W_u, W_c)
    assert np.array_equal(Yp, Y[p]), "permuting candidates must permute output rows"
    q = rng.permutation(U.shape[0])       # new label of old user u is inv[u]
    inv = np.argsort(q)
    Yq = f(U[q], C, inv[mp].astype(np.int32), W_u, W_c)
    assert np.array_equal(Yq, Y), "relabelling users must not change the output"


def pin_tag(f, dtype):
    for (B_u, B_c) in [(1, 3), (5, 17), (15, 40)]:
        rng = np.random.default_rng(B_c)
        mp = rng.integers(0, B_u, B_c).astype(np.int32)
        K_u, K_c, M, D = 3, 2, 4, 8
        U = np.zeros((B_u, K_u, D), np.float32)
        U[:, 0, :] = (np.arange(B_u, dtype=np.float32) + 1)[:, None]
        W_u = np.zeros((M, K_u), np.float32)
        W_u[:, 0] = 1
        like = np.zeros(1, np.uint16 if dtype == "bf16" else np.float32)
        Y = f(_store_like(U, like), _store_like(np.zeros((B_c, K_c, D)), like), mp,
              _store_like(W_u, like), _store_like(np.zeros((M, K_c)), like))
        want = np.broadcast_to((mp + 1).astype(np.float64)[:, None, None], (B_c, M, D))
        assert np.array_equal(Y, want), "gather tag: Y[b] must equal map[b] + 1"


def pin_closed_form_constants(f, dtype):
    # U = a, C = c, W_u = w_u, W_c = w_c everywhere: Y = K_u*w_u*a + K_c*w_c*c.
    B_u, B_c, K_u, K_c, M, D = 2, 3, 13, 11, 8, 16
    a, c, wu, wc = 0.5, -1.25, 2.0, 0.75
    like = np.zeros(1, np.uint16 if dtype == "bf16" else np.float32)
    U = _store_like(np.full((B_u, K_u, D), a), like)
    C = _store_like(np.full((B_c, K_c, D), c), like)
    W_u = _store_like(np.full((M, K_u), wu), like)
    W_c = _store_like(np.full((M, K_c), wc), like)
    Y = f(U, C, np.array([0, 1, 1], np.int32), W_u, W_c)
    assert np.array_equal(Y, np.full((B_c, M, D), K_u * wu * a + K_c * wc * c)), "constant closed form"
    # bf16 widening: 1.0078125 = 1 + 2^-7 is a bf16 value; 3 * 1.0078125 = 3.0234375.
    U = _store_like(np.full((B_u, 1, 1), 1.0078125), like)
    C = _store_like(np.zeros((B_c, 1, 1)), like)
    W1 = _store_like(np.full((1, 1), 3.0), like)
    Y = f(U, C, np.array([0, 0, 1], np.int32), W1, _store_like(np.zeros((1, 1)), like))
    assert np.array_equal(Y, np.full((B_c, 1, 1), 3.0234375)), "exact widening of stored values"


ALL_PINS = [
    ("orientation", pin_orientation),
    ("library", pin_library_special_cases),
    ("decomposed", pin_decomposed_equals_materialised),
    ("padding", pin_zero_padding),
    ("linearity", pin_linearity),
    ("permutations", pin_permutations),
    ("tag", pin_tag),
    ("closed_form", pin_closed_form_constants),
]


def run_all(f, dtype, with_bruteforce=True):
    """Run every pin; return the names of those that failed."""
    failed = []
    for name, pin in ALL_PINS:
        try:
            pin(f, dtype)
        except AssertionError:
            failed.append(name)
    if with_bruteforce:
        try:
            pin_bruteforce(f, np.random.default_rng(3), dtype)
        except AssertionError:
            failed.append("bruteforce")
    return failed
