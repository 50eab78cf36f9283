"""Pins for the oracle's backward: facts it cannot supply itself.

Each ``pin_*`` takes ``g(dY, U, C, map, W_u, W_c) -> (dU, dC, dW_u, dW_c)`` (numpy in,
float64 out) and raises AssertionError when ``g`` disagrees with the fact it pins.

The backward is the gradient of L = <dY, Y> with Y the LCE forward (IKBO recsys blog,
"Deep Dive: Linear Compression": Y[b] = W_u . U[map[b]] + W_c . C[b]).  The pages give
no training formulas, so the facts come from the definition of a gradient and plain
linear algebra:
  * exact gradient: L is linear in (U, C) and, separately, in (W_u, W_c), so setting
    one input element x_i to zero lowers L by exactly x_i * dL/dx_i; with bf16/fp32
    numbers as exact rationals this is brute force in ``Fraction``;
  * adjoint identities: <dY, Y(U', C')> = <dU, U'> + <dC, C'> for every U', C' and
    <dY, Y_{W'}> = <dW_u, W_u'> + <dW_c, W_c'> for every W' (exact on integer data);
  * closed forms: a one-hot dY at (b0, m0, d0) gives dC[b0, :, d0] = W_c[m0, :],
    dU[map[b0], :, d0] = W_u[m0, :], dW_c[m0, :] = C[b0, :, d0], dW_u[m0, :] =
    U[map[b0], :, d0] and zeros elsewhere;
  * library special case: the identity map reduces every gradient to numpy matmuls;
  * users that no candidate maps to get dU = 0 exactly; candidates of one user add.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

import pins
from pins import _f, rand_case


def _draw_dy(rng, dtype, B_c, M, D, ints=False):
    x = rng.integers(-3, 4, size=(B_c, M, D)).astype(np.float32) if ints else \
        rng.standard_normal((B_c, M, D)).astype(np.float32)
    return pins._store_like(x, np.zeros(1, np.uint16) if dtype == "bf16" else np.zeros(1, np.float32))


def _forward_np(U, C, mp, W_u, W_c):
    """Y in fp64 from exact float views (decomposed form, numpy matmul)."""
    Uf, Cf, Wuf, Wcf = (_f(a) for a in (U, C, W_u, W_c))
    return np.matmul(Wuf, Uf)[mp] + np.matmul(Wcf, Cf)


def _exact_loss(dY, U, C, mp, W_u, W_c):
    """L = <dY, Y> as an exact Fraction."""
    Y, _ = pins.fraction_bruteforce(U, C, mp, W_u, W_c)
    dYf = _f(dY)
    tot = Fraction(0)
    for idx in np.ndindex(Y.shape):
        tot += Fraction(float(dYf[idx])) * Y[idx]
    return tot


def pin_bwd_bruteforce(g, rng, dtype):
    """Every gradient element equals (L(x) - L(x with x_i = 0)) / x_i in exact arithmetic."""
    B_u, B_c, K_u, K_c, M, D = 3, 4, 2, 3, 2, 2
    U, C, mp, W_u, W_c = rand_case(rng, dtype, B_u, B_c, K_u, K_c, M, D)
    mp[:] = [2, 0, 2, 2]                      # user 1 has no candidate; user 2 has three
    dY = _draw_dy(rng, dtype, B_c, M, D)
    got = g(dY, U, C, mp, W_u, W_c)
    base = _exact_loss(dY, U, C, mp, W_u, W_c)
    names = ("dU", "dC", "dW_u", "dW_c")
    for k, (arr, out) in enumerate(zip((U, C, W_u, W_c), got)):
        assert out.shape == arr.shape, f"{names[k]} shape {out.shape} != {arr.shape}"
        for idx in np.ndindex(arr.shape):
            x_i = Fraction(float(_f(arr)[idx]))
            assert x_i != 0
            # L is linear along e_i, so zeroing x_i removes exactly x_i * dL/dx_i.
            a = arr.copy()
            a[idx] = 0
            args = [U, C, W_u, W_c]
            args[k] = a
            exact = (base - _exact_loss(dY, args[0], args[1], mp, args[2], args[3])) / x_i
            assert abs(Fraction(float(out[idx])) - exact) <= Fraction(1, 10 ** 9) * (1 + abs(exact)), (
                f"{names[k]}{idx}: {float(out[idx])} vs exact {float(exact)}")


def pin_bwd_adjoint(g, dtype):
    """<dY, Y(U', C')> = <dU, U'> + <dC, C'> and the same in the weights, exactly."""
    rng = np.random.default_rng(21)
    B_u, B_c, K_u, K_c, M, D = 4, 13, 9, 7, 5, 8
    U, C, mp, W_u, W_c = rand_case(rng, dtype, B_u, B_c, K_u, K_c, M, D, ints=True)
    dY = _draw_dy(rng, dtype, B_c, M, D, ints=True)
    dU, dC, dW_u, dW_c = g(dY, U, C, mp, W_u, W_c)
    dYf = _f(dY)
    for t in range(3):
        U2, C2, _, W_u2, W_c2 = rand_case(np.random.default_rng(100 + t), dtype, B_u, B_c, K_u, K_c, M, D,
                                          ints=True)
        lhs = float(np.sum(dYf * _forward_np(U2, C2, mp, W_u, W_c)))
        rhs = float(np.sum(dU * _f(U2)) + np.sum(dC * _f(C2)))
        assert lhs == rhs, f"input adjoint: {lhs} != {rhs}"
        lhs = float(np.sum(dYf * _forward_np(U, C, mp, W_u2, W_c2)))
        rhs = float(np.sum(dW_u * _f(W_u2)) + np.sum(dW_c * _f(W_c2)))
        assert lhs == rhs, f"weight adjoint: {lhs} != {rhs}"


def pin_bwd_one_hot(g, dtype):
    """A one-hot upstream gradient selects one row or column of each operand."""
    rng = np.random.default_rng(22)
    B_u, B_c, K_u, K_c, M, D = 3, 6, 5, 4, 3, 4
    U, C, mp, W_u, W_c = rand_case(rng, dtype, B_u, B_c, K_u, K_c, M, D)
    b0, m0, d0 = 4, 2, 1
    dY = pins._store_like(np.zeros((B_c, M, D), np.float32), U)
    dY[b0, m0, d0] = pins._store_like(np.ones(1, np.float32), U)[0]
    dU, dC, dW_u, dW_c = g(dY, U, C, mp, W_u, W_c)
    e_dC = np.zeros_like(dC); e_dC[b0, :, d0] = _f(W_c)[m0]
    e_dU = np.zeros_like(dU); e_dU[mp[b0], :, d0] = _f(W_u)[m0]
    e_dWc = np.zeros_like(dW_c); e_dWc[m0] = _f(C)[b0, :, d0]
    e_dWu = np.zeros_like(dW_u); e_dWu[m0] = _f(U)[mp[b0], :, d0]
    for name, got, exp in (("dC", dC, e_dC), ("dU", dU, e_dU), ("dW_c", dW_c, e_dWc), ("dW_u", dW_u, e_dWu)):
        assert np.array_equal(got, exp), f"{name} differs from the one-hot closed form"


def pin_bwd_identity_map(g, dtype):
    """map = arange(B_c) (one candidate per user): every gradient is a numpy matmul."""
    rng = np.random.default_rng(23)
    B, K_u, K_c, M, D = 5, 6, 7, 4, 8
    U, C, _, W_u, W_c = rand_case(rng, dtype, B, B, K_u, K_c, M, D)
    mp = np.arange(B, dtype=np.int32)
    dY = _draw_dy(rng, dtype, B, M, D)
    dU, dC, dW_u, dW_c = g(dY, U, C, mp, W_u, W_c)
    dYf, Uf, Cf, Wuf, Wcf = (_f(a) for a in (dY, U, C, W_u, W_c))
    np.testing.assert_allclose(dU, np.matmul(Wuf.T, dYf), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dC, np.matmul(Wcf.T, dYf), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dW_u, np.matmul(dYf, Uf.transpose(0, 2, 1)).sum(0), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dW_c, np.matmul(dYf, Cf.transpose(0, 2, 1)).sum(0), rtol=1e-12, atol=1e-12)


def pin_bwd_segments(g, dtype):
    """Unmapped users get exactly zero; duplicating a candidate doubles its user's share."""
    rng = np.random.default_rng(24)
    B_u, B_c, K_u, K_c, M, D = 5, 6, 4, 3, 3, 8
    U, C, mp, W_u, W_c = rand_case(rng, dtype, B_u, B_c, K_u, K_c, M, D, ints=True)
    mp[:] = [3, 3, 0, 3, 0, 0]                # users 1, 2 and 4 have no candidate
    dY = _draw_dy(rng, dtype, B_c, M, D, ints=True)
    dU, dC, dW_u, dW_c = g(dY, U, C, mp, W_u, W_c)
    for u in (1, 2, 4):
        assert np.all(dU[u] == 0.0), f"user {u} has no candidate but dU != 0"
    # Two copies of candidate 0 (same C row, same user, same dY row): dC rows repeat and
    # user 3's gradient gains that candidate's share once more.
    sel = np.array([0, 0, 1, 2, 3, 4, 5])
    dU2, dC2, dW_u2, dW_c2 = g(np.ascontiguousarray(dY[sel]), U, np.ascontiguousarray(C[sel]),
                               np.ascontiguousarray(mp[sel]), W_u, W_c)
    assert np.array_equal(dC2, dC[sel])
    one = g(np.ascontiguousarray(dY[:1]), U, np.ascontiguousarray(C[:1]), np.ascontiguousarray(mp[:1]), W_u, W_c)
    assert np.array_equal(dU2, dU + one[0])
    assert np.array_equal(dW_u2, dW_u + one[2]) and np.array_equal(dW_c2, dW_c + one[3])


ALL_PINS = [
    ("adjoint", pin_bwd_adjoint),
    ("one_hot", pin_bwd_one_hot),
    ("identity_map", pin_bwd_identity_map),
    ("segments", pin_bwd_segments),
]


def run_all(g, dtype, with_bruteforce=True):
    """Names of the pins g fails (empty list: g passes them all)."""
    failed = []
    for name, pin in ALL_PINS:
        try:
            pin(g, dtype)
        except AssertionError:
            failed.append(name)
    if with_bruteforce:
        try:
            pin_bwd_bruteforce(g, np.random.default_rng(5), dtype)
        except AssertionError:
            failed.append("bruteforce")
    return failed
