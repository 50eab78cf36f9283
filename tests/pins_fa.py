"""Pins for the oracle's IKBO target attention: facts it cannot supply itself.

Each ``pin_*`` takes ``f(Q, K, V, map, scale=None) -> O`` (numpy in, float64 out) and
raises AssertionError when ``f`` disagrees with the fact it pins.  The operation (IKBO
recsys blog, "Deep Dive: Flash Attention"): the queries of candidate b attend over the
keys and values of its user map[b], O = softmax(scale * Q K^T) V per head.  Facts:
  * softmax weights sum to one: V rows all equal to c give O = c; K = 0 gives equal
    weights, so O is the mean of the V rows; with V[u] = u + 1 everywhere that is a
    gather tag, O[b] = map[b] + 1;
  * two keys: O = sigma(s0 - s1) V0 + sigma(s1 - s0) V1, with the scores computed exactly
    (``Fraction``) and the logistic function from ``math``;
  * a key whose score exceeds every other by 60 takes all the weight up to e^-60;
  * O is a convex combination of the V rows (inside their columnwise range);
  * permuting keys (K and V rows together) leaves O unchanged; permuting candidates
    permutes O; relabelling users changes nothing; doubling Q equals doubling the scale.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

from pins import _f, _store_like


def _draw(rng, dtype, shape, ints=False, scale=1.0):
    x = (rng.integers(-2, 3, size=shape) if ints else rng.standard_normal(shape) * scale).astype(np.float32)
    return _store_like(x, np.zeros(1, np.uint16) if dtype == "bf16" else np.zeros(1, np.float32))


def case(rng, dtype, B_u=3, B_c=7, H=2, L_q=3, L_kv=5, hd=8):
    Q = _draw(rng, dtype, (B_c, H, L_q, hd))
    K = _draw(rng, dtype, (B_u, H, L_kv, hd))
    V = _draw(rng, dtype, (B_u, H, L_kv, hd))
    mp = rng.integers(0, B_u, B_c).astype(np.int32)
    return Q, K, V, mp


def pin_weights_sum_to_one(f, dtype):
    rng = np.random.default_rng(31)
    Q, K, V, mp = case(rng, dtype)
    c = _draw(rng, dtype, (3, 2, 1, 8))
    Vc = np.ascontiguousarray(np.broadcast_to(c, V.shape))
    O = f(Q, K, Vc, mp)
    exp = np.broadcast_to(_f(c)[mp], O.shape)
    assert np.allclose(O, exp, rtol=1e-13, atol=1e-13), "V rows equal to c must give O = c"
    Kz = np.zeros_like(K)
    O = f(Q, Kz, V, mp)
    mean = _f(V).mean(axis=2, keepdims=True)[mp]
    assert np.allclose(O, np.broadcast_to(mean, O.shape), rtol=1e-13, atol=1e-13), "K = 0 must average V"


def pin_gather_tag(f, dtype):
    rng = np.random.default_rng(32)
    Q, K, V, mp = case(rng, dtype, B_u=5, B_c=11)
    tag = (np.arange(5, dtype=np.float32) + 1.0)[:, None, None, None]
    Vt = _store_like(np.broadcast_to(tag, V.shape).copy(), V)
    O = f(Q, np.zeros_like(K), Vt, mp)
    assert np.array_equal(O, np.broadcast_to((mp + 1.0)[:, None, None, None], O.shape)), "gather tag"


def pin_two_keys(f, dtype):
    rng = np.random.default_rng(33)
    Q, K, V, mp = case(rng, dtype, L_kv=2, hd=4)
    O = f(Q, K, V, mp, scale=0.5)
    Qf, Kf, Vf = _f(Q), _f(K), _f(V)
    for b in range(Q.shape[0]):
        u = mp[b]
        for h in range(Q.shape[1]):
            for q in range(Q.shape[2]):
                s = [Fraction(1, 2) * sum(Fraction(float(Qf[b, h, q, d])) * Fraction(float(Kf[u, h, k, d]))
                                          for d in range(Q.shape[3])) for k in range(2)]
                w0 = 1.0 / (1.0 + math.exp(float(s[1] - s[0])))
                exp = w0 * Vf[u, h, 0] + (1.0 - w0) * Vf[u, h, 1]
                assert np.allclose(O[b, h, q], exp, rtol=1e-12, atol=1e-12), f"two keys at {(b, h, q)}"


def pin_dominant_key(f, dtype):
    rng = np.random.default_rng(34)
    Q, K, V, mp = case(rng, dtype, L_kv=6, hd=4)
    Q = np.zeros_like(Q)
    K = np.zeros_like(K)
    one = _store_like(np.ones(1, np.float32), Q)[0]
    Q[..., 0] = one
    big = _store_like(np.full(1, 60.0, np.float32), K)[0]
    K[:, :, 4, 0] = big                      # key 4 scores 60, the others 0
    O = f(Q, K, V, mp, scale=1.0)
    exp = np.broadcast_to(_f(V)[mp][:, :, 4:5, :], O.shape)
    assert np.allclose(O, exp, rtol=0, atol=1e-24 + 12 * math.exp(-60) * np.abs(_f(V)).max()), "dominant key"


def pin_convex(f, dtype):
    rng = np.random.default_rng(35)
    Q, K, V, mp = case(rng, dtype, L_kv=9)
    O = f(Q, K, V, mp)
    Vf = _f(V)[mp]
    lo, hi = Vf.min(axis=2, keepdims=True), Vf.max(axis=2, keepdims=True)
    assert np.all(O >= lo - 1e-13) and np.all(O <= hi + 1e-13), "O outside the range of the V rows"
    assert np.any(O > lo + 1e-3), "O sits on the minimum everywhere"


def pin_permutations(f, dtype):
    rng = np.random.default_rng(36)
    Q, K, V, mp = case(rng, dtype, B_u=4, B_c=9, L_kv=7)
    O = f(Q, K, V, mp)
    pk = rng.permutation(7)
    O2 = f(Q, np.ascontiguousarray(K[:, :, pk]), np.ascontiguousarray(V[:, :, pk]), mp)
    assert np.allclose(O2, O, rtol=1e-13, atol=1e-13), "key permutation"
    pc = rng.permutation(9)
    O3 = f(np.ascontiguousarray(Q[pc]), K, V, np.ascontiguousarray(mp[pc]))
    assert np.array_equal(O3, O[pc]), "candidate permutation"
    sig = rng.permutation(4)
    inv = np.argsort(sig)
    O4 = f(Q, np.ascontiguousarray(K[inv]), np.ascontiguousarray(V[inv]), sig[mp].astype(np.int32))
    assert np.array_equal(O4, O), "user relabelling"


def pin_scale(f, dtype):
    rng = np.random.default_rng(37)
    Q, K, V, mp = case(rng, dtype)
    Q2 = _store_like(2.0 * _f(Q), Q)
    assert np.array_equal(f(Q2, K, V, mp, scale=0.25), f(Q, K, V, mp, scale=0.5)), "doubling Q vs scale"
    hd = Q.shape[-1]
    assert np.array_equal(f(Q, K, V, mp), f(Q, K, V, mp, scale=1.0 / math.sqrt(hd))), "default scale"


ALL_PINS = [
    ("weights_sum_to_one", pin_weights_sum_to_one),
    ("gather_tag", pin_gather_tag),
    ("two_keys", pin_two_keys),
    ("dominant_key", pin_dominant_key),
    ("convex", pin_convex),
    ("permutations", pin_permutations),
    ("scale", pin_scale),
]


def run_all(f, dtype):
    failed = []
    for name, pin in ALL_PINS:
        try:
            pin(f, dtype)
        except AssertionError:
            failed.append(name)
    return failed
