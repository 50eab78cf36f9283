"""CPU oracle for the IKBO Linear Compression Embedding forward and its backward, and for
IKBO target attention.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product package never imports this
module, and this module imports nothing from the product package.

The arithmetic lives in ``ikbo_oracle.c`` (plain C, fp64): it materialises the
broadcast ``X_b = [U[map[b]] ; C[b]]`` and computes ``Y[b] = [W_u | W_c] . X_b``
(IKBO recsys blog, "Deep Dive: Linear Compression": the baseline batched matmul
and the stage-1 decomposition it equals by linearity).  The backward is the
adjoint of that same materialised product, step by step: ``dX_b = W^T dY[b]``,
whose user rows are scattered back onto ``dU[map[b]]`` (the replication's adjoint)
and whose candidate rows are ``dC[b]``, and ``dW = sum_b dY[b] X_b^T``.  The pages
give no training formulas; this is the plain chain rule of the forward they define.
This wrapper only marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ikbo_oracle.c")
_LIB = os.path.join(_HERE, "libikbo_oracle.so")

ORACLE_BF16 = 0
ORACLE_F32 = 1


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc (always recompiles)."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
           "-std=c11", "-Wall", "-Wextra", "-o", _LIB + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.ikbo_oracle_lce_f64.restype = ctypes.c_int
        lib.ikbo_oracle_lce_f64.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int]
        lib.ikbo_oracle_lce_backward_f64.restype = ctypes.c_int
        lib.ikbo_oracle_lce_backward_f64.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int64] * 6 + [
            ctypes.c_int] + [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p] * 3 + [ctypes.c_int]
        lib.ikbo_oracle_fa_f64.restype = ctypes.c_int
        lib.ikbo_oracle_fa_f64.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64] * 6 + [
            ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int]
        lib.ikbo_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().ikbo_oracle_max_threads())


class OracleError(RuntimeError):
    pass


def lce_f64(U: np.ndarray, C: np.ndarray, mp: np.ndarray, W_u: np.ndarray, W_c: np.ndarray,
            rows: Optional[Sequence[int]] = None, threads: int = 0) -> np.ndarray:
    """Y[b] = W_u . U[map[b]] + W_c . C[b] in fp64, via the materialised form.

    Floating inputs are either all ``uint16`` bfloat16 bit patterns or all
    ``float32``.  ``rows`` selects candidates (default: all); the result has
    shape [len(rows), M, D] (or [B_c, M, D]).
    """
    dt = U.dtype
    if not all(a.dtype == dt for a in (C, W_u, W_c)):
        raise TypeError("U, C, W_u, W_c must share one dtype")
    if dt == np.uint16:
        code = ORACLE_BF16
    elif dt == np.float32:
        code = ORACLE_F32
    else:
        raise TypeError(f"unsupported dtype {dt}")
    B_u, K_u, D = U.shape
    B_c, K_c, D2 = C.shape
    M, K_u2 = W_u.shape
    M2, K_c2 = W_c.shape
    if (D, K_u, K_c, M) != (D2, K_u2, K_c2, M2) or mp.shape != (B_c,):
        raise ValueError("inconsistent shapes")
    U = np.ascontiguousarray(U)
    C = np.ascontiguousarray(C)
    W_u = np.ascontiguousarray(W_u)
    W_c = np.ascontiguousarray(W_c)
    mp = np.ascontiguousarray(mp, dtype=np.int32)
    if rows is None:
        n = B_c
        rows_arr = None
        rows_ptr = None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = rows_arr.shape[0]
        rows_ptr = rows_arr.ctypes.data
    Y = np.empty((n, M, D), dtype=np.float64)
    st = _load().ikbo_oracle_lce_f64(
        U.ctypes.data, C.ctypes.data, mp.ctypes.data, W_u.ctypes.data, W_c.ctypes.data,
        Y.ctypes.data, B_u, B_c, K_u, K_c, M, D, code, rows_ptr, n, int(threads))
    if st != 0:
        raise OracleError(f"oracle returned {st}")
    return Y


def _check_backward_args(dY, U, C, mp, W_u, W_c):
    dt = U.dtype
    if not all(a.dtype == dt for a in (dY, C, W_u, W_c)):
        raise TypeError("dY, U, C, W_u, W_c must share one dtype")
    if dt == np.uint16:
        code = ORACLE_BF16
    elif dt == np.float32:
        code = ORACLE_F32
    else:
        raise TypeError(f"unsupported dtype {dt}")
    B_u, K_u, D = U.shape
    B_c, K_c, D2 = C.shape
    M, K_u2 = W_u.shape
    M2, K_c2 = W_c.shape
    if (D, K_u, K_c, M) != (D2, K_u2, K_c2, M2) or mp.shape != (B_c,) or dY.shape != (B_c, M, D):
        raise ValueError("inconsistent shapes")
    return code, (B_u, B_c, K_u, K_c, M, D)


def _pairs(x) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(x, dtype=np.int64).reshape(-1, 2))
    return a


def lce_backward_rows_f64(dY: np.ndarray, U: np.ndarray, C: np.ndarray, mp: np.ndarray, W_u: np.ndarray,
                          W_c: np.ndarray, dc_rows=(), du_rows=(), dw_elems=(), threads: int = 0):
    """Sampled gradients of L = <dY, Y> for Y = LCE(U, C, map, W_u, W_c), in fp64.

    dc_rows: (b, k) pairs -> dC[b, k, :]; du_rows: (u, k) pairs -> dU[u, k, :];
    dw_elems: (m, kk) pairs -> dW_u[m, kk] for kk < K_u, else dW_c[m, kk - K_u].
    Returns (dC_rows [n, D], dU_rows [n, D], dW [n]).  dY and the floating inputs share
    one storage dtype (``uint16`` bf16 bit patterns or ``float32``)."""
    code, (B_u, B_c, K_u, K_c, M, D) = _check_backward_args(dY, U, C, mp, W_u, W_c)
    dY, U, C, W_u, W_c = (np.ascontiguousarray(a) for a in (dY, U, C, W_u, W_c))
    mp = np.ascontiguousarray(mp, dtype=np.int32)
    pc, pu, pw = _pairs(dc_rows), _pairs(du_rows), _pairs(dw_elems)
    oc, ou, ow = np.empty((len(pc), D)), np.empty((len(pu), D)), np.empty(len(pw))
    st = _load().ikbo_oracle_lce_backward_f64(
        dY.ctypes.data, U.ctypes.data, C.ctypes.data, mp.ctypes.data, W_u.ctypes.data, W_c.ctypes.data,
        B_u, B_c, K_u, K_c, M, D, code,
        pc.ctypes.data, len(pc), oc.ctypes.data, pu.ctypes.data, len(pu), ou.ctypes.data,
        pw.ctypes.data, len(pw), ow.ctypes.data, int(threads))
    if st != 0:
        raise OracleError(f"oracle returned {st}")
    return oc, ou, ow


def lce_backward_f64(dY: np.ndarray, U: np.ndarray, C: np.ndarray, mp: np.ndarray, W_u: np.ndarray,
                     W_c: np.ndarray, threads: int = 0):
    """All gradients: (dU [B_u, K_u, D], dC [B_c, K_c, D], dW_u [M, K_u], dW_c [M, K_c]).

    Users that no candidate maps to get dU = 0."""
    _, (B_u, B_c, K_u, K_c, M, D) = _check_backward_args(dY, U, C, mp, W_u, W_c)
    grid = lambda a, b: np.stack(np.meshgrid(np.arange(a), np.arange(b), indexing="ij"), -1).reshape(-1, 2)
    oc, ou, ow = lce_backward_rows_f64(dY, U, C, mp, W_u, W_c, grid(B_c, K_c), grid(B_u, K_u),
                                       grid(M, K_u + K_c), threads)
    dW = ow.reshape(M, K_u + K_c)
    return (ou.reshape(B_u, K_u, D), oc.reshape(B_c, K_c, D), np.ascontiguousarray(dW[:, :K_u]),
            np.ascontiguousarray(dW[:, K_u:]))


def fa_f64(Q: np.ndarray, K: np.ndarray, V: np.ndarray, mp: np.ndarray, rows=None,
           scale: Optional[float] = None, threads: int = 0) -> np.ndarray:
    """IKBO target attention in fp64: O[b,h,q] = softmax(scale * Q[b,h,q] . K[map[b],h]^T) V[map[b],h].

    Q [B_c, H, L_q, hd]; K, V [B_u, H, L_kv, hd]; all ``uint16`` bf16 bit patterns or all
    ``float32``.  ``scale`` defaults to 1/sqrt(hd).  ``rows``: (b, h, q) triples (default:
    every row); the result is [n, hd] for a list, else [B_c, H, L_q, hd]."""
    dt = Q.dtype
    if not all(a.dtype == dt for a in (K, V)):
        raise TypeError("Q, K, V must share one dtype")
    code = ORACLE_BF16 if dt == np.uint16 else ORACLE_F32 if dt == np.float32 else None
    if code is None:
        raise TypeError(f"unsupported dtype {dt}")
    B_c, H, L_q, hd = Q.shape
    B_u, H2, L_kv, hd2 = K.shape
    if K.shape != V.shape or (H, hd) != (H2, hd2) or mp.shape != (B_c,):
        raise ValueError("inconsistent shapes")
    if scale is None:
        scale = 1.0 / float(np.sqrt(hd))
    Q, K, V = (np.ascontiguousarray(a) for a in (Q, K, V))
    mp = np.ascontiguousarray(mp, dtype=np.int32)
    full = rows is None
    if full:
        rows = np.stack(np.meshgrid(np.arange(B_c), np.arange(H), np.arange(L_q), indexing="ij"), -1).reshape(-1, 3)
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
    O = np.empty((len(r), hd))
    st = _load().ikbo_oracle_fa_f64(Q.ctypes.data, K.ctypes.data, V.ctypes.data, mp.ctypes.data, B_u, B_c, H, L_q,
                                    L_kv, hd, float(scale), code, r.ctypes.data, len(r), O.ctypes.data, int(threads))
    if st != 0:
        raise OracleError(f"oracle returned {st}")
    return O.reshape(B_c, H, L_q, hd) if full else O


def fa_weight_bound(Q: np.ndarray, K: np.ndarray, V: np.ndarray, mp: np.ndarray, rows=None) -> np.ndarray:
    """2^-8 * sum_k w_k |V_k| per output element (w: the softmax weights), from the oracle's
    attention applied to |V|: twice the bound on what bf16 rounding of the weights (each off by
    at most 2^-9 of itself) can move an attention output."""
    Vabs = (V & np.uint16(0x7FFF)) if V.dtype == np.uint16 else np.abs(V)
    return fa_f64(Q, K, Vabs, mp, rows=rows) * 2.0 ** -8


def tolerance_violations(Y_gpu: np.ndarray, Y_ref: np.ndarray, atol: float = 1e-3,
                         rtol: float = 1.6e-2, extra=None):
    """Count elements outside the parity bar and return (count, max_excess).

    A finite reference value r admits y when |y - r| <= atol + rtol*|r| (+ extra, elementwise,
    when given): bf16 inputs and fp32 accumulation, the acceptance bound of the IKBO LCE parity
    contract.  Special values must match exactly: an infinite reference admits only the same
    infinity, a NaN reference only a NaN, and a NaN or infinite y only the same reference value.
    A non-finite bound (an infinite or NaN ``extra``) admits nothing but exact equality.  The
    excess of a special-value mismatch is reported as infinity."""
    Y_gpu = np.asarray(Y_gpu, dtype=np.float64)
    Y_ref = np.asarray(Y_ref, dtype=np.float64)
    if Y_gpu.shape != Y_ref.shape:
        raise ValueError(f"shape mismatch: {Y_gpu.shape} against {Y_ref.shape}")
    fin = np.isfinite(Y_gpu) & np.isfinite(Y_ref)
    with np.errstate(invalid="ignore", over="ignore"):
        err = np.abs(Y_gpu - Y_ref)
        bound = atol + rtol * np.abs(Y_ref)
        if extra is not None:
            bound = bound + np.asarray(extra, dtype=np.float64)
    fin_ok = fin & np.isfinite(bound) & (err <= bound)
    special_ok = ~fin & ((np.isnan(Y_gpu) & np.isnan(Y_ref)) | (Y_gpu == Y_ref))
    exact_ok = fin & ~np.isfinite(bound) & (Y_gpu == Y_ref)
    bad = ~(fin_ok | special_ok | exact_ok)
    with np.errstate(invalid="ignore"):
        excess = np.where(bad, np.where(fin & np.isfinite(bound), err - bound, np.inf), 0.0)
    ex = float(excess.max()) if excess.size else 0.0
    return int(bad.sum()), ex
