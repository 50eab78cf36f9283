"""broadcast_gemm_amd -- IKBO Linear Compression Embedding forward (and backward) for AMD MI355X.

    Y[b] = W_u . U[map[b]] + W_c . C[b]

Python binding of the C ABI in ``include/ikbo.h`` (``libikbo.so``).  This layer
only marshals arguments: every step of the forward runs in the library's HIP
kernels.  PyTorch supplies device memory and streams.  There is no CPU path:
if the library is not built, every call raises.

    plan = LcePlan(max_B_u, max_B_c, K_u, K_c, M, D, dtype="bf16", variant="S4")
    Y = plan.forward(U, C, map, W_u, W_c)        # torch tensors on the GPU

    plan = LcePlan(..., flags=FLAG_BACKWARD)     # the backward's workspace as well
    dU, dC, dW_u, dW_c = plan.backward(dY, U, C, map, W_u, W_c)

    from broadcast_gemm_amd.autograd import IkboLce   # training: autograd over both calls
    Y = IkboLce(K_u, K_c, M, D).cuda()(U, C, map); Y.backward(dY)

    fa = FaPlan(max_B_u, max_B_c, H, L_q, L_kv, head_dim)   # IKBO target attention
    O = fa.forward(Q, K, V, map)
"""
from __future__ import annotations

import ctypes
import json
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libikbo.so")

IKBO_OK = 0
IKBO_ERR_INVALID_ARG = -1
IKBO_ERR_UNSUPPORTED = -2
IKBO_ERR_HIP = -3
IKBO_ERR_ALIGNMENT = -4
IKBO_ERR_TIMEOUT = -5
IKBO_ERR_MAP_RANGE = -6

DTYPES = {"bf16": 0, "f32": 1}
VARIANTS = {"auto": 0, "S0": 1, "S1": 2, "S2": 3, "S3": 4, "S4": 5}
FLAG_DEBUG_DELAY_USER = 2
FLAG_DEBUG_SKIP_USER = 4
FLAG_DEBUG_POISON_USER = 16
FLAG_BACKWARD = 8

# Every symbol include/ikbo.h declares.
EXPORTED = ("ikbo_lce_plan", "ikbo_lce_forward", "ikbo_lce_forward_noalloc", "ikbo_lce_backward", "ikbo_lce_check",
            "ikbo_fa_plan", "ikbo_fa_forward", "ikbo_fa_forward_fused", "ikbo_fa_check", "ikbo_fa_plan_destroy", "ikbo_lce_plan_info",
            "ikbo_lce_plan_set_spin_limit", "ikbo_lce_plan_destroy", "ikbo_status_str",
            "ikbo_last_error_message")


class IkboError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        msg = f"{what}: " if what else ""
        msg += f"{status_str(status)} ({status})"
        if status == IKBO_ERR_HIP:
            msg += f": {last_error_message()}"
        super().__init__(msg)


_lib = None


def lib() -> ctypes.CDLL:
    """Load libikbo.so with its prototypes; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m broadcast_gemm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, ip, i, u32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_uint32, ctypes.c_size_t
        L.ikbo_lce_plan.argtypes = [ctypes.POINTER(vp), i, i, i, i, i, i, i, i, ctypes.c_uint]
        L.ikbo_lce_plan.restype = ip
        L.ikbo_lce_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp]
        L.ikbo_lce_forward.restype = ip
        L.ikbo_lce_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp]
        L.ikbo_lce_forward_noalloc.restype = ip
        L.ikbo_lce_backward.argtypes = [vp] + [vp] * 10 + [i] * 6 + [vp]
        L.ikbo_lce_backward.restype = ip
        L.ikbo_fa_plan.argtypes = [ctypes.POINTER(vp), i, i, i, i, i, i, i, ctypes.c_uint]
        L.ikbo_fa_plan.restype = ip
        L.ikbo_fa_forward.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, ctypes.c_float, vp]
        L.ikbo_fa_forward.restype = ip
        L.ikbo_fa_forward_fused.argtypes = [vp] * 8 + [i] * 7 + [ctypes.c_float, vp]
        L.ikbo_fa_forward_fused.restype = ip
        L.ikbo_fa_check.argtypes = [vp, vp]
        L.ikbo_fa_check.restype = ip
        L.ikbo_fa_plan_destroy.argtypes = [vp]
        L.ikbo_fa_plan_destroy.restype = ip
        L.ikbo_lce_check.argtypes = [vp, vp]
        L.ikbo_lce_check.restype = ip
        L.ikbo_lce_plan_info.argtypes = [vp, ctypes.c_char_p, sz]
        L.ikbo_lce_plan_info.restype = ip
        L.ikbo_lce_plan_set_spin_limit.argtypes = [vp, u32]
        L.ikbo_lce_plan_set_spin_limit.restype = ip
        L.ikbo_lce_plan_destroy.argtypes = [vp]
        L.ikbo_lce_plan_destroy.restype = ip
        L.ikbo_status_str.argtypes = [ip]
        L.ikbo_status_str.restype = ctypes.c_char_p
        L.ikbo_last_error_message.argtypes = []
        L.ikbo_last_error_message.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().ikbo_status_str(int(status)).decode()


def last_error_message() -> str:
    return lib().ikbo_last_error_message().decode()


def _torch():
    import torch
    return torch


def _stream_handle(stream) -> Optional[int]:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def forward_noalloc_ptrs(U: int, C: int, mp: int, W_u: int, W_c: int, Y: int, B_u: int, B_c: int,
                         K_u: int, K_c: int, M: int, D: int, stream: Optional[int] = None) -> int:
    """Raw ``ikbo_lce_forward_noalloc`` call on device pointers; returns the status code."""
    return lib().ikbo_lce_forward_noalloc(U, C, mp, W_u, W_c, Y, B_u, B_c, K_u, K_c, M, D, stream)


def forward_noalloc(U, C, mp, W_u, W_c, out, stream=None):
    """Y = W_u . U[map] + W_c . C into ``out`` without a plan and without allocating device
    memory (``ikbo_lce_forward_noalloc``; bf16 tensors on the GPU).  Returns ``out``."""
    torch = _torch()
    for name, t in (("U", U), ("C", C), ("W_u", W_u), ("W_c", W_c), ("out", out)):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bfloat16 tensor on the GPU")
    if mp.dtype != torch.int32 or not mp.is_contiguous():
        raise ValueError("map must be a contiguous int32 tensor")
    B_u, K_u, D = U.shape
    B_c, K_c = C.shape[0], C.shape[1]
    M = W_u.shape[0]
    if tuple(C.shape) != (B_c, K_c, D) or tuple(W_c.shape) != (M, K_c) or tuple(W_u.shape) != (M, K_u) \
            or tuple(out.shape) != (B_c, M, D) or tuple(mp.shape) != (B_c,):
        raise IkboError(IKBO_ERR_INVALID_ARG, "inconsistent shapes")
    st = forward_noalloc_ptrs(U.data_ptr(), C.data_ptr(), mp.data_ptr(), W_u.data_ptr(), W_c.data_ptr(),
                              out.data_ptr(), B_u, B_c, K_u, K_c, M, D, _stream_handle(stream))
    if st != IKBO_OK:
        raise IkboError(st, "ikbo_lce_forward_noalloc")
    return out


class LcePlan:
    """A plan for one shape range; owns the device workspace (see ``ikbo_lce_plan``)."""

    def __init__(self, max_B_u: int, max_B_c: int, K_u: int, K_c: int, M: int, D: int,
                 dtype: str = "bf16", variant: str = "auto", flags: int = 0):
        self.dims = (K_u, K_c, M, D)
        self.max_B_u, self.max_B_c = max_B_u, max_B_c
        self.dtype = dtype
        self.variant = variant
        h = ctypes.c_void_p()
        st = lib().ikbo_lce_plan(ctypes.byref(h), max_B_u, max_B_c, K_u, K_c, M, D, DTYPES[dtype],
                                 VARIANTS[variant], flags)
        if st != IKBO_OK:
            raise IkboError(st, "ikbo_lce_plan")
        self._h = h

    @property
    def handle(self) -> ctypes.c_void_p:
        if self._h is None:
            raise ValueError("plan destroyed")
        return self._h

    def info(self) -> dict:
        buf = ctypes.create_string_buffer(2048)
        n = lib().ikbo_lce_plan_info(self.handle, buf, len(buf))
        if n < 0:
            raise IkboError(n, "ikbo_lce_plan_info")
        return json.loads(buf.value.decode())

    def set_spin_limit(self, polls: int) -> None:
        st = lib().ikbo_lce_plan_set_spin_limit(self.handle, polls)
        if st != IKBO_OK:
            raise IkboError(st, "ikbo_lce_plan_set_spin_limit")

    def forward_ptrs(self, U: int, C: int, mp: int, W_u: int, W_c: int, Y: int, B_u: int, B_c: int,
                     stream: Optional[int] = None) -> int:
        """Raw C-ABI call on device pointers; returns the status code."""
        K_u, K_c, M, D = self.dims
        return lib().ikbo_lce_forward(self.handle, U, C, mp, W_u, W_c, Y, B_u, B_c, K_u, K_c, M, D, stream)

    def forward(self, U, C, mp, W_u, W_c, out=None, stream=None):
        """Y = W_u . U[map] + W_c . C on the current (or given) stream; returns Y."""
        torch = _torch()
        tdt = torch.bfloat16 if self.dtype == "bf16" else torch.float32
        for name, t in (("U", U), ("C", C), ("W_u", W_u), ("W_c", W_c)):
            if t.dtype != tdt or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous {tdt} tensor on the GPU")
        if mp.dtype != torch.int32:
            mp = mp.to(torch.int32)
        mp = mp.contiguous()
        B_u, K_u, D = U.shape
        B_c = C.shape[0]
        M = W_u.shape[0]
        if out is None:
            out = torch.empty((B_c, M, D), dtype=tdt, device=C.device)
        elif out.dtype != tdt or not out.is_contiguous() or tuple(out.shape) != (B_c, M, D):
            raise ValueError("out must be a contiguous tensor of shape [B_c, M, D]")
        K_u2, K_c, M2, D2 = self.dims
        if (K_u, C.shape[1], M, D) != (K_u2, K_c, M2, D2) or tuple(W_c.shape) != (M2, K_c) \
                or tuple(C.shape[2:]) != (D2,) or tuple(W_u.shape) != (M2, K_u2) or mp.shape != (B_c,):
            raise IkboError(IKBO_ERR_INVALID_ARG, "shape differs from the plan")
        st = self.forward_ptrs(U.data_ptr(), C.data_ptr(), mp.data_ptr(), W_u.data_ptr(), W_c.data_ptr(),
                               out.data_ptr(), B_u, B_c, _stream_handle(stream))
        if st != IKBO_OK:
            raise IkboError(st, "ikbo_lce_forward")
        return out

    def backward_ptrs(self, dY: int, U: int, C: int, mp: int, W_u: int, W_c: int, dU: int, dC: int,
                      dW_u: int, dW_c: int, B_u: int, B_c: int, stream: Optional[int] = None) -> int:
        """Raw C-ABI call on device pointers; returns the status code."""
        K_u, K_c, M, D = self.dims
        return lib().ikbo_lce_backward(self.handle, dY, U, C, mp, W_u, W_c, dU, dC, dW_u, dW_c,
                                       B_u, B_c, K_u, K_c, M, D, stream)

    def backward(self, dY, U, C, mp, W_u, W_c, out=None, stream=None):
        """Gradients (dU, dC, dW_u, dW_c) of <dY, Y> on the current (or given) stream.

        Needs a plan made with ``flags=FLAG_BACKWARD``.  dU and dC come back in the plan's
        dtype (bf16), dW_u and dW_c in float32.  ``out`` may supply the four tensors."""
        torch = _torch()
        tdt = torch.bfloat16 if self.dtype == "bf16" else torch.float32
        for name, t in (("dY", dY), ("U", U), ("C", C), ("W_u", W_u), ("W_c", W_c)):
            if t.dtype != tdt or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous {tdt} tensor on the GPU")
        if mp.dtype != torch.int32:
            mp = mp.to(torch.int32)
        mp = mp.contiguous()
        K_u, K_c, M, D = self.dims
        B_u, B_c = U.shape[0], C.shape[0]
        if tuple(U.shape) != (B_u, K_u, D) or tuple(C.shape) != (B_c, K_c, D) or tuple(dY.shape) != (B_c, M, D) \
                or tuple(W_u.shape) != (M, K_u) or tuple(W_c.shape) != (M, K_c) or mp.shape != (B_c,):
            raise IkboError(IKBO_ERR_INVALID_ARG, "shape differs from the plan")
        shapes = ((B_u, K_u, D), (B_c, K_c, D), (M, K_u), (M, K_c))
        dts = (tdt, tdt, torch.float32, torch.float32)
        if out is None:
            out = tuple(torch.empty(sh, dtype=dt, device=U.device) for sh, dt in zip(shapes, dts))
        else:
            out = tuple(out)
            for t, sh, dt in zip(out, shapes, dts):
                if t.dtype != dt or not t.is_contiguous() or tuple(t.shape) != sh:
                    raise ValueError("out must be (dU, dC, dW_u, dW_c) contiguous tensors of the gradient shapes")
        dU, dC, dW_u, dW_c = out
        st = self.backward_ptrs(dY.data_ptr(), U.data_ptr(), C.data_ptr(), mp.data_ptr(), W_u.data_ptr(),
                                W_c.data_ptr(), dU.data_ptr(), dC.data_ptr(), dW_u.data_ptr(), dW_c.data_ptr(),
                                B_u, B_c, _stream_handle(stream))
        if st != IKBO_OK:
            raise IkboError(st, "ikbo_lce_backward")
        return out

    def check(self, stream=None) -> int:
        """Synchronise and return (and clear) the device-side status."""
        return lib().ikbo_lce_check(self.handle, _stream_handle(stream))

    def close(self) -> None:
        if getattr(self, "_h", None) is not None:
            st = lib().ikbo_lce_plan_destroy(self._h)
            self._h = None
            if st != IKBO_OK:
                raise IkboError(st, "ikbo_lce_plan_destroy")

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


class FaPlan:
    """A plan for IKBO target attention (see ``ikbo_fa_plan``): the queries of each
    candidate attend over the keys and values of its user, which are never replicated."""

    def __init__(self, max_B_u: int, max_B_c: int, H: int, L_q: int, L_kv: int, head_dim: int,
                 dtype: str = "bf16"):
        self.dims = (H, L_q, L_kv, head_dim)
        self.max_B_u, self.max_B_c = max_B_u, max_B_c
        h = ctypes.c_void_p()
        st = lib().ikbo_fa_plan(ctypes.byref(h), max_B_u, max_B_c, H, L_q, L_kv, head_dim, DTYPES[dtype], 0)
        if st != IKBO_OK:
            raise IkboError(st, "ikbo_fa_plan")
        self._h = h

    @property
    def handle(self) -> ctypes.c_void_p:
        if self._h is None:
            raise ValueError("plan destroyed")
        return self._h

    def forward_ptrs(self, Q: int, K: int, V: int, mp: int, O: int, B_u: int, B_c: int, scale: float = 0.0,
                     stream: Optional[int] = None) -> int:
        """Raw C-ABI call on device pointers; returns the status code."""
        H, L_q, L_kv, hd = self.dims
        return lib().ikbo_fa_forward(self.handle, Q, K, V, mp, O, B_u, B_c, H, L_q, L_kv, hd, float(scale), stream)

    def forward(self, Q, K, V, mp, out=None, scale: float = 0.0, stream=None):
        """O = softmax(scale Q K[map]^T) V[map] per head on the current (or given) stream."""
        torch = _torch()
        for name, t in (("Q", Q), ("K", K), ("V", V)):
            if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous bfloat16 tensor on the GPU")
        if mp.dtype != torch.int32:
            mp = mp.to(torch.int32)
        mp = mp.contiguous()
        H, L_q, L_kv, hd = self.dims
        B_c, B_u = Q.shape[0], K.shape[0]
        if tuple(Q.shape) != (B_c, H, L_q, hd) or tuple(K.shape) != (B_u, H, L_kv, hd) or K.shape != V.shape \
                or mp.shape != (B_c,):
            raise IkboError(IKBO_ERR_INVALID_ARG, "shape differs from the plan")
        if out is None:
            out = torch.empty_like(Q)
        elif out.dtype != torch.bfloat16 or not out.is_contiguous() or out.shape != Q.shape:
            raise ValueError("out must be a contiguous bfloat16 tensor shaped like Q")
        st = self.forward_ptrs(Q.data_ptr(), K.data_ptr(), V.data_ptr(), mp.data_ptr(), out.data_ptr(), B_u, B_c,
                               scale, _stream_handle(stream))
        if st != IKBO_OK:
            raise IkboError(st, "ikbo_fa_forward")
        return out

    def forward_fused_ptrs(self, Q: int, K: int, V: int, mp: int, O: int, Q_self: int, O_self: int, B_u: int,
                           B_c: int, L_self: int, scale: float = 0.0, stream: Optional[int] = None) -> int:
        H, L_q, L_kv, hd = self.dims
        return lib().ikbo_fa_forward_fused(self.handle, Q, K, V, mp, O, Q_self, O_self, B_u, B_c, H, L_q, L_kv,
                                           L_self, hd, float(scale), stream)

    def forward_fused(self, Q, K, V, mp, Q_self, out=None, out_self=None, scale: float = 0.0, stream=None):
        """Target attention of the candidates and self-attention of the users' own queries
        Q_self [B_u, H, L_self, hd] over the same K/V, in one launch; returns (O, O_self)."""
        torch = _torch()
        for name, t in (("Q", Q), ("K", K), ("V", V), ("Q_self", Q_self)):
            if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous bfloat16 tensor on the GPU")
        mp = mp.to(torch.int32).contiguous()
        H, L_q, L_kv, hd = self.dims
        B_c, B_u, L_self = Q.shape[0], K.shape[0], Q_self.shape[2]
        if tuple(Q.shape) != (B_c, H, L_q, hd) or tuple(K.shape) != (B_u, H, L_kv, hd) or K.shape != V.shape \
                or tuple(Q_self.shape) != (B_u, H, L_self, hd) or mp.shape != (B_c,):
            raise IkboError(IKBO_ERR_INVALID_ARG, "shape differs from the plan")
        out = torch.empty_like(Q) if out is None else out
        out_self = torch.empty_like(Q_self) if out_self is None else out_self
        st = self.forward_fused_ptrs(Q.data_ptr(), K.data_ptr(), V.data_ptr(), mp.data_ptr(), out.data_ptr(),
                                     Q_self.data_ptr(), out_self.data_ptr(), B_u, B_c, L_self, scale,
                                     _stream_handle(stream))
        if st != IKBO_OK:
            raise IkboError(st, "ikbo_fa_forward_fused")
        return out, out_self

    def check(self, stream=None) -> int:
        """Synchronise and return (and clear) the device-side status."""
        return lib().ikbo_fa_check(self.handle, _stream_handle(stream))

    def close(self) -> None:
        if getattr(self, "_h", None) is not None:
            st = lib().ikbo_fa_plan_destroy(self._h)
            self._h = None
            if st != IKBO_OK:
                raise IkboError(st, "ikbo_fa_plan_destroy")

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def lce_forward(U, C, mp, W_u, W_c, variant: str = "auto"):
    """One-shot forward with a temporary plan sized to these inputs."""
    torch = _torch()
    dtype = "bf16" if U.dtype == torch.bfloat16 else "f32"
    B_u, K_u, D = U.shape
    B_c, K_c, _ = C.shape
    M = W_u.shape[0]
    with LcePlan(B_u, B_c, K_u, K_c, M, D, dtype=dtype, variant=variant) as plan:
        Y = plan.forward(U, C, mp, W_u, W_c)
        st = plan.check()
        if st != IKBO_OK:
            raise IkboError(st, "device status")
        return Y
