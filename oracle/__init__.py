"""fp64 CPU oracle for the FLARE / FLARE++ forward operator.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may use this package; the GPU library and its
Python binding never import it. It shares no code with the GPU path.

The arithmetic lives in ``flare_oracle.c`` (plain fp64 loops, one function per
definition on the FLARE pages). This module only builds and loads that
library, widens stored inputs exactly to fp64, and loops over (batch, head).

Inputs follow the storage convention of ``flare_inputs``: fp32 tensors are
``float32`` arrays, bf16 tensors are ``uint16`` arrays of bf16 bit patterns.
Shapes: Q is [H, M, D] (shared over the batch) or [B, H, M, D]; K and V are
[B, H, N, D]; the token queries q of ``attend`` are [B, H, N, D] and its Z is
[B, H, M, D]; the results are fp64 arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "flare_oracle.c")
_LIB = os.path.join(_HERE, "libflare_oracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, strict IEEE: no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
               "-ffp-contract=off", "-std=c99", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        lib.flare_oracle_encode.argtypes = [_dp, _dp, _dp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _dp]
        lib.flare_oracle_decode.argtypes = [_dp, _dp, _dp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                            _i64p, ctypes.c_int64, _dp]
        lib.flare_oracle_forward.argtypes = [_dp, _dp, _dp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                             _i64p, ctypes.c_int64, _dp, _dp]
        lib.flare_oracle_pp_forward.argtypes = [_dp, _dp, _dp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                                _i64p, ctypes.c_int64, _dp, _dp, _dp]
        lib.flare_oracle_backward.argtypes = [_dp, _dp, _dp, _dp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                              _dp, _dp, _dp]
        lib.flare_oracle_backward.restype = ctypes.c_int
        for f in ("flare_oracle_encode_backward", "flare_oracle_pp_backward"):
            getattr(lib, f).argtypes = [_dp, _dp, _dp, _dp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _dp,
                                        _dp, _dp]
            getattr(lib, f).restype = ctypes.c_int
        lib.flare_oracle_attend.argtypes = [_dp, _dp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _i64p,
                                            ctypes.c_int64, _dp]
        for f in ("flare_oracle_encode", "flare_oracle_decode", "flare_oracle_forward", "flare_oracle_pp_forward",
                  "flare_oracle_attend"):
            getattr(lib, f).restype = ctypes.c_int
        lib.flare_oracle_threads.restype = ctypes.c_int
        lib.flare_oracle_set_threads.argtypes = [ctypes.c_int]
        _lib = lib
    return _lib


def threads() -> int:
    return _load().flare_oracle_threads()


def set_threads(n: int) -> None:
    _load().flare_oracle_set_threads(int(n))


def widen(x: np.ndarray) -> np.ndarray:
    """Exact fp64 value of stored inputs: float32/float64 as is, uint16 as bf16 bits."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if x.dtype in (np.float32, np.float64):
        return x.astype(np.float64)
    raise TypeError(f"unsupported stored dtype {x.dtype}")


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_dp)


def _check(rc: int, what: str) -> None:
    if rc == -1:
        raise MemoryError(f"oracle {what}: scratch allocation failed")
    if rc == -2:
        raise IndexError(f"oracle {what}: token row out of range")
    if rc != 0:
        raise RuntimeError(f"oracle {what}: status {rc}")


def _c64(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _q_for(Q: np.ndarray, b: int, h: int) -> np.ndarray:
    return Q[h] if Q.ndim == 3 else Q[b, h]


def encode_head(Q, K, V) -> np.ndarray:
    """Z[M,D] of one head from fp64 Q[M,D], K[N,D], V[N,D]."""
    Q, K, V = _c64(Q), _c64(K), _c64(V)
    N, D = K.shape
    M = Q.shape[0]
    Z = np.empty((M, D), np.float64)
    _check(_load().flare_oracle_encode(_ptr(Q), _ptr(K), _ptr(V), N, M, D, _ptr(Z)), "encode")
    return Z


def decode_head(Q, K, Z, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Y[R,D] of one head for the selected token rows (all tokens if None)."""
    Q, K, Z = _c64(Q), _c64(K), _c64(Z)
    N, D = K.shape
    M = Q.shape[0]
    if rows is None:
        R, rp = N, None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        R, rp = rows.shape[0], rows.ctypes.data_as(_i64p)
    Y = np.empty((R, D), np.float64)
    _check(_load().flare_oracle_decode(_ptr(Q), _ptr(K), _ptr(Z), N, M, D, rp, R, _ptr(Y)), "decode")
    return Y


def attend_head(q, Z, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Y[R,D] of one head: token queries q[N,D] attend to Z[M,D] (keys and values)."""
    q, Z = _c64(q), _c64(Z)
    N, D = q.shape
    M = Z.shape[0]
    if rows is None:
        R, rp = N, None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        R, rp = rows.shape[0], rows.ctypes.data_as(_i64p)
    Y = np.empty((R, D), np.float64)
    _check(_load().flare_oracle_attend(_ptr(q), _ptr(Z), N, M, D, rp, R, _ptr(Y)), "attend")
    return Y


def backward_head(Q, K, V, dY):
    """(dQ[M,D], dK[N,D], dV[N,D]) of one head's FLARE forward for the upstream gradient dY[N,D]."""
    Q, K, V, dY = _c64(Q), _c64(K), _c64(V), _c64(dY)
    N, D = K.shape
    M = Q.shape[0]
    dQ, dK, dV = np.empty((M, D)), np.empty((N, D)), np.empty((N, D))
    _check(_load().flare_oracle_backward(_ptr(Q), _ptr(K), _ptr(V), _ptr(dY), N, M, D, _ptr(dQ), _ptr(dK),
                                         _ptr(dV)), "backward")
    return dQ, dK, dV


def encode_backward_head(Q, K, V, dZ):
    """(dQ[M,D], dK[N,D], dV[N,D]) of one head's encode for the upstream gradient dZ[M,D]."""
    Q, K, V, dZ = _c64(Q), _c64(K), _c64(V), _c64(dZ)
    N, D = K.shape
    M = Q.shape[0]
    dQ, dK, dV = np.empty((M, D)), np.empty((N, D)), np.empty((N, D))
    _check(_load().flare_oracle_encode_backward(_ptr(Q), _ptr(K), _ptr(V), _ptr(dZ), N, M, D, _ptr(dQ), _ptr(dK),
                                                _ptr(dV)), "encode_backward")
    return dQ, dK, dV


def pp_backward_head(Q, K, V, dY):
    """(dQ[M,D], dK[N,D], dV[N,D]) of one head's FLARE++ forward for the upstream gradient dY[N,D]."""
    Q, K, V, dY = _c64(Q), _c64(K), _c64(V), _c64(dY)
    N, D = K.shape
    M = Q.shape[0]
    dQ, dK, dV = np.empty((M, D)), np.empty((N, D)), np.empty((N, D))
    _check(_load().flare_oracle_pp_backward(_ptr(Q), _ptr(K), _ptr(V), _ptr(dY), N, M, D, _ptr(dQ), _ptr(dK),
                                            _ptr(dV)), "pp_backward")
    return dQ, dK, dV


def pp_forward_head(Q, K, V, rows: Optional[np.ndarray] = None):
    """(Y, Q', Z) of one head for FLARE++."""
    Q, K, V = _c64(Q), _c64(K), _c64(V)
    N, D = K.shape
    M = Q.shape[0]
    if rows is None:
        R, rp = N, None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        R, rp = rows.shape[0], rows.ctypes.data_as(_i64p)
    Y = np.empty((R, D), np.float64)
    Qp = np.empty((M, D), np.float64)
    Z = np.empty((M, D), np.float64)
    _check(_load().flare_oracle_pp_forward(_ptr(Q), _ptr(K), _ptr(V), N, M, D, rp, R, _ptr(Y), _ptr(Qp),
                                           _ptr(Z)), "pp_forward")
    return Y, Qp, Z


# ---------------------------------------------------------------- batched API
def encode(Q, K, V, heads=None) -> np.ndarray:
    """Z[B,H,M,D] (fp64). ``heads`` optionally restricts to a list of (b, h)."""
    B, H, N, D = K.shape
    M = Q.shape[-2]
    Z = np.full((B, H, M, D), np.nan)
    for b, h in (heads or [(b, h) for b in range(B) for h in range(H)]):
        Z[b, h] = encode_head(widen(_q_for(Q, b, h)), widen(K[b, h]), widen(V[b, h]))
    return Z


def decode(Q, K, Z, rows=None, heads=None) -> np.ndarray:
    """Y[B,H,R,D] (fp64) with Z given as stored values or fp64."""
    B, H, N, D = K.shape
    R = N if rows is None else len(rows)
    Y = np.full((B, H, R, D), np.nan)
    for b, h in (heads or [(b, h) for b in range(B) for h in range(H)]):
        Y[b, h] = decode_head(widen(_q_for(Q, b, h)), widen(K[b, h]), widen(Z[b, h]), rows)
    return Y


def attend(q, Z, rows=None, heads=None) -> np.ndarray:
    """Y[B,H,R,D] (fp64): token queries q[B,H,N,D] attend to Z[B,H,M,D]."""
    B, H, N, D = q.shape
    R = N if rows is None else len(rows)
    Y = np.full((B, H, R, D), np.nan)
    for b, h in (heads or [(b, h) for b in range(B) for h in range(H)]):
        Y[b, h] = attend_head(widen(q[b, h]), widen(Z[b, h]), rows)
    return Y


def backward(Q, K, V, dY):
    """(dQ[H,M,D], dK[B,H,N,D], dV[B,H,N,D]) of the FLARE forward, fp64. Q is shared over the
    batch, so dQ sums the batch entries' gradients."""
    B, H, N, D = K.shape
    M = Q.shape[-2]
    dQ = np.zeros((H, M, D))
    dK = np.empty((B, H, N, D))
    dV = np.empty((B, H, N, D))
    for b in range(B):
        for h in range(H):
            q, k, v, g = widen(Q[h]), widen(K[b, h]), widen(V[b, h]), widen(dY[b, h])
            dq, dK[b, h], dV[b, h] = backward_head(q, k, v, g)
            dQ[h] += dq
    return dQ, dK, dV


def pp_backward(Q, K, V, dY):
    """(dQ[H,M,D], dK[B,H,N,D], dV[B,H,N,D]) of the FLARE++ forward, fp64. Q is shared over the
    batch, so dQ sums the batch entries' gradients."""
    B, H, N, D = K.shape
    M = Q.shape[-2]
    dQ = np.zeros((H, M, D))
    dK = np.empty((B, H, N, D))
    dV = np.empty((B, H, N, D))
    for b in range(B):
        for h in range(H):
            q, k, v, g = widen(Q[h]), widen(K[b, h]), widen(V[b, h]), widen(dY[b, h])
            dq, dK[b, h], dV[b, h] = pp_backward_head(q, k, v, g)
            dQ[h] += dq
    return dQ, dK, dV


def forward(Q, K, V, rows=None, heads=None):
    """(Y[B,H,R,D], Z[B,H,M,D]) of FLARE in fp64."""
    B, H, N, D = K.shape
    M = Q.shape[-2]
    R = N if rows is None else len(rows)
    Y = np.full((B, H, R, D), np.nan)
    Z = np.full((B, H, M, D), np.nan)
    for b, h in (heads or [(b, h) for b in range(B) for h in range(H)]):
        q, k = widen(_q_for(Q, b, h)), widen(K[b, h])
        Z[b, h] = encode_head(q, k, widen(V[b, h]))
        Y[b, h] = decode_head(q, k, Z[b, h], rows)
    return Y, Z


def pp_forward(Q, K, V, rows=None, heads=None):
    """(Y[B,H,R,D], Q'[B,H,M,D], Z[B,H,M,D]) of FLARE++ in fp64."""
    B, H, N, D = K.shape
    M = Q.shape[-2]
    R = N if rows is None else len(rows)
    Y = np.full((B, H, R, D), np.nan)
    Qp = np.full((B, H, M, D), np.nan)
    Z = np.full((B, H, M, D), np.nan)
    for b, h in (heads or [(b, h) for b in range(B) for h in range(H)]):
        Y[b, h], Qp[b, h], Z[b, h] = pp_forward_head(widen(_q_for(Q, b, h)), widen(K[b, h]), widen(V[b, h]),
                                                     rows)
    return Y, Qp, Z
