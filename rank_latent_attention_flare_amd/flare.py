"""Python binding of libflare: argument marshalling only.

Each function has the name of the C entry point it calls (include/flare.h)
and passes device pointers, sizes, the dtype code and the current torch
stream. No arithmetic of the operator happens here; PyTorch provides device
memory and streams. If libflare.so has not been built the first call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libflare.so")

FLARE_F32, FLARE_BF16 = 0, 1
FLARE_OP_ENCODE, FLARE_OP_DECODE, FLARE_OP_FORWARD, FLARE_OP_PP_FORWARD, FLARE_OP_BACKWARD = 0, 1, 2, 3, 4
FLARE_OP_PP_BACKWARD = 5
FLARE_OP_PP_QUERIES = 6
FLARE_LAYOUT_BHND, FLARE_LAYOUT_BNHD = 0, 1
FLARE_TUNE_CHUNKS, FLARE_TUNE_ENC_MBW, FLARE_TUNE_ENC_WM, FLARE_TUNE_ENC_WT = 0, 1, 2, 3
FLARE_TUNE_DEC_TB, FLARE_TUNE_DEC_GROUPS, FLARE_TUNE_FAIL_ALLOC, FLARE_TUNE_DEC_HEADS = 4, 5, 6, 7
FLARE_TUNE_KEYS = 8
FLARE_KERNEL_KINDS = 4
KERNEL_KIND_NAMES = ("encode_partial", "combine", "decode", "backward")

STATUS = {0: "FLARE_OK", 1: "FLARE_ERR_INVALID_ARG", 2: "FLARE_ERR_UNSUPPORTED", 3: "FLARE_ERR_NO_MEMORY",
          4: "FLARE_ERR_HIP"}


class FlareError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


_lib = None
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_ENTRY = ["flare_encode", "flare_decode", "flare_forward", "flare_pp_forward"]
_ENTRY_WS = _ENTRY + ["flare_pp_queries"]  # entry points with a *_ws variant


def lib() -> ctypes.CDLL:
    """Load libflare.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m rank_latent_attention_flare_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        base = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, ctypes.c_int, _vp]
        for name in _ENTRY_WS:
            getattr(L, name).argtypes = base
            getattr(L, name).restype = ctypes.c_int
            getattr(L, name + "_ws").argtypes = base + [_vp, ctypes.c_size_t]
            getattr(L, name + "_ws").restype = ctypes.c_int
        for name in _ENTRY:
            getattr(L, name + "_ex").argtypes = base[:10] + [ctypes.c_int, _vp, _vp, ctypes.c_size_t]
            getattr(L, name + "_ex").restype = ctypes.c_int
        bw = [_vp] * 7 + [_i64] * 5 + [ctypes.c_int, _vp]
        L.flare_backward.argtypes = bw
        L.flare_backward.restype = ctypes.c_int
        L.flare_backward_ws.argtypes = bw + [_vp, ctypes.c_size_t]
        L.flare_backward_ws.restype = ctypes.c_int
        L.flare_pp_backward.argtypes = bw
        L.flare_pp_backward.restype = ctypes.c_int
        L.flare_pp_backward_ws.argtypes = bw + [_vp, ctypes.c_size_t]
        L.flare_pp_backward_ws.restype = ctypes.c_int
        for name in ("flare_backward_ex", "flare_pp_backward_ex"):
            getattr(L, name).argtypes = bw[:13] + [ctypes.c_int, _vp, _vp, ctypes.c_size_t]
            getattr(L, name).restype = ctypes.c_int
        L.flare_forward_noalloc.argtypes = base
        L.flare_forward_noalloc.restype = ctypes.c_int
        L.flare_attend.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _vp]
        L.flare_attend.restype = ctypes.c_int
        L.flare_workspace_size.argtypes = [ctypes.c_int, _i64, _i64, _i64, _i64, _i64, ctypes.c_int]
        L.flare_workspace_size.restype = ctypes.c_size_t
        L.flare_status_string.argtypes = [ctypes.c_int]
        L.flare_status_string.restype = ctypes.c_char_p
        L.flare_last_error.argtypes = []
        L.flare_last_error.restype = ctypes.c_char_p
        L.flare_set_tuning.argtypes = [ctypes.c_int, _i64]
        L.flare_set_tuning.restype = ctypes.c_int
        L.flare_timing_enable.argtypes = [ctypes.c_int]
        L.flare_timing_enable.restype = ctypes.c_int
        L.flare_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i64)]
        L.flare_timing_read.restype = ctypes.c_int
        L.flare_copy_kernel.argtypes = [_vp, _vp, ctypes.c_size_t, _vp]
        L.flare_copy_kernel.restype = ctypes.c_int
        L.flare_read_kernel.argtypes = [_vp, ctypes.c_size_t, _vp, ctypes.c_size_t, _vp]
        L.flare_read_kernel.restype = ctypes.c_int
        L.flare_probe_lanes.argtypes = []
        L.flare_probe_lanes.restype = ctypes.c_size_t
        L.flare_probe_peak.argtypes = [ctypes.c_int, _i64, _vp, ctypes.c_size_t, ctypes.POINTER(ctypes.c_double), _vp]
        L.flare_probe_peak.restype = ctypes.c_int
        L.flare_describe_plan.argtypes = [ctypes.c_int, _i64, _i64, _i64, _i64, _i64, ctypes.c_int,
                                          ctypes.c_char_p, ctypes.c_size_t]
        L.flare_describe_plan.restype = ctypes.c_int
        _lib = L
    return _lib


def _raise(st: int) -> None:
    if st != 0:
        raise FlareError(st, lib().flare_last_error().decode())


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return FLARE_F32
    if dt == torch.bfloat16:
        return FLARE_BF16
    raise TypeError(f"libflare handles float32 and bfloat16 tensors, not {dt}")


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dims(op: int, Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor):
    if Q.dim() != 3 or K.dim() != 4 or V.dim() != 4:
        raise ValueError("expected Q [H, M, D], K [B, H, N, D] and V [B, H, N, D] (Z [B, H, M, D] for decode)")
    H, M, D = Q.shape
    B, H2, N, D2 = K.shape
    if H2 != H or D2 != D:
        raise ValueError(f"K shape {tuple(K.shape)} does not match Q shape {tuple(Q.shape)}")
    want_v = (B, H, M, D) if op == FLARE_OP_DECODE else (B, H, N, D)
    if tuple(V.shape) != want_v:
        raise ValueError(f"{'Z' if op == FLARE_OP_DECODE else 'V'} shape {tuple(V.shape)}, expected {want_v}")
    for t in (Q, K, V):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != Q.dtype:
            raise ValueError("Q, K and V must be contiguous device tensors of one dtype")
    return B, H, N, M, D


def _out(op, B, H, N, M, D, like: torch.Tensor, out: Optional[torch.Tensor]) -> torch.Tensor:
    shape = (B, H, M, D) if op in (FLARE_OP_ENCODE, FLARE_OP_PP_QUERIES) else (B, H, N, D)
    if out is None:
        return torch.empty(shape, dtype=like.dtype, device=like.device)
    if tuple(out.shape) != shape or out.dtype != like.dtype or not out.is_contiguous() or not out.is_cuda:
        raise ValueError(f"out must be a contiguous {like.dtype} device tensor of shape {shape}")
    return out


def _call(op: int, name: str, Q, K, V, out, stream, workspace):
    B, H, N, M, D = _dims(op, Q, K, V)
    Y = _out(op, B, H, N, M, D, Q, out)
    dt = dtype_code(Q.dtype)
    args = [Q.data_ptr(), K.data_ptr(), V.data_ptr(), Y.data_ptr(), B, H, N, M, D, dt, _stream(stream)]
    L = lib()
    if workspace is None:
        _raise(getattr(L, name)(*args))
    else:
        _raise(getattr(L, name + "_ws")(*args, workspace.data_ptr(), workspace.numel() * workspace.element_size()))
    return Y


def flare_encode(Q, K, V, out=None, stream=None, workspace=None) -> torch.Tensor:
    """Z [B, H, M, D] = encode(Q [H, M, D], K, V [B, H, N, D])."""
    return _call(FLARE_OP_ENCODE, "flare_encode", Q, K, V, out, stream, workspace)


def flare_decode(Q, K, Z, out=None, stream=None, workspace=None) -> torch.Tensor:
    """Y [B, H, N, D] = decode(Q [H, M, D], K [B, H, N, D], Z [B, H, M, D])."""
    return _call(FLARE_OP_DECODE, "flare_decode", Q, K, Z, out, stream, workspace)


def flare_forward(Q, K, V, out=None, stream=None, workspace=None) -> torch.Tensor:
    """Y [B, H, N, D] = FLARE(Q, K, V)."""
    return _call(FLARE_OP_FORWARD, "flare_forward", Q, K, V, out, stream, workspace)


def flare_pp_forward(Q, K, V, out=None, stream=None, workspace=None) -> torch.Tensor:
    """Y [B, H, N, D] = FLARE++(Q, K, V)."""
    return _call(FLARE_OP_PP_FORWARD, "flare_pp_forward", Q, K, V, out, stream, workspace)


def flare_forward_noalloc(Q, K, V, out=None, stream=None) -> torch.Tensor:
    """Y [B, H, N, D] = FLARE(Q, K, V) with the library's static scratch (no allocation in the library;
    pass `out` to allocate nothing at all)."""
    return _call(FLARE_OP_FORWARD, "flare_forward_noalloc", Q, K, V, out, stream, None)


def flare_pp_queries(Q, K, V, out=None, stream=None, workspace=None) -> torch.Tensor:
    """Q' [B, H, M, D] = Q + encode(Q, K, V) in the operator dtype: the corrected queries FLARE++ uses."""
    return _call(FLARE_OP_PP_QUERIES, "flare_pp_queries", Q, K, V, out, stream, workspace)


def _call_ex(op: int, name: str, Q, K, V, layout: int, out, stream, workspace):
    """K, V and Y token-major ([B, N, H, D]) with FLARE_LAYOUT_BNHD; Z stays [B, H, M, D]."""
    if layout == FLARE_LAYOUT_BHND:
        B, H, N, M, D = _dims(op, Q, K, V)
    else:
        if Q.dim() != 3 or K.dim() != 4 or V.dim() != 4:
            raise ValueError("expected Q [H, M, D], K [B, N, H, D] and V [B, N, H, D] (Z [B, H, M, D] for decode)")
        H, M, D = Q.shape
        B, N, H2, D2 = K.shape
        if H2 != H or D2 != D:
            raise ValueError(f"K shape {tuple(K.shape)} does not match Q shape {tuple(Q.shape)}")
        want_v = (B, H, M, D) if op == FLARE_OP_DECODE else (B, N, H, D)
        if tuple(V.shape) != want_v:
            raise ValueError(f"{'Z' if op == FLARE_OP_DECODE else 'V'} shape {tuple(V.shape)}, expected {want_v}")
        for t in (Q, K, V):
            if not t.is_cuda or not t.is_contiguous() or t.dtype != Q.dtype:
                raise ValueError("Q, K and V must be contiguous device tensors of one dtype")
    if op == FLARE_OP_ENCODE:
        shape = (B, H, M, D)
    else:
        shape = (B, H, N, D) if layout == FLARE_LAYOUT_BHND else (B, N, H, D)
    if out is None:
        out = torch.empty(shape, dtype=Q.dtype, device=Q.device)
    elif tuple(out.shape) != shape or out.dtype != Q.dtype or not out.is_contiguous() or not out.is_cuda:
        raise ValueError(f"out must be a contiguous {Q.dtype} device tensor of shape {shape}")
    ws, nws = (None, 0) if workspace is None else (workspace.data_ptr(), workspace.numel() * workspace.element_size())
    _raise(getattr(lib(), name + "_ex")(Q.data_ptr(), K.data_ptr(), V.data_ptr(), out.data_ptr(), B, H, N, M, D,
                                        dtype_code(Q.dtype), layout, _stream(stream), ws, nws))
    return out


def flare_encode_ex(Q, K, V, layout, out=None, stream=None, workspace=None) -> torch.Tensor:
    """Z [B, H, M, D] = encode(Q, K, V) with K, V in `layout`."""
    return _call_ex(FLARE_OP_ENCODE, "flare_encode", Q, K, V, layout, out, stream, workspace)


def flare_decode_ex(Q, K, Z, layout, out=None, stream=None, workspace=None) -> torch.Tensor:
    """Y = decode(Q, K, Z) with K and Y in `layout` (Z [B, H, M, D])."""
    return _call_ex(FLARE_OP_DECODE, "flare_decode", Q, K, Z, layout, out, stream, workspace)


def flare_forward_ex(Q, K, V, layout, out=None, stream=None, workspace=None) -> torch.Tensor:
    """Y = FLARE(Q, K, V) with K, V and Y in `layout`."""
    return _call_ex(FLARE_OP_FORWARD, "flare_forward", Q, K, V, layout, out, stream, workspace)


def flare_pp_forward_ex(Q, K, V, layout, out=None, stream=None, workspace=None) -> torch.Tensor:
    """Y = FLARE++(Q, K, V) with K, V and Y in `layout`."""
    return _call_ex(FLARE_OP_PP_FORWARD, "flare_pp_forward", Q, K, V, layout, out, stream, workspace)


def flare_attend(q, Z, layout=FLARE_LAYOUT_BHND, out=None, stream=None) -> torch.Tensor:
    """Y = softmax_M(s q Z^T) Z: token queries q ([B, H, N, D], or [B, N, H, D] token-major) attend to
    the latent states Z [B, H, M, D]; Y has q's layout."""
    if q.dim() != 4 or Z.dim() != 4:
        raise ValueError("expected q [B, H, N, D] (or [B, N, H, D]) and Z [B, H, M, D]")
    if layout == FLARE_LAYOUT_BHND:
        B, H, N, D = q.shape
    else:
        B, N, H, D = q.shape
    B2, H2, M, D2 = Z.shape
    if (B2, H2, D2) != (B, H, D):
        raise ValueError(f"Z shape {tuple(Z.shape)} does not match q shape {tuple(q.shape)}")
    for t in (q, Z):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != q.dtype:
            raise ValueError("q and Z must be contiguous device tensors of one dtype")
    if out is None:
        out = torch.empty_like(q)
    elif tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype or not out.is_contiguous() or not out.is_cuda:
        raise ValueError(f"out must be a contiguous {q.dtype} device tensor of shape {tuple(q.shape)}")
    _raise(lib().flare_attend(q.data_ptr(), Z.data_ptr(), out.data_ptr(), B, H, N, M, D, dtype_code(q.dtype),
                              layout, _stream(stream)))
    return out


def flare_backward(Q, K, V, dY, stream=None, workspace=None, out=None):
    """(dQ [H, M, D], dK, dV [B, H, N, D]): gradients of the FLARE forward for the upstream gradient dY."""
    B, H, N, M, D = _dims(FLARE_OP_FORWARD, Q, K, V)
    if tuple(dY.shape) != (B, H, N, D) or dY.dtype != Q.dtype or not dY.is_contiguous() or not dY.is_cuda:
        raise ValueError(f"dY must be a contiguous {Q.dtype} device tensor of shape {(B, H, N, D)}")
    if out is None:
        out = (torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V))
    dQ, dK, dV = out
    args = [Q.data_ptr(), K.data_ptr(), V.data_ptr(), dY.data_ptr(), dQ.data_ptr(), dK.data_ptr(), dV.data_ptr(),
            B, H, N, M, D, dtype_code(Q.dtype), _stream(stream)]
    if workspace is None:
        _raise(lib().flare_backward(*args))
    else:
        _raise(lib().flare_backward_ws(*args, workspace.data_ptr(), workspace.numel() * workspace.element_size()))
    return dQ, dK, dV


def flare_pp_backward(Q, K, V, dY, stream=None, workspace=None, out=None):
    """(dQ [H, M, D], dK, dV [B, H, N, D]): gradients of the FLARE++ forward for the upstream gradient dY."""
    B, H, N, M, D = _dims(FLARE_OP_PP_FORWARD, Q, K, V)
    if tuple(dY.shape) != (B, H, N, D) or dY.dtype != Q.dtype or not dY.is_contiguous() or not dY.is_cuda:
        raise ValueError(f"dY must be a contiguous {Q.dtype} device tensor of shape {(B, H, N, D)}")
    if out is None:
        out = (torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V))
    dQ, dK, dV = out
    args = [Q.data_ptr(), K.data_ptr(), V.data_ptr(), dY.data_ptr(), dQ.data_ptr(), dK.data_ptr(), dV.data_ptr(),
            B, H, N, M, D, dtype_code(Q.dtype), _stream(stream)]
    if workspace is None:
        _raise(lib().flare_pp_backward(*args))
    else:
        _raise(lib().flare_pp_backward_ws(*args, workspace.data_ptr(), workspace.numel() * workspace.element_size()))
    return dQ, dK, dV


def _backward_ex(name: str, Q, K, V, dY, layout: int, stream, workspace, out):
    if layout == FLARE_LAYOUT_BHND:
        B, H, N, M, D = _dims(FLARE_OP_FORWARD, Q, K, V)
        tok = (B, H, N, D)
    else:
        if Q.dim() != 3 or K.dim() != 4:
            raise ValueError("expected Q [H, M, D] and K, V, dY [B, N, H, D]")
        H, M, D = Q.shape
        B, N = K.shape[:2]
        tok = (B, N, H, D)
    for t in (K, V, dY):
        if tuple(t.shape) != tok or t.dtype != Q.dtype or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"K, V and dY must be contiguous {Q.dtype} device tensors of shape {tok}")
    if not Q.is_cuda or not Q.is_contiguous():
        raise ValueError("Q must be a contiguous device tensor")
    if out is None:
        out = (torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V))
    dQ, dK, dV = out
    ws, nws = (None, 0) if workspace is None else (workspace.data_ptr(), workspace.numel() * workspace.element_size())
    _raise(getattr(lib(), name)(Q.data_ptr(), K.data_ptr(), V.data_ptr(), dY.data_ptr(), dQ.data_ptr(),
                                dK.data_ptr(), dV.data_ptr(), B, H, N, M, D, dtype_code(Q.dtype), layout,
                                _stream(stream), ws, nws))
    return dQ, dK, dV


def flare_backward_ex(Q, K, V, dY, layout, stream=None, workspace=None, out=None):
    """flare_backward with K, V, dY (and dK, dV) in `layout` ([B, N, H, D] with FLARE_LAYOUT_BNHD)."""
    return _backward_ex("flare_backward_ex", Q, K, V, dY, layout, stream, workspace, out)


def flare_pp_backward_ex(Q, K, V, dY, layout, stream=None, workspace=None, out=None):
    """flare_pp_backward with K, V, dY (and dK, dV) in `layout`."""
    return _backward_ex("flare_pp_backward_ex", Q, K, V, dY, layout, stream, workspace, out)


def flare_workspace_size(op: int, B: int, H: int, N: int, M: int, D: int, dtype: torch.dtype) -> int:
    return int(lib().flare_workspace_size(op, B, H, N, M, D, dtype_code(dtype)))


def workspace_for(op: int, Q: torch.Tensor, K: torch.Tensor) -> torch.Tensor:
    """Caller-owned workspace tensor for the *_ws variants (256-byte aligned by torch's allocator)."""
    H, M, D = Q.shape
    B, _, N, _ = K.shape
    n = flare_workspace_size(op, B, H, N, M, D, Q.dtype)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=Q.device)


def flare_describe_plan(op: int, B: int, H: int, N: int, M: int, D: int, dtype: torch.dtype) -> str:
    buf = ctypes.create_string_buffer(512)
    _raise(lib().flare_describe_plan(op, B, H, N, M, D, dtype_code(dtype), buf, 512))
    return buf.value.decode()


def flare_set_tuning(key: int, value: int) -> None:
    """Process-wide launch-plan override (FLARE_TUNE_*); 0 restores the library's choice."""
    _raise(lib().flare_set_tuning(int(key), int(value)))


def flare_timing_enable(on: bool) -> None:
    _raise(lib().flare_timing_enable(1 if on else 0))


def flare_timing_read():
    """{kind name: (total ms, launches)} since the last read or enable."""
    ms = (ctypes.c_double * FLARE_KERNEL_KINDS)()
    cnt = (_i64 * FLARE_KERNEL_KINDS)()
    _raise(lib().flare_timing_read(ms, cnt))
    return {KERNEL_KIND_NAMES[i]: (ms[i], cnt[i]) for i in range(FLARE_KERNEL_KINDS)}


FLARE_PROBE_MFMA_BF16, FLARE_PROBE_EXP = 0, 1


def flare_probe_peak(kind: int, iters: int, out: torch.Tensor, stream=None) -> float:
    """Launch a peak probe (FLARE_PROBE_MFMA_BF16 or FLARE_PROBE_EXP) on the stream; returns the work
    launched (flops, or exponentials). `out` is a float32 device tensor of at least flare_probe_lanes()."""
    if out.dtype != torch.float32 or not out.is_cuda or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 device tensor")
    work = ctypes.c_double(0.0)
    _raise(lib().flare_probe_peak(kind, iters, out.data_ptr(), out.numel(), ctypes.byref(work), _stream(stream)))
    return work.value


def flare_read_kernel(src: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    """Streaming read of all of src's bytes (a calibration kernel); out: float32, >= flare_probe_lanes()."""
    if out.dtype != torch.float32 or not out.is_cuda or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 device tensor")
    _raise(lib().flare_read_kernel(src.data_ptr(), src.numel() * src.element_size(), out.data_ptr(), out.numel(),
                                   _stream(stream)))


def flare_probe_lanes() -> int:
    return int(lib().flare_probe_lanes())


def flare_copy_kernel(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    n = src.numel() * src.element_size()
    _raise(lib().flare_copy_kernel(src.data_ptr(), dst.data_ptr(), n, _stream(stream)))
