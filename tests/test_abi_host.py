"""Host-side checks of the C ABI that need no GPU.

The library must load, export every function include/flare.h declares, and
reject bad arguments before touching the device (validation runs before any
HIP call, so these tests are safe on a machine without a GPU).
"""
import ctypes
import os
import re

import pytest

from rank_latent_attention_flare_amd import flare as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flare.h")

pytestmark = pytest.mark.skipif(not os.path.exists(F.LIB_PATH), reason="libflare.so not built")

OK, INVALID, UNSUPPORTED, NOMEM = 0, 1, 2, 3
# fake, 256-byte aligned, non-overlapping "device" addresses (never dereferenced)
PQ, PK, PV, PY, PW = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flare_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 14
    L = F.lib()
    for n in names:
        assert hasattr(L, n), n


def call(name, *args, ws=None):
    L = F.lib()
    fn = getattr(L, name if ws is None else name + "_ws")
    base = list(args) + [None]
    if ws is not None:
        base += list(ws)
    return fn(*base)


def fwd_args(q=PQ, k=PK, v=PV, y=PY, B=1, H=2, N=100, M=64, D=64, dt=F.FLARE_BF16):
    return (q, k, v, y, B, H, N, M, D, dt)


@pytest.mark.parametrize("name", ["flare_encode", "flare_decode", "flare_forward", "flare_pp_forward",
                                  "flare_pp_queries"])
def test_null_pointers_rejected(name):
    for i in range(4):
        a = list(fwd_args())
        a[i] = None
        assert call(name, *a) == INVALID
        assert "null" in F.lib().flare_last_error().decode()


@pytest.mark.parametrize("field", [4, 5, 6, 7, 8])
def test_sizes_below_one_rejected(field):
    for bad in (0, -3):
        a = list(fwd_args())
        a[field] = bad
        assert call("flare_forward", *a) == INVALID


@pytest.mark.parametrize("dt,D,M", [(F.FLARE_BF16, 16, 64), (F.FLARE_BF16, 48, 64), (F.FLARE_BF16, 64, 513),
                                    (F.FLARE_BF16, 32, 600), (F.FLARE_BF16, 128, 513),
                                    (F.FLARE_F32, 12, 8), (F.FLARE_F32, 256, 8), (F.FLARE_F32, 16, 5000)])
def test_unsupported_shapes(dt, D, M):
    assert call("flare_forward", *fwd_args(D=D, M=M, dt=dt)) == UNSUPPORTED
    assert F.lib().flare_workspace_size(F.FLARE_OP_FORWARD, 1, 2, 100, M, D, dt) == 0


def test_bad_dtype_and_grid_limits():
    assert call("flare_forward", *fwd_args(dt=7)) == INVALID
    assert call("flare_forward", *fwd_args(B=300, H=300)) == UNSUPPORTED


def test_misaligned_pointers_rejected():
    assert call("flare_forward", *fwd_args(k=PK + 8)) == INVALID
    assert "aligned" in F.lib().flare_last_error().decode()


def test_output_aliasing_rejected():
    assert call("flare_forward", *fwd_args(y=PK)) == INVALID
    assert "overlaps" in F.lib().flare_last_error().decode()
    # partial overlap of Y with V
    assert call("flare_forward", *fwd_args(y=PV + 4096)) == INVALID


def test_workspace_sizes_consistent():
    L = F.lib()
    args = (1, 16, 1 << 20, 256, 64, F.FLARE_BF16)
    enc = L.flare_workspace_size(F.FLARE_OP_ENCODE, *args)
    dec = L.flare_workspace_size(F.FLARE_OP_DECODE, *args)
    fwd = L.flare_workspace_size(F.FLARE_OP_FORWARD, *args)
    pp = L.flare_workspace_size(F.FLARE_OP_PP_FORWARD, *args)
    assert dec == 0 and 0 < enc < fwd < pp
    # partials stay small next to the 8 GiB of K/V/Y traffic
    assert fwd < 0.03 * (1 << 33)
    assert L.flare_workspace_size(9, *args) == 0


def test_workspace_checks():
    need = F.lib().flare_workspace_size(F.FLARE_OP_FORWARD, 1, 2, 100, 64, 64, F.FLARE_BF16)
    assert call("flare_forward", *fwd_args(), ws=(PW, need - 1)) == INVALID
    assert "too small" in F.lib().flare_last_error().decode()
    assert call("flare_forward", *fwd_args(), ws=(None, need)) == INVALID
    assert call("flare_forward", *fwd_args(), ws=(PW + 16, need)) == INVALID


def test_injected_allocation_failure():
    F.flare_set_tuning(F.FLARE_TUNE_FAIL_ALLOC, 1)
    try:
        assert call("flare_forward", *fwd_args()) == NOMEM
        assert call("flare_pp_queries", *fwd_args()) == NOMEM
        assert "injected" in F.lib().flare_last_error().decode()
    finally:
        F.flare_set_tuning(F.FLARE_TUNE_FAIL_ALLOC, 0)


def test_tuning_keys_validated():
    L = F.lib()
    assert L.flare_set_tuning(F.FLARE_TUNE_CHUNKS, -1) == INVALID
    assert L.flare_set_tuning(99, 1) == INVALID
    assert L.flare_set_tuning(-1, 1) == INVALID
    # an override changes the plan, and 0 restores the library's own
    buf = ctypes.create_string_buffer(512)
    args = (F.FLARE_OP_FORWARD, 4, 8, 65536, 128, 32, F.FLARE_BF16, buf, 512)
    assert L.flare_describe_plan(*args) == OK
    default = buf.value.decode()
    F.flare_set_tuning(F.FLARE_TUNE_CHUNKS, 3)
    try:
        assert L.flare_describe_plan(*args) == OK
        assert "encode grid (3,32)" in buf.value.decode()
    finally:
        F.flare_set_tuning(F.FLARE_TUNE_CHUNKS, 0)
    assert L.flare_describe_plan(*args) == OK
    assert buf.value.decode() == default


def test_status_strings_and_plan():
    L = F.lib()
    for code, name in F.STATUS.items():
        assert L.flare_status_string(code).decode() == name
    buf = ctypes.create_string_buffer(512)
    assert L.flare_describe_plan(F.FLARE_OP_FORWARD, 4, 8, 65536, 128, 32, F.FLARE_BF16, buf, 512) == OK
    txt = buf.value.decode()
    assert "encode grid" in txt and "decode grid" in txt
    assert L.flare_describe_plan(F.FLARE_OP_FORWARD, 4, 8, 65536, 128, 33, F.FLARE_BF16, buf, 512) == UNSUPPORTED


def test_copy_kernel_argument_checks():
    L = F.lib()
    assert L.flare_copy_kernel(PK, PV, 1000, None) == INVALID  # not a multiple of 16
    assert L.flare_copy_kernel(PK, PK + 256, 4096, None) == INVALID  # overlap
    assert L.flare_copy_kernel(None, PV, 4096, None) == INVALID


def test_timing_read_without_events():
    import ctypes as C
    ms = (C.c_double * 3)()
    cnt = (C.c_int64 * 3)()
    L = F.lib()
    assert L.flare_timing_enable(1) == OK
    assert L.flare_timing_read(ms, cnt) == OK
    assert list(cnt) == [0, 0, 0]
    assert L.flare_timing_enable(0) == OK


@pytest.mark.parametrize("name", ["flare_encode_ex", "flare_decode_ex", "flare_forward_ex", "flare_pp_forward_ex"])
def test_layout_variants_validate_before_launch(name):
    fn = getattr(F.lib(), name)
    # an unknown layout, a null pointer and an unsupported size are all
    # rejected before any device work (with or without a workspace)
    for ws in ((None, 0), (PW, 1 << 30)):
        assert fn(*fwd_args(), 7, None, *ws) == INVALID
        assert "layout" in F.lib().flare_last_error().decode()
        assert fn(*fwd_args(k=None), F.FLARE_LAYOUT_BNHD, None, *ws) == INVALID
        assert fn(*fwd_args(D=48), F.FLARE_LAYOUT_BNHD, None, *ws) == UNSUPPORTED
    # a too-small caller workspace is rejected too
    if name != "flare_decode_ex":
        assert fn(*fwd_args(), F.FLARE_LAYOUT_BNHD, None, PW, 256) == INVALID
        assert "workspace" in F.lib().flare_last_error().decode()


def test_attend_validates_before_launch():
    fn = F.lib().flare_attend
    args = [PQ, PK, PY, 1, 2, 100, 64, 64, F.FLARE_BF16]
    assert fn(*args, 7, None) == INVALID and "layout" in F.lib().flare_last_error().decode()
    assert fn(None, *args[1:], 0, None) == INVALID and "null" in F.lib().flare_last_error().decode()
    assert fn(PQ, PK, PQ + 256, *args[3:], 0, None) == INVALID  # Y overlaps q
    assert fn(PQ, PK, PY + 8, *args[3:], 0, None) == INVALID    # misaligned
    assert fn(PQ, PK, PY, 1, 2, 100, 600, 64, F.FLARE_BF16, 0, None) == UNSUPPORTED


def test_backward_validates_before_launch():
    fn = F.lib().flare_backward
    PG, PDQ, PDK, PDV = 0x60000000, 0x70000000, 0x80000000, 0x90000000
    ok = [PQ, PK, PV, PG, PDQ, PDK, PDV, 1, 2, 100, 64, 32, F.FLARE_BF16, None]
    a = list(ok); a[3] = None
    assert fn(*a) == INVALID and "null" in F.lib().flare_last_error().decode()
    a = list(ok); a[5] = PK  # dK aliases K
    assert fn(*a) == INVALID and "overlap" in F.lib().flare_last_error().decode()
    a = list(ok); a[11] = 256  # D = 256: neither forward nor backward
    assert fn(*a) == UNSUPPORTED
    a = list(ok); a[11] = 96  # bf16 has no D = 96
    assert fn(*a) == UNSUPPORTED
    ws = F.lib().flare_workspace_size(F.FLARE_OP_BACKWARD, 1, 2, 100, 64, 32, F.FLARE_BF16)
    assert ws >= F.lib().flare_workspace_size(F.FLARE_OP_FORWARD, 1, 2, 100, 64, 32, F.FLARE_BF16) > 0
    assert F.lib().flare_backward_ws(*ok, PW, 256) == INVALID
    # the layout variant: a bad layout, and the same checks as the plain entry
    ex = F.lib().flare_backward_ex
    assert ex(*ok[:13], 7, None, None, 0) == INVALID and "layout" in F.lib().flare_last_error().decode()
    a = list(ok); a[5] = PK
    assert ex(*a[:13], F.FLARE_LAYOUT_BNHD, None, None, 0) == INVALID
    assert ex(*ok[:13], F.FLARE_LAYOUT_BNHD, None, PW, 256) == INVALID
    assert "workspace" in F.lib().flare_last_error().decode()


def test_pp_backward_validates_before_launch():
    fn = F.lib().flare_pp_backward
    PG, PDQ, PDK, PDV = 0x60000000, 0x70000000, 0x80000000, 0x90000000
    ok = [PQ, PK, PV, PG, PDQ, PDK, PDV, 1, 2, 100, 64, 32, F.FLARE_BF16, None]
    a = list(ok); a[6] = None
    assert fn(*a) == INVALID and "null" in F.lib().flare_last_error().decode()
    a = list(ok); a[4] = PQ + 64  # dQ overlaps Q
    assert fn(*a) == INVALID and "overlap" in F.lib().flare_last_error().decode()
    a = list(ok); a[11] = 256  # D = 256: neither forward nor backward
    assert fn(*a) == UNSUPPORTED
    ex = F.lib().flare_pp_backward_ex
    assert ex(*ok[:13], 7, None, None, 0) == INVALID and "layout" in F.lib().flare_last_error().decode()
    a = list(ok); a[4] = PQ + 64
    assert ex(*a[:13], F.FLARE_LAYOUT_BNHD, None, None, 0) == INVALID
    # its workspace holds a FLARE backward's plus Q', dQ', a zero dY and the first stage's dQ
    args = (2, 2, 100, 64, 32, F.FLARE_BF16)
    ws = F.lib().flare_workspace_size(F.FLARE_OP_PP_BACKWARD, *args)
    tok = 2 * 2 * 100 * 32 * 2
    assert ws >= F.lib().flare_workspace_size(F.FLARE_OP_BACKWARD, *args) + tok > 0
    assert F.lib().flare_pp_backward_ws(*ok, PW, 256) == INVALID
    assert "workspace" in F.lib().flare_last_error().decode()


def test_noalloc_rejects_oversized_workspace():
    # the forward workspace of (64, 16, 2^22, 512, 64) bf16 (262 MiB) exceeds
    # the 64 MiB static scratch: rejected before any device call
    L = F.lib()
    need = L.flare_workspace_size(F.FLARE_OP_FORWARD, 64, 16, 1 << 22, 512, 64, F.FLARE_BF16)
    assert need > (64 << 20)
    args = (PQ, PK, PV, PY, 64, 16, 1 << 22, 512, 64, F.FLARE_BF16, None)
    assert L.flare_forward_noalloc(*args) == UNSUPPORTED
    assert "static scratch" in L.flare_last_error().decode()
    assert L.flare_forward_noalloc(PQ, PK, PV, PY, 0, 1, 10, 10, 64, F.FLARE_BF16, None) == INVALID


def test_probe_validates_before_launch():
    import ctypes
    L = F.lib()
    n = L.flare_probe_lanes()
    assert n == 256 * 4 * 4 * 64
    work = ctypes.c_double(0.0)
    fn = L.flare_probe_peak
    assert fn(7, 10, PY, n, ctypes.byref(work), None) == INVALID and "kind" in L.flare_last_error().decode()
    assert fn(F.FLARE_PROBE_MFMA_BF16, 0, PY, n, ctypes.byref(work), None) == INVALID
    assert fn(F.FLARE_PROBE_EXP, (1 << 20) + 1, PY, n, ctypes.byref(work), None) == INVALID
    assert fn(F.FLARE_PROBE_EXP, 10, None, n, ctypes.byref(work), None) == INVALID
    assert fn(F.FLARE_PROBE_EXP, 10, PY, n - 1, ctypes.byref(work), None) == INVALID
    assert fn(F.FLARE_PROBE_EXP, 10, PY, n, None, None) == INVALID


def test_read_kernel_validates_before_launch():
    L = F.lib()
    n = L.flare_probe_lanes()
    assert L.flare_read_kernel(None, 1024, PY, n, None) == INVALID
    assert L.flare_read_kernel(PK, 1000, PY, n, None) == INVALID  # not a multiple of 16
    assert L.flare_read_kernel(PK + 8, 1024, PY, n, None) == INVALID
    assert L.flare_read_kernel(PK, 1024, PY, n - 1, None) == INVALID
