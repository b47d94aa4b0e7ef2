"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/w12.h declares, and rejects bad arguments with the
documented status codes before touching the GPU."""
import ctypes
import os
import re

import pytest

from lossless_compressed_weight_amd import w12

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w12.h")

# Fake, 256-byte aligned device addresses: argument checks must reject the
# calls below before any HIP call could dereference them.
FAKE = 0x7F0000000000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w \*]*?\b(w12_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    lib = w12.lib()
    names = declared_functions()
    assert len(names) >= 12
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(w12._SIGNATURES), "binding and header disagree"


def test_versions_and_status_strings():
    lib = w12.lib()
    assert lib.w12_abi_version() == w12.ABI_VERSION
    for code in range(-8, 1):
        assert w12.status_str(code)
    assert w12.status_str(-99) == "unknown status"
    assert w12.last_error() == ""


def _mat(n=1024, k=1024, version=w12.FORMAT_VERSION, n_esc=0, records=FAKE, esc=FAKE):
    return w12.MatrixC(n, k, records, FAKE + 0x100000, FAKE + 0x200000, esc, n_esc, version)


def _gemm(m, x=FAKE, M=1, ldx=None, y=FAKE, ldy=None, dt=w12.BF16, ws=FAKE, wsb=1 << 30):
    ldx = m.k if ldx is None else ldx
    ldy = m.n if ldy is None else ldy
    return w12.lib().w12_gemm(ctypes.byref(m), x, M, ldx, y, ldy, dt, ws, wsb, None)


def test_gemm_argument_errors():
    lib = w12.lib()
    assert lib.w12_gemm(None, FAKE, 1, 1024, FAKE, 1024, 0, FAKE, 1 << 20, None) == w12.E_INVALID_ARG
    assert _gemm(_mat(n=1000)) == w12.E_UNSUPPORTED_SHAPE
    assert _gemm(_mat(k=1000)) == w12.E_UNSUPPORTED_SHAPE
    assert _gemm(_mat(n=0)) == w12.E_UNSUPPORTED_SHAPE
    assert _gemm(_mat(version=2)) == w12.E_VERSION
    assert _gemm(_mat(), M=0) == w12.E_M_RANGE
    assert _gemm(_mat(), M=65) == w12.E_M_RANGE
    assert _gemm(_mat(), x=0) == w12.E_INVALID_ARG
    assert _gemm(_mat(), y=0) == w12.E_INVALID_ARG
    assert _gemm(_mat(), ldx=1000) == w12.E_INVALID_ARG
    assert _gemm(_mat(), ldx=1028) == w12.E_INVALID_ARG       # rows not 16-byte aligned
    assert _gemm(_mat(), x=FAKE + 2) == w12.E_INVALID_ARG
    assert _gemm(_mat(), ldy=1000) == w12.E_INVALID_ARG
    assert _gemm(_mat(), dt=7) == w12.E_INVALID_ARG
    assert _gemm(_mat(records=FAKE + 8)) == w12.E_INVALID_ARG
    assert _gemm(_mat(n_esc=5, esc=0)) == w12.E_INVALID_ARG
    assert _gemm(_mat(), ws=0) == w12.E_WORKSPACE
    assert _gemm(_mat(), wsb=16) == w12.E_WORKSPACE
    m = _mat()
    assert lib.w12_gemm_q8(ctypes.byref(m), FAKE, 1, 1024, FAKE, 1024, 0, 4, FAKE, 1 << 30, None) == w12.E_INVALID_ARG
    assert lib.w12_lmhead_argmax(ctypes.byref(m), FAKE, 70, 1024, FAKE, None, FAKE, 1 << 30, None) == w12.E_M_RANGE
    assert lib.w12_decode(ctypes.byref(_mat(k=100)), FAKE, None) == w12.E_UNSUPPORTED_SHAPE
    assert lib.w12_decode(ctypes.byref(m), 0, None) == w12.E_INVALID_ARG
    assert lib.w12_validate(ctypes.byref(m), 0, 0, None) == w12.E_WORKSPACE


def test_encode_argument_errors():
    lib = w12.lib()
    n_esc = ctypes.c_int64(0)
    assert lib.w12_encode_plan(FAKE, 1024, 1000, FAKE, FAKE, ctypes.byref(n_esc), FAKE, 1 << 20, None) == \
        w12.E_UNSUPPORTED_SHAPE
    assert lib.w12_encode_plan(0, 1024, 1024, FAKE, FAKE, ctypes.byref(n_esc), FAKE, 1 << 20, None) == \
        w12.E_INVALID_ARG
    assert lib.w12_encode_plan(FAKE, 1024, 1024, FAKE, FAKE, None, FAKE, 1 << 20, None) == w12.E_INVALID_ARG
    assert lib.w12_encode_plan(FAKE, 1024, 1024, FAKE, FAKE, ctypes.byref(n_esc), FAKE, 16, None) == \
        w12.E_WORKSPACE
    assert lib.w12_encode(FAKE, 16, 512, FAKE, FAKE, 0, FAKE, None) == w12.E_INVALID_ARG
    assert lib.w12_encode(FAKE + 4, 16, 512, FAKE, FAKE, FAKE, FAKE, None) == w12.E_INVALID_ARG
    # a matrix whose escape count could overflow 32-bit CSR offsets is refused
    assert lib.w12_encode(FAKE, 1 << 17, 1 << 16, FAKE, FAKE, FAKE, FAKE, None) == w12.E_UNSUPPORTED_SHAPE


def test_workspace_sizes():
    assert w12.workspace_bytes(w12.OP_ENCODE_PLAN, 17408, 5120) == 17408 * 4 + 0  # already 256-aligned
    assert w12.workspace_bytes(w12.OP_GEMM, 1000, 1024, 1) == 0            # bad shape
    assert w12.workspace_bytes(w12.OP_GEMM, 1024, 1024, 0) == 0            # bad M
    assert w12.workspace_bytes(99, 1024, 1024, 1) == 0
    for m in (1, 8, 15, 16, 32, 33, 64):
        g = w12.workspace_bytes(w12.OP_GEMM, 17408, 5120, m)
        a = w12.workspace_bytes(w12.OP_LMHEAD_ARGMAX, 17408, 5120, m)
        assert g > 0 and a > g and g % 256 == 0
    # the grid override changes the plan and therefore the size
    old = w12.set_tuning(w12.TUNE_GRID, 7)
    try:
        small = w12.workspace_bytes(w12.OP_GEMM, 17408, 5120, 32)
    finally:
        w12.set_tuning(w12.TUNE_GRID, old)
    assert 0 < small < w12.workspace_bytes(w12.OP_GEMM, 17408, 5120, 32)


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(w12, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(w12, "_lib", None)
    with pytest.raises(ImportError):
        w12.lib()
