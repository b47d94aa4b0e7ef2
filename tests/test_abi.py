"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/w12.h declares, and rejects bad arguments with the
documented status codes before touching the GPU."""
import ctypes
import os
import re

import pytest

from lossless_compressed_weight_amd import w12

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

# Fake, 256-byte aligned device addresses: argument checks must reject the
# calls below before any HIP call could dereference them.
FAKE = 0x7F0000000000


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*[A-Za-z_][\w \*]*?\b(w12_\w+)\s*\(", text, flags=re.M))
    return sorted(names)


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
    assert lib.w12_encode(FAKE, 16, 512, FAKE, FAKE, 0, FAKE, 8, None) == w12.E_INVALID_ARG
    assert lib.w12_encode(FAKE + 4, 16, 512, FAKE, FAKE, FAKE, FAKE, 8, None) == w12.E_INVALID_ARG
    # escapes need a buffer: NULL esc with a nonzero capacity, or a bad capacity, is refused
    assert lib.w12_encode(FAKE, 16, 512, FAKE, FAKE, FAKE, None, 3, None) == w12.E_INVALID_ARG
    assert lib.w12_encode(FAKE, 16, 512, FAKE, FAKE, FAKE, FAKE, -1, None) == w12.E_INVALID_ARG
    assert lib.w12_encode(FAKE, 16, 512, FAKE, FAKE, FAKE, FAKE, 16 * 512 + 1, None) == w12.E_INVALID_ARG
    # a matrix whose escape count could overflow 32-bit CSR offsets is refused
    assert lib.w12_encode(FAKE, 1 << 17, 1 << 16, FAKE, FAKE, FAKE, FAKE, 8, None) == w12.E_UNSUPPORTED_SHAPE


def test_workspace_sizes():
    assert w12.workspace_bytes(w12.OP_ENCODE_PLAN, 17408, 5120) == 17408 * 4 + 0  # already 256-aligned
    assert w12.workspace_bytes(w12.OP_GEMM, 1000, 1024, 1) == 0            # bad shape
    assert w12.workspace_bytes(w12.OP_GEMM, 1024, 1024, 0) == 0            # bad M
    assert w12.workspace_bytes(99, 1024, 1024, 1) == 0
    for m in (1, 8, 15, 16, 32, 33, 64):
        for op in (w12.OP_GEMM, w12.OP_GEMM_Q8, w12.OP_LMHEAD_ARGMAX):
            b = w12.workspace_bytes(op, 17408, 5120, m)
            assert b > 0 and b % 256 == 0
            # whichever kernel the escape density selects, its plan fits
            for n_esc in (0, 24000, 17408 * 100):
                plan = w12.plan_info(_mat(17408, 5120, n_esc=n_esc), op, m)
                assert plan["workspace_bytes"] <= b, (op, m, n_esc, plan)
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


def _plan_covers_rows(plan, n):
    """Whole tiles and split tiles of a plan cover rows [0, n) exactly once."""
    whole_rows = plan["grid"] * plan["whole_tiles"] * plan["tile_rows"]
    split_rows = plan["split_tiles"] * plan["split_tile_rows"]
    if plan["split_tiles"] == 0:
        assert whole_rows >= n and whole_rows - n < plan["tile_rows"], plan
    else:
        assert whole_rows < n and whole_rows + split_rows >= n, plan
        assert whole_rows + split_rows - n < plan["split_tile_rows"], plan
    assert plan["split_units"] == plan["split_tiles"] * (plan["split_units"] // max(plan["split_tiles"], 1))
    assert plan["split_tiles"] >= 0 and plan["split_units"] >= 0 and plan["whole_tiles"] >= 0


@pytest.mark.parametrize("n,k,m", [
    (12784, 5120, 32), (4112, 5120, 64), (16336, 4096, 8), (16336, 4096, 1),   # last whole tile cut short by N
    (17408, 5120, 1), (17408, 5120, 32), (5120, 17408, 32), (1024, 5120, 64),
    (151936, 5120, 16), (6144, 5120, 48), (16, 512, 3), (48, 1024, 40),
])
def test_plan_arithmetic(n, k, m):
    """Host-side plan of every op: no negative split counts, every row covered
    exactly once, a grid within [1, 4096] and no larger than the work units."""
    for op in (w12.OP_GEMM, w12.OP_GEMM_Q8, w12.OP_LMHEAD_ARGMAX):
        for n_esc in (0, n * 2, n * 50):
            plan = w12.plan_info(_mat(n, k, n_esc=n_esc), op, m)
            assert 1 <= plan["grid"] <= 4096
            units = -(-n // plan["tile_rows"]) * (k // plan["unit_cols"])
            assert plan["grid"] <= units
            _plan_covers_rows(plan, n)
            # dense escapes: the GEMM runs without escape work, a fix-up kernel follows
            dense = n_esc > 8 * n and op == w12.OP_GEMM
            assert plan["fixup"] == int(dense)
            if op == w12.OP_LMHEAD_ARGMAX:
                assert plan["kernel"] in (w12.KERNEL_GEMV, w12.KERNEL_MFMA_HELPER)
            if m <= 2:
                assert plan["kernel"] == w12.KERNEL_GEMV
            elif (tiles := -(-(n // 16) // 4)) < 256 and op != w12.OP_LMHEAD_ARGMAX and (m > 16 or (tiles >= 32 and k <= 8192)):
                assert plan["kernel"] == w12.KERNEL_MFMA_STREAM and plan["prepass"] == int(dense)
            else:
                assert plan["kernel"] == w12.KERNEL_MFMA_HELPER


@pytest.mark.parametrize("m", [3, 8, 16, 17, 32])
def test_helper_prepass_rule(m):
    """Whether the helper-wave MFMA kernel's activation pre-pass runs: always
    beyond 16 activation rows (the operand-order copy); up to 16 rows only
    for the transposed copy, when escapes are many per row (escape lines
    above 16 per row) and more than 256 per workgroup."""
    n, k = 17408, 5120   # 272 tiles: the helper-wave kernel at every M from 3
    for op, flags in ((w12.OP_GEMM, 0), (w12.OP_GEMM_Q8, 0), (w12.OP_GEMM_Q8, w12.Q8_APPLY_ESCAPES),
                      (w12.OP_LMHEAD_ARGMAX, 0)):
        fix = op != w12.OP_GEMM_Q8 or flags != 0
        for n_esc in (0, 2000, 24000, 100000):
            plan = w12.plan_info(_mat(n, k, n_esc=n_esc), op, m, flags)
            assert plan["kernel"] == w12.KERNEL_MFMA_HELPER, plan
            many_lines = fix and n_esc * 16 * -(-m // 16) > 16 * n
            want = m > 16 or (many_lines and n_esc > 256 * plan["grid"])
            assert plan["prepass"] == int(want), (op, flags, n_esc, m, plan)


@pytest.mark.parametrize("path,n,k", [
    (2, 12784, 5120),   # helper-wave kernel: 799 row blocks in 200 tiles on 200 workgroups
    (3, 16368, 1024),   # stream kernel: 1023 row blocks in 256 tiles on 256 workgroups
])
def test_plan_of_whole_tiles_past_n_has_no_split_tiles(path, n, k):
    """Whole tiles that already reach past N (the last one cut short) leave no
    rows to split (a negative remainder once sent the kernel past N)."""
    old = w12.set_tuning(w12.TUNE_PATH, path)
    try:
        plan = w12.plan_info(_mat(n, k), w12.OP_GEMM, 32)
    finally:
        w12.set_tuning(w12.TUNE_PATH, old)
    assert plan["whole_tiles"] == 1 and plan["split_tiles"] == 0 and plan["split_units"] == 0, plan
    assert plan["grid"] * plan["whole_tiles"] * plan["tile_rows"] >= n


def test_plan_info_argument_errors():
    assert w12.lib().w12_plan_info(None, w12.OP_GEMM, 1, 0, None) == w12.E_INVALID_ARG
    out = w12.PlanC()
    lib = w12.lib()
    assert lib.w12_plan_info(ctypes.byref(_mat(n=1000)), w12.OP_GEMM, 1, 0, ctypes.byref(out)) == \
        w12.E_UNSUPPORTED_SHAPE
    assert lib.w12_plan_info(ctypes.byref(_mat()), 99, 1, 0, ctypes.byref(out)) == w12.E_INVALID_ARG
    assert lib.w12_plan_info(ctypes.byref(_mat()), w12.OP_GEMM, 65, 0, ctypes.byref(out)) == w12.E_M_RANGE
    assert lib.w12_plan_info(ctypes.byref(_mat()), w12.OP_GEMM_Q8, 1, 8, ctypes.byref(out)) == w12.E_INVALID_ARG


def test_tuning_hooks_are_per_thread():
    """A tuning hook set on one thread leaves another thread's plans alone."""
    import threading
    base = w12.plan_info(_mat(17408, 5120), w12.OP_GEMM, 32)
    seen = {}

    def other():
        seen["plan"] = w12.plan_info(_mat(17408, 5120), w12.OP_GEMM, 32)

    old = w12.set_tuning(w12.TUNE_GRID, 7)
    try:
        assert w12.plan_info(_mat(17408, 5120), w12.OP_GEMM, 32)["grid"] == 7
        th = threading.Thread(target=other)
        th.start()
        th.join()
    finally:
        w12.set_tuning(w12.TUNE_GRID, old)
    assert seen["plan"] == base


def test_wrappers_check_tensors_before_calling():
    """The Python wrappers refuse host tensors, wrong dtypes and wrong shapes
    before anything reaches the library (nothing here touches a GPU)."""
    import torch
    mat = w12.W12Matrix(32, 512, torch.zeros(2 * w12.REC_BYTES, dtype=torch.uint8),
                        torch.zeros(32, dtype=torch.uint8), torch.zeros(33, dtype=torch.int32),
                        torch.zeros(1, dtype=torch.int64), 0)
    x = torch.zeros((4, 512), dtype=torch.bfloat16)
    y = torch.zeros((4, 32), dtype=torch.float32)
    ws = torch.zeros(1024, dtype=torch.uint8)
    with pytest.raises(ValueError, match="device"):
        w12.w12_gemm(mat, x, y, ws)
    with pytest.raises(ValueError, match="device"):
        w12.w12_gemm_q8(mat, x, y, 0, ws)
    with pytest.raises(ValueError, match="device"):
        w12.w12_lmhead_argmax(mat, x, torch.zeros(4, dtype=torch.int32), None, ws)
    with pytest.raises(TypeError):
        w12.w12_gemm(mat, torch.zeros((4, 512), dtype=torch.float32), y, ws)
    with pytest.raises(ValueError, match="device"):
        w12.w12_decode(mat, torch.zeros((32, 512), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="int64"):
        w12.w12_encode(torch.zeros((32, 512), dtype=torch.int16), None, None, None,
                       torch.zeros(4, dtype=torch.int32))


def test_noalloc_refuses_shapes_beyond_its_scratch():
    """w12_gemm_noalloc checks its arguments and the workspace the shape needs
    against the static scratch before any HIP call (fake pointers: nothing
    may be launched)."""
    lib = w12.lib()
    big_k = 1 << 20
    assert w12.workspace_bytes(w12.OP_GEMM, 16, big_k, 64) > w12.NOALLOC_SCRATCH_BYTES
    m = w12.MatrixC(16, big_k, FAKE, FAKE, FAKE, 0, 0, w12.FORMAT_VERSION)
    assert lib.w12_gemm_noalloc(ctypes.byref(m), FAKE, 64, big_k, FAKE, 16, w12.F32, None) == w12.E_WORKSPACE
    assert b"scratch" in lib.w12_last_error()
    m = w12.MatrixC(1024, 1024, FAKE, FAKE, FAKE, 0, 0, w12.FORMAT_VERSION)
    assert lib.w12_gemm_noalloc(ctypes.byref(m), FAKE, 0, 1024, FAKE, 1024, w12.F32, None) == w12.E_M_RANGE
    assert lib.w12_gemm_noalloc(ctypes.byref(m), FAKE, 4, 1000, FAKE, 1024, w12.F32, None) == w12.E_INVALID_ARG
    assert lib.w12_gemm_noalloc(None, FAKE, 4, 1024, FAKE, 1024, w12.F32, None) == w12.E_INVALID_ARG


def test_certified_head_argument_errors():
    """The certified LM head checks its arguments and workspace before any HIP
    call (fake pointers: nothing may be launched)."""
    lib = w12.lib()
    m = w12.MatrixC(151936, 5120, FAKE, FAKE, FAKE, 0, 0, w12.FORMAT_VERSION)
    need = w12.workspace_bytes(w12.OP_LMHEAD_CERTIFIED, 151936, 5120, 32)
    assert need > 32 * 151936 * 4                       # holds the Q logits
    assert need >= w12.workspace_bytes(w12.OP_LMHEAD_ARGMAX, 151936, 5120, 32)
    call = lambda b, mm, ws_bytes: lib.w12_lmhead_argmax_certified(  # noqa: E731
        ctypes.byref(m), b, FAKE, mm, 5120, FAKE, None, None, FAKE, ws_bytes, None)
    assert call(FAKE, 32, need - 1) == w12.E_WORKSPACE
    assert call(None, 32, need) == w12.E_INVALID_ARG
    assert call(FAKE, 0, need) == w12.E_M_RANGE
    assert call(FAKE, 65, need) == w12.E_M_RANGE
    assert lib.w12_certify_bounds(ctypes.byref(m), None, None) == w12.E_INVALID_ARG
    assert lib.w12_certify_bounds(ctypes.byref(m), FAKE + 4, None) == w12.E_INVALID_ARG
    bad = w12.MatrixC(151936, 5120, FAKE, FAKE, FAKE, 0, 0, 99)
    assert lib.w12_certify_bounds(ctypes.byref(bad), FAKE, None) == w12.E_VERSION
