"""Python binding of libw12 (include/w12.h).

Argument marshalling only: every step of encode, decode, GEMM, Q pass and
argmax runs in the library's HIP kernels. PyTorch provides device memory and
the current stream. The functions named like the C entry points take and
return torch tensors; ``encode``/``gemm``/``gemm_q8``/``lmhead_argmax``/
``decode`` are conveniences that allocate outputs and workspaces.

Importing this module loads libw12.so and fails loudly if it is missing:
there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw12.so")

# constants mirrored from include/w12.h
ABI_VERSION = 2
FORMAT_VERSION = 1
REC_ROWS, REC_COLS, REC_BYTES, REC_VIEW_BYTES = 16, 512, 12288, 8192
MAX_M = 64
NOALLOC_SCRATCH_BYTES = 16 << 20
WS_COUNTER_BYTES = 50432
OK, E_INVALID_ARG, E_UNSUPPORTED_SHAPE, E_M_RANGE, E_WORKSPACE, E_VERSION, E_HIP, E_NOT_IMPLEMENTED, E_CORRUPT = (
    0, -1, -2, -3, -4, -5, -6, -7, -8)
BF16, F32 = 0, 1
OP_ENCODE_PLAN, OP_GEMM, OP_GEMM_Q8, OP_LMHEAD_ARGMAX, OP_LMHEAD_CERTIFIED = 1, 2, 3, 4, 5
CERT_MAX_SURVIVORS = 256
Q8_APPLY_ESCAPES = 1
TUNE_PATH, TUNE_GRID = 1, 2
PATH_DENSE = 4          # W12_TUNE_PATH value forcing the dense-escape path
KERNEL_GEMV, KERNEL_MFMA_HELPER, KERNEL_MFMA_STREAM = 1, 2, 3
KERNEL_NAMES = {KERNEL_GEMV: "gemv", KERNEL_MFMA_HELPER: "mfma_helper", KERNEL_MFMA_STREAM: "mfma_stream"}


class W12Error(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = f"{where}: {status_str(status)} ({status})"
        if status == E_HIP:
            msg += f": {last_error()}"
        super().__init__(msg)
        self.status = status


class EscapeC(ctypes.Structure):
    _fields_ = [("col", ctypes.c_uint32), ("bits", ctypes.c_uint16), ("ph", ctypes.c_uint16)]


class MatrixC(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("k", ctypes.c_int64), ("records", ctypes.c_void_p),
                ("e_top", ctypes.c_void_p), ("esc_row_ptr", ctypes.c_void_p), ("esc", ctypes.c_void_p),
                ("n_esc", ctypes.c_int64), ("format_version", ctypes.c_uint32)]


class PlanC(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("grid", ctypes.c_int32), ("threads", ctypes.c_int32),
                ("tile_rows", ctypes.c_int32), ("whole_tiles", ctypes.c_int32), ("split_tiles", ctypes.c_int32),
                ("split_tile_rows", ctypes.c_int32), ("unit_cols", ctypes.c_int32), ("split_units", ctypes.c_int64),
                ("prepass", ctypes.c_int32), ("fixup", ctypes.c_int32), ("workspace_bytes", ctypes.c_size_t)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_SIGNATURES = {
    "w12_abi_version": (ctypes.c_int, []),
    "w12_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "w12_last_error": (ctypes.c_char_p, []),
    "w12_workspace_bytes": (_SZ, [ctypes.c_int, _I64, _I64, _I64]),
    "w12_encode_plan": (ctypes.c_int, [_P, _I64, _I64, _P, _P, ctypes.POINTER(_I64), _P, _SZ, _P]),
    "w12_encode": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P, _P, _I64, _P]),
    "w12_decode": (ctypes.c_int, [ctypes.POINTER(MatrixC), _P, _P]),
    "w12_gemm": (ctypes.c_int, [ctypes.POINTER(MatrixC), _P, _I64, _I64, _P, _I64, ctypes.c_int, _P, _SZ, _P]),
    "w12_certify_bounds": (ctypes.c_int, [ctypes.POINTER(MatrixC), _P, _P]),
    "w12_lmhead_argmax_certified": (ctypes.c_int, [ctypes.POINTER(MatrixC), _P, _P, _I64, _I64, _P, _P, _P, _P,
                                                   _SZ, _P]),
    "w12_gemm_noalloc": (ctypes.c_int, [ctypes.POINTER(MatrixC), _P, _I64, _I64, _P, _I64, ctypes.c_int, _P]),
    "w12_gemm_q8": (ctypes.c_int, [ctypes.POINTER(MatrixC), _P, _I64, _I64, _P, _I64, ctypes.c_int,
                                   ctypes.c_uint32, _P, _SZ, _P]),
    "w12_lmhead_argmax": (ctypes.c_int, [ctypes.POINTER(MatrixC), _P, _I64, _I64, _P, _P, _P, _SZ, _P]),
    "w12_validate": (ctypes.c_int, [ctypes.POINTER(MatrixC), _P, _SZ, _P]),
    "w12_set_tuning": (_I64, [ctypes.c_int, _I64]),
    "w12_plan_info": (ctypes.c_int, [ctypes.POINTER(MatrixC), ctypes.c_int, _I64, ctypes.c_uint32,
                                     ctypes.POINTER(PlanC)]),
    # include/w12_probe.h
    "w12_probe_read": (ctypes.c_int, [_P, _SZ, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _SZ,
                                      ctypes.c_int, _P, _P, _SZ, _P]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libw12.so (built by ``lossless_compressed_weight_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m lossless_compressed_weight_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        if handle.w12_abi_version() != ABI_VERSION:
            raise ImportError("libw12.so ABI version mismatch")
        _lib = handle
    return _lib


def status_str(status: int) -> str:
    return lib().w12_status_str(status).decode()


def last_error() -> str:
    return lib().w12_last_error().decode()


def _check(status: int, where: str):
    if status != OK:
        raise W12Error(status, where)


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def set_tuning(key: int, value: int) -> int:
    return int(lib().w12_set_tuning(key, value))


def plan_info(mat_or_desc, op: int, m: int, flags: int = 0) -> dict:
    """The plan the library would run (w12_plan_info): a dict of the w12_plan
    fields plus the kernel's name. Host-only; accepts a W12Matrix or a
    MatrixC descriptor (only n, k and n_esc are read)."""
    d = mat_or_desc.desc() if hasattr(mat_or_desc, "desc") else mat_or_desc
    out = PlanC()
    _check(lib().w12_plan_info(ctypes.byref(d), op, m, flags, ctypes.byref(out)), "w12_plan_info")
    rec = {f: getattr(out, f) for f, _ in PlanC._fields_}
    rec["kernel_name"] = KERNEL_NAMES.get(out.kernel, "?")
    return rec


def workspace_bytes(op: int, n: int, k: int, m: int = 0) -> int:
    return int(lib().w12_workspace_bytes(op, n, k, m))


def new_workspace(op: int, n: int, k: int, m: int = 0, device="cuda") -> torch.Tensor:
    """A zero-filled workspace for `op` (the GEMM ops need their counter words
    zero before the first call; every call leaves them zero again)."""
    nb = workspace_bytes(op, n, k, m)
    return torch.zeros(max(nb, 1), dtype=torch.uint8, device=device)


def _workspace(op, n, k, m, device):
    ws = new_workspace(op, n, k, m, device)
    return ws, ws.numel()


@dataclass
class W12Matrix:
    """An encoded matrix: device tensors plus sizes (format v1)."""
    n: int
    k: int
    records: torch.Tensor   # uint8 [(n/16)(k/512) * 12288]
    e_top: torch.Tensor     # uint8 [n]
    row_ptr: torch.Tensor   # int32 [n + 1] (bit pattern of uint32)
    esc: torch.Tensor       # int64 [n_esc] (bit pattern of the 8-byte entries)
    n_esc: int

    def desc(self) -> MatrixC:
        return MatrixC(self.n, self.k, self.records.data_ptr(), self.e_top.data_ptr(), self.row_ptr.data_ptr(),
                       self.esc.data_ptr() if self.n_esc > 0 else 0, self.n_esc, FORMAT_VERSION)

    @property
    def device(self):
        return self.records.device

    def nbytes(self) -> int:
        return self.records.numel() + self.e_top.numel() + 4 * self.row_ptr.numel() + 8 * self.n_esc


def _as_bits16(t: torch.Tensor) -> torch.Tensor:
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return t
    raise TypeError(f"expected BF16 data (bfloat16, int16 or uint16 tensor), got {t.dtype}")


def _on(mat: "W12Matrix", t: torch.Tensor, what: str):
    if not t.is_cuda or t.device != mat.device:
        raise ValueError(f"{what} must live on the matrix's device {mat.device}, got {t.device}")


def _check_x(mat: "W12Matrix", x: torch.Tensor):
    """Activations: BF16 bits, [M, K] with unit column stride, on mat's device."""
    _as_bits16(x)
    _on(mat, x, "x")
    if x.dim() != 2 or x.shape[1] != mat.k or (x.shape[0] > 0 and x.stride(1) != 1):
        raise ValueError(f"x must be [M, {mat.k}] with unit column stride, got {tuple(x.shape)} "
                         f"strides {tuple(x.stride())}")


def _check_y(mat: "W12Matrix", y: torch.Tensor, m: int) -> int:
    """Output: float32 or bfloat16 [M, N] with unit column stride; returns its dtype code."""
    if y.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"y must be float32 or bfloat16, got {y.dtype}")
    _on(mat, y, "y")
    if y.dim() != 2 or tuple(y.shape) != (m, mat.n) or (m > 0 and y.stride(1) != 1):
        raise ValueError(f"y must be [{m}, {mat.n}] with unit column stride, got {tuple(y.shape)} "
                         f"strides {tuple(y.stride())}")
    return F32 if y.dtype == torch.float32 else BF16


def _check_ws(mat: "W12Matrix", ws: torch.Tensor):
    _on(mat, ws, "workspace")
    if ws.dtype != torch.uint8 or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")


# ---------------------------------------------------------------- C-named calls
def w12_encode_plan(w: torch.Tensor, e_top: torch.Tensor, row_ptr: torch.Tensor, ws: torch.Tensor,
                    stream=None) -> int:
    n, k = w.shape
    n_esc = _I64(0)
    _check(lib().w12_encode_plan(_ptr(w), n, k, _ptr(e_top), _ptr(row_ptr), ctypes.byref(n_esc), _ptr(ws),
                                 ws.numel(), _stream(stream)), "w12_encode_plan")
    return int(n_esc.value)


def w12_encode(w, e_top, row_ptr, records, esc, stream=None, n_esc=None):
    """esc: int64 device tensor of at least n_esc entries (n_esc: the count
    w12_encode_plan returned; default: all of esc), or None when it is 0."""
    n, k = w.shape
    cap = 0 if esc is None else (esc.numel() if n_esc is None else n_esc)
    if esc is not None and (esc.dtype != torch.int64 or not esc.is_cuda or esc.numel() < cap):
        raise ValueError("esc must be an int64 device tensor with room for the escape entries")
    _check(lib().w12_encode(_ptr(w), n, k, _ptr(e_top), _ptr(row_ptr), _ptr(records),
                            _ptr(esc) if cap else ctypes.c_void_p(0), cap, _stream(stream)), "w12_encode")


def w12_decode(mat: W12Matrix, out: torch.Tensor, stream=None):
    _on(mat, out, "out")
    if out.element_size() != 2 or not out.is_contiguous() or out.numel() != mat.n * mat.k:
        raise ValueError(f"out must be a contiguous 16-bit tensor of {mat.n} x {mat.k} elements")
    d = mat.desc()
    _check(lib().w12_decode(ctypes.byref(d), _ptr(out), _stream(stream)), "w12_decode")


def w12_gemm(mat: W12Matrix, x, y, ws, stream=None):
    _check_x(mat, x)
    ydt = _check_y(mat, y, x.shape[0])
    _check_ws(mat, ws)
    d = mat.desc()
    _check(lib().w12_gemm(ctypes.byref(d), _ptr(x), x.shape[0], x.stride(0), _ptr(y), y.stride(0), ydt,
                          _ptr(ws), ws.numel(), _stream(stream)), "w12_gemm")


def w12_gemm_noalloc(mat: W12Matrix, x, y, stream=None):
    """w12_gemm on the library's static per-device scratch (no workspace)."""
    _check_x(mat, x)
    ydt = _check_y(mat, y, x.shape[0])
    d = mat.desc()
    _check(lib().w12_gemm_noalloc(ctypes.byref(d), _ptr(x), x.shape[0], x.stride(0), _ptr(y), y.stride(0), ydt,
                                  _stream(stream)), "w12_gemm_noalloc")


def w12_gemm_q8(mat: W12Matrix, x, y, flags, ws, stream=None):
    _check_x(mat, x)
    ydt = _check_y(mat, y, x.shape[0])
    _check_ws(mat, ws)
    d = mat.desc()
    _check(lib().w12_gemm_q8(ctypes.byref(d), _ptr(x), x.shape[0], x.stride(0), _ptr(y), y.stride(0), ydt,
                             flags, _ptr(ws), ws.numel(), _stream(stream)), "w12_gemm_q8")


def w12_lmhead_argmax(mat: W12Matrix, x, idx, max_logit, ws, stream=None):
    _check_x(mat, x)
    m = x.shape[0]
    _on(mat, idx, "idx")
    if idx.dtype != torch.int32 or idx.numel() < m or not idx.is_contiguous():
        raise ValueError("idx must be a contiguous int32 tensor of M entries")
    if max_logit is not None:       # optional: NULL skips the maximum logits
        _on(mat, max_logit, "max_logit")
        if max_logit.dtype != torch.float32 or max_logit.numel() < m or not max_logit.is_contiguous():
            raise ValueError("max_logit must be a contiguous float32 tensor of M entries")
    _check_ws(mat, ws)
    d = mat.desc()
    _check(lib().w12_lmhead_argmax(ctypes.byref(d), _ptr(x), x.shape[0], x.stride(0), _ptr(idx), _ptr(max_logit),
                                   _ptr(ws), ws.numel(), _stream(stream)), "w12_lmhead_argmax")


def w12_certify_bounds(mat: W12Matrix, bounds: torch.Tensor, stream=None):
    _on(mat, bounds, "bounds")
    if bounds.dtype != torch.float32 or bounds.numel() < 2 * mat.n or not bounds.is_contiguous():
        raise ValueError(f"bounds must be a contiguous float32 tensor of 2 * {mat.n} entries")
    d = mat.desc()
    _check(lib().w12_certify_bounds(ctypes.byref(d), _ptr(bounds), _stream(stream)), "w12_certify_bounds")


def w12_lmhead_argmax_certified(mat: W12Matrix, bounds, x, idx, max_logit, survivors, ws, stream=None):
    _check_x(mat, x)
    m = x.shape[0]
    for t, name, dt in ((idx, "idx", torch.int32), (max_logit, "max_logit", torch.float32),
                        (survivors, "survivors", torch.int32)):
        if t is None and name == "idx":
            raise ValueError("idx is required")
        if t is not None:
            _on(mat, t, name)
            if t.dtype != dt or t.numel() < m or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous {dt} tensor of M entries")
    _on(mat, bounds, "bounds")
    if bounds.dtype != torch.float32 or bounds.numel() < 2 * mat.n:
        raise ValueError("bounds must come from w12_certify_bounds (float32, 2 N entries)")
    _check_ws(mat, ws)
    d = mat.desc()
    _check(lib().w12_lmhead_argmax_certified(ctypes.byref(d), _ptr(bounds), _ptr(x), m, x.stride(0), _ptr(idx),
                                             _ptr(max_logit), _ptr(survivors), _ptr(ws), ws.numel(),
                                             _stream(stream)), "w12_lmhead_argmax_certified")


def w12_validate(mat: W12Matrix, ws: torch.Tensor, stream=None) -> int:
    _check_ws(mat, ws)
    d = mat.desc()
    return int(lib().w12_validate(ctypes.byref(d), _ptr(ws), ws.numel(), _stream(stream)))


PROBE_STATIC, PROBE_DYNAMIC, PROBE_STRIDE, PROBE_PIECES = 0, 1, 2, 3
PROBE_WS_BYTES = 256


def w12_probe_read(buf: torch.Tensor, nbytes: int, grid: int, block: int, loads: int, mode: int,
                   stamps, ws: torch.Tensor, stream=None, lds_bytes: int = 0, piece: int = 0):
    """Read-bandwidth probe (include/w12_probe.h) over the first `nbytes` of `buf`."""
    if not buf.is_cuda or nbytes > buf.numel() * buf.element_size():
        raise ValueError("probe buffer must be a device tensor holding nbytes")
    if stamps is not None and (not stamps.is_cuda or stamps.numel() < 3 * grid or stamps.element_size() != 8):
        raise ValueError("stamps must be a device tensor of 3 * grid 64-bit entries")
    _check(lib().w12_probe_read(_ptr(buf), nbytes, grid, block, loads, mode, piece, lds_bytes, _ptr(stamps),
                                _ptr(ws), ws.numel(), _stream(stream)), "w12_probe_read")


# ---------------------------------------------------------------- conveniences
def encode(w: torch.Tensor, stream=None) -> W12Matrix:
    """Encode a BF16 matrix [N, K] that lives on a GPU."""
    w = _as_bits16(w)
    if w.dim() != 2 or not w.is_contiguous():
        raise ValueError("w must be a contiguous 2-D tensor")
    n, k = w.shape
    dev = w.device
    e_top = torch.empty(n, dtype=torch.uint8, device=dev)
    row_ptr = torch.empty(n + 1, dtype=torch.int32, device=dev)
    ws, _ = _workspace(OP_ENCODE_PLAN, n, k, 0, dev)
    n_esc = w12_encode_plan(w, e_top, row_ptr, ws, stream)
    records = torch.empty((n // REC_ROWS) * (k // REC_COLS) * REC_BYTES, dtype=torch.uint8, device=dev)
    esc = torch.empty(max(n_esc, 1), dtype=torch.int64, device=dev)
    w12_encode(w, e_top, row_ptr, records, esc if n_esc else None, stream, n_esc=n_esc)
    return W12Matrix(n, k, records, e_top, row_ptr, esc[:n_esc], n_esc)


def decode(mat: W12Matrix, stream=None) -> torch.Tensor:
    out = torch.empty((mat.n, mat.k), dtype=torch.bfloat16, device=mat.device)
    w12_decode(mat, out, stream)
    return out


def gemm(mat: W12Matrix, x: torch.Tensor, out_dtype=torch.bfloat16, stream=None) -> torch.Tensor:
    x = _as_bits16(x)
    y = torch.empty((x.shape[0], mat.n), dtype=out_dtype, device=mat.device)
    ws, _ = _workspace(OP_GEMM, mat.n, mat.k, x.shape[0], mat.device)
    w12_gemm(mat, x, y, ws, stream)
    return y


def gemm_q8(mat: W12Matrix, x: torch.Tensor, out_dtype=torch.bfloat16, apply_escapes=False,
            stream=None) -> torch.Tensor:
    x = _as_bits16(x)
    y = torch.empty((x.shape[0], mat.n), dtype=out_dtype, device=mat.device)
    ws, _ = _workspace(OP_GEMM_Q8, mat.n, mat.k, x.shape[0], mat.device)
    w12_gemm_q8(mat, x, y, Q8_APPLY_ESCAPES if apply_escapes else 0, ws, stream)
    return y


def lmhead_argmax(mat: W12Matrix, x: torch.Tensor, stream=None):
    x = _as_bits16(x)
    m = x.shape[0]
    idx = torch.empty(m, dtype=torch.int32, device=mat.device)
    mx = torch.empty(m, dtype=torch.float32, device=mat.device)
    ws, _ = _workspace(OP_LMHEAD_ARGMAX, mat.n, mat.k, m, mat.device)
    w12_lmhead_argmax(mat, x, idx, mx, ws, stream)
    return idx, mx


def certify_bounds(mat: W12Matrix, stream=None) -> torch.Tensor:
    """Per-row bounds [N, 2] (r_n, a_n) of the certified LM head."""
    b = torch.empty((mat.n, 2), dtype=torch.float32, device=mat.device)
    w12_certify_bounds(mat, b, stream)
    return b


def lmhead_argmax_certified(mat: W12Matrix, bounds: torch.Tensor, x: torch.Tensor, stream=None):
    """(idx, max_logit, survivors) of the certified argmax LM head."""
    x = _as_bits16(x)
    m = x.shape[0]
    idx = torch.empty(m, dtype=torch.int32, device=mat.device)
    mx = torch.empty(m, dtype=torch.float32, device=mat.device)
    sv = torch.empty(m, dtype=torch.int32, device=mat.device)
    ws, _ = _workspace(OP_LMHEAD_CERTIFIED, mat.n, mat.k, m, mat.device)
    w12_lmhead_argmax_certified(mat, bounds, x, idx, mx, sv, ws, stream)
    return idx, mx, sv
