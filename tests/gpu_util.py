"""Helpers shared by the GPU parity tests: moving BF16 bit arrays between
NumPy and the device, uploading oracle encodings, and the tolerance checks.

Tolerance (the GEMM is fp32 accumulation over BF16 inputs, compared with the
oracle's float64 product y64): with fp32 output, every element must satisfy
    |y - y64| <= 2e-3 * max(|y64|, 1e-3 * s_m),
where s_m is the largest |y64| in the checked part of row m (the floor keeps
elements that cancel to near zero from demanding a relative accuracy no fp32
sum can give); with BF16 output, y must equal the round-to-nearest-even of the
same call's fp32 output and lie within (2e-3 + 2^-8) of y64 on that scale.
"""
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle as o  # noqa: E402
from lossless_compressed_weight_amd import w12  # noqa: E402

REL = 2e-3
FLOOR = 1e-3
BF16_ULP = 2.0 ** -8


def log(msg):
    print(msg, flush=True)


def dev16(a: np.ndarray) -> torch.Tensor:
    """uint16 NumPy array -> int16 CUDA tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def host16(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def upload(enc: "o.Encoded") -> w12.W12Matrix:
    """A device W12Matrix holding the oracle's encoding."""
    rec = torch.from_numpy(enc.records.copy()).cuda()
    e_top = torch.from_numpy(enc.e_top.copy()).cuda()
    row_ptr = torch.from_numpy(enc.row_ptr.view(np.int32).copy()).cuda()
    esc = torch.from_numpy(enc.esc.view(np.int64).copy() if enc.n_esc else np.zeros(1, np.int64)).cuda()
    return w12.W12Matrix(enc.n, enc.k, rec, e_top, row_ptr, esc[:enc.n_esc], enc.n_esc)


def download(mat: w12.W12Matrix):
    """(records, e_top, row_ptr, esc) of a device matrix as NumPy arrays."""
    rec = mat.records.cpu().numpy()
    e_top = mat.e_top.cpu().numpy()
    row_ptr = mat.row_ptr.cpu().numpy().view(np.uint32)
    esc = mat.esc.cpu().numpy().view(o.ESC_DTYPE) if mat.n_esc else np.zeros(0, o.ESC_DTYPE)
    return rec, e_top, row_ptr, esc



def check_f32(y: np.ndarray, y64: np.ndarray, what: str):
    y = np.asarray(y, dtype=np.float64)
    s = np.max(np.abs(y64), axis=1, keepdims=True)
    denom = np.maximum(np.abs(y64), FLOOR * s)
    err = np.abs(y - y64) / np.where(denom > 0, denom, 1.0)
    worst = float(err.max()) if err.size else 0.0
    assert worst <= REL, f"{what}: max scaled error {worst:.3e} > {REL}"
    return worst


def check_bf16(y_bf16_bits: np.ndarray, y_f32: np.ndarray, y64: np.ndarray, what: str):
    assert np.array_equal(y_bf16_bits, o.f64_to_bf16_rne(np.asarray(y_f32, dtype=np.float64))), \
        f"{what}: BF16 output is not the RNE of the fp32 output"
    yb = o.bf16_to_f64(y_bf16_bits)
    s = np.max(np.abs(y64), axis=1, keepdims=True)
    denom = np.maximum(np.abs(y64), FLOOR * s)
    err = np.abs(yb - y64) / np.where(denom > 0, denom, 1.0)
    assert float(err.max()) <= REL + BF16_ULP, f"{what}: BF16 error {float(err.max()):.3e}"


def check_bf16_value(y_bf16_bits: np.ndarray, y64: np.ndarray, what: str):
    """A BF16 output on its own (no fp32 twin): within (2e-3 + 2^-8) of y64."""
    yb = o.bf16_to_f64(y_bf16_bits)
    s = np.max(np.abs(y64), axis=1, keepdims=True)
    denom = np.maximum(np.abs(y64), FLOOR * s)
    err = np.abs(yb - y64) / np.where(denom > 0, denom, 1.0)
    assert float(err.max()) <= REL + BF16_ULP, f"{what}: BF16 error {float(err.max()):.3e}"


def argmax_logits_f32(mat, x_dev):
    """fp32 logits from the kernel the fused argmax runs (the helper-wave MFMA
    kernel from 3 activation rows, the GEMV below), so that the argmax can be
    compared with them bit for bit."""
    m = x_dev.shape[0]
    old = w12.set_tuning(w12.TUNE_PATH, w12.KERNEL_MFMA_HELPER if m >= 3 else 0)
    try:
        return w12.gemm(mat, x_dev, torch.float32)
    finally:
        w12.set_tuning(w12.TUNE_PATH, old)


def gemm_both(mat, x_dev, q=False, apply_escapes=False):
    """fp32 and BF16 outputs of one GEMM (exact or Q pass) as NumPy arrays."""
    if q:
        yf = w12.gemm_q8(mat, x_dev, torch.float32, apply_escapes)
        yb = w12.gemm_q8(mat, x_dev, torch.bfloat16, apply_escapes)
    else:
        yf = w12.gemm(mat, x_dev, torch.float32)
        yb = w12.gemm(mat, x_dev, torch.bfloat16)
    torch.cuda.synchronize()
    return yf.cpu().numpy(), host16(yb)
