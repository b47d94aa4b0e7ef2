"""w12_gemm_noalloc (no workspace argument, static per-device scratch)
against w12_gemm through the C ABI: the same plan and kernels, so the same
bits; both within the tolerance of the fp64 oracle (SpecPilot section 4.1,
Figure 5b: the exact W12 GEMM)."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from gpu_util import check_f32, dev16, log, o, w12

pytestmark = pytest.mark.gpu


def _c_noalloc(mat, x, y):
    d = mat.desc()
    ydt = w12.F32 if y.dtype == torch.float32 else w12.BF16
    return w12.lib().w12_gemm_noalloc(ctypes.byref(d), ctypes.c_void_p(x.data_ptr()), x.shape[0], x.stride(0),
                                      ctypes.c_void_p(y.data_ptr()), y.stride(0), ydt, None)


def _c_gemm(mat, x, y):
    d = mat.desc()
    ydt = w12.F32 if y.dtype == torch.float32 else w12.BF16
    ws = w12.new_workspace(w12.OP_GEMM, mat.n, mat.k, x.shape[0])
    return w12.lib().w12_gemm(ctypes.byref(d), ctypes.c_void_p(x.data_ptr()), x.shape[0], x.stride(0),
                              ctypes.c_void_p(y.data_ptr()), y.stride(0), ydt, ctypes.c_void_p(ws.data_ptr()),
                              ws.numel(), None)


def _case(w, m, seed, out_dtype, what):
    log(f"[noalloc] {what} {w.shape} M={m} {out_dtype}")
    x = synth.make_activations(m, w.shape[1], seed=seed)
    mat = w12.encode(dev16(w))
    xd = dev16(x)
    y_ref = torch.full((m, w.shape[0]), 3.0, dtype=out_dtype, device="cuda")
    y_new = torch.full((m, w.shape[0]), -5.0, dtype=out_dtype, device="cuda")
    assert _c_gemm(mat, xd, y_ref) == w12.OK
    assert _c_noalloc(mat, xd, y_new) == w12.OK
    torch.cuda.synchronize()
    assert torch.equal(y_new.view(torch.int16) if out_dtype == torch.bfloat16 else y_new,
                       y_ref.view(torch.int16) if out_dtype == torch.bfloat16 else y_ref), what
    if out_dtype == torch.float32:
        check_f32(y_new.cpu().numpy(), o.gemm_ref(x, w), what)
    return w12.plan_info(mat, w12.OP_GEMM, m)["kernel"]


# Pairs of calls in a row, the second on a smaller input: the stream kernel
# (split tiles: counters and partial slots), the helper-wave MFMA kernel and
# the lane-per-row GEMV.
PAIRS = [
    ("stream", (1, 0, 1024, 5120), 32, (0, 0, 256, 1024), 8),
    ("helper", (1, 2, 1024, 17408), 48, (0, 0, 512, 1024), 17),
    ("gemv", (1, 1, 2048, 5120), 2, (0, 0, 256, 1024), 1),
]


@pytest.mark.parametrize("name,big,m1,small,m2", PAIRS, ids=[p[0] for p in PAIRS])
def test_noalloc_matches_gemm_on_two_calls(name, big, m1, small, m2):
    wl, idx, rows, cols = big
    w1 = synth.workload_matrix(wl, idx, rows=slice(0, rows))[:, :cols]
    wl, idx, rows, cols = small
    w2 = synth.workload_matrix(wl, idx, rows=slice(0, max(rows, 256)))[:rows, :cols]
    k1 = _case(w1, m1, 11, torch.float32, f"{name} first")
    k2 = _case(w2, m2, 12, torch.bfloat16, f"{name} second (smaller)")
    assert k1 in (w12.KERNEL_GEMV, w12.KERNEL_MFMA_HELPER, w12.KERNEL_MFMA_STREAM) and k2 > 0


def test_noalloc_largest_workload_shape():
    """The 5120 x 17408 down projection at M = 64 (the largest workspace the
    workload shapes need) fits the scratch; a small call follows it."""
    w = synth.workload_matrix(1, 2, rows=slice(0, 5120))
    assert w12.workspace_bytes(w12.OP_GEMM, 5120, 17408, 64) <= w12.NOALLOC_SCRATCH_BYTES
    _case(w, 64, 13, torch.float32, "down projection")
    _case(w[:256, :1024], 3, 14, torch.float32, "down projection slice, smaller")
